"""GPU parity of the quantizer's defined edge behaviour, through every writer
of codes: the rank-sort append (fp32 inputs), the matrix-core prefill
(bfloat16 inputs), the flush of the fused decode step and the flush of the
chunked step.

The quantizer is percentile clipping with asymmetric affine scaling (paper
page, section 5.3) or the RMS-normalized symmetric grid (appendix B.3), with
2^b equally spaced levels.  The readings fix three edge behaviours, which the
continuous seeded data never reach:
  * a value exactly on a level boundary z16 + (c + 1/2) s16 rounds to the
    even level;
  * a group whose binary16 scale is zero (constant groups, and ranges below
    half the smallest binary16 step) gets all-zero codes;
  * a scale or zero beyond the binary16 range saturates at +-65504.
The key transform is the identity, so the quantizer sees the hand-built rows
exactly, and every code, scale and zero must equal the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_wushkv_amd.device_cache import DeviceCache

from cachepack import read_unit
from gpu_checks import check_attention, check_codes, check_windows

pytestmark = pytest.mark.gpu

D = 128
N_KV = 2
S = 4
RMS_ALPHA = {2: 1.5, 3: 3.5, 4: 7.5}  # scale 2 f on rows of RMS 2 f: every even multiple of f a boundary


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_wushkv_amd import build
    if build.is_stale():
        build.build()
    torch.cuda.set_device(0)


# ------------------------------------------------------------------ rows

def _with_ends(rng, lo, hi, body, below, above):
    """A group whose two smallest values are lo (one smaller value below them)
    and whose two largest below the maximum are hi, so that the 1st / 99th
    linear-interpolation percentiles of 128 values are exactly lo and hi."""
    row = np.concatenate([[below, lo, lo, hi, hi, above], body])
    assert row.size == D
    return row[rng.permutation(D)]


def tie_row(rng, bits):
    """Percentile clip ends lo = z, hi = z + (2^b - 1) s with s a power of two:
    the body takes level values and the boundaries between them."""
    n = (1 << bits) - 1
    s = 2.0 ** int(rng.integers(-3, 3))
    z = s / 2 * int(rng.integers(-2 * n, 2 * n + 1))
    pts = np.array([z + (c + 0.5) * s for c in range(n)] + [z + c * s for c in range(n + 1)])
    body = pts[rng.integers(0, pts.size, D - 6)]
    return _with_ends(rng, z, z + n * s, body, z - s * int(rng.integers(0, 4)),
                      z + n * s + s * int(rng.integers(0, 4)))


def rms_tie_row(rng, bits):
    """RMS exactly 2 f (magnitudes 6, 4, 3, 2, 0 times f in fixed counts, random
    signs); with alpha = RMS_ALPHA[bits] the scale is 2 f and the even
    multiples of f are level boundaries."""
    f = 2.0 ** int(rng.integers(-3, 3))
    mags = np.concatenate([np.full(4, 6.0), np.full(8, 4.0), np.full(16, 3.0), np.full(24, 2.0),
                           np.zeros(76)])
    signs = np.where(rng.random(D) < 0.5, -1.0, 1.0)
    return (mags * signs * f)[rng.permutation(D)]


def const_row(rng, bits):
    """All 128 values equal: zero range, binary16 scale 0, all codes 0."""
    c = [0.0, 1.5, -3.25, 1024.0, 2.0 ** -20, -96.0][int(rng.integers(0, 6))]
    return np.full(D, c)


def tiny_row(rng, bits):
    """Ranges at the bottom of binary16: one bfloat16 step at 2^-20 (the scale
    rounds to 0) or 2^b - 1 steps of 2^-24 at 2^-17 (the scale is the smallest
    subnormal)."""
    n = (1 << bits) - 1
    if rng.random() < 0.5:
        a, u, k = 2.0 ** -20, 2.0 ** -27, 1
    else:
        a, u, k = 2.0 ** -17, 2.0 ** -24, n
    body = a + u * rng.integers(0, k + 1, D - 6)
    return _with_ends(rng, a, a + k * u, body, a, a + k * u)


def sat_row(rng, bits):
    """Clip ends beyond the binary16 range: scale and zero saturate at +-65504
    (either or both)."""
    n = (1 << bits) - 1
    kind = int(rng.integers(0, 4))
    if kind == 0:
        lo, hi = -98304.0, 98304.0           # both saturate
    elif kind == 1:
        lo, hi = 69632.0, 69632.0 + n * 512  # zero saturates high
    elif kind == 2:
        lo, hi = -69632.0 - n * 512, -69632.0  # zero saturates low
    else:
        lo, hi = -1024.0, 196608.0           # scale saturates
    body = oracle.bf16(rng.uniform(lo, hi, D - 6))
    return _with_ends(rng, lo, hi, body, lo - 512 * int(rng.integers(0, 3)), hi)


def normal_row(rng, bits):
    return oracle.bf16(rng.standard_normal(D) * rng.lognormal(0, 1, D))


def make_rows(rng, L, bits, family, rms):
    """Rows [L, N_KV, D] of one edge family (mixed with a few Gaussian rows)."""
    gens = {"edge": [rms_tie_row if rms else tie_row, const_row, tiny_row],
            "sat": [sat_row]}[family]
    out = np.empty((L, N_KV, D))
    for p in range(L):
        for h in range(N_KV):
            if rng.random() < 0.1:
                out[p, h] = normal_row(rng, bits)
            else:
                g = gens[int(rng.integers(0, len(gens)))]
                out[p, h] = g(rng, bits)
    assert np.array_equal(oracle.bf16(out), out), "rows must be exact bfloat16 values"
    return out


# ------------------------------------------------------------------ writers

def _cache(bits, G, io, R, F, rms, ctx):
    kw = dict(codec=1, clip_alpha=RMS_ALPHA[bits]) if rms else {}
    return DeviceCache(n_layers=1, n_q_heads=N_KV * G, n_kv_heads=N_KV, bits=bits, sink=S,
                       recent=R, flush=F, max_batch=1, ctx_cap=ctx, io_dtype=io, device="cuda",
                       **kw)


def _t(x, io):
    return torch.from_numpy(x.astype(np.float32)).to(io).contiguous().cuda()


WRITERS = {
    # name: (io dtype, G, recent, flush)
    "rank_sort": (torch.float32, 4, 8, 1),
    "prefill": (torch.bfloat16, 4, 8, 1),
    "step_g1": (torch.bfloat16, 1, 8, 1),
    "step_g4_newest": (torch.bfloat16, 4, 0, 1),
    "chunk_g1": (torch.bfloat16, 1, 4, 2),
    "chunk_g8": (torch.bfloat16, 8, 4, 2),
}


def _run(writer, bits, family, rms, L=320, seed=0):
    io, G, R, F = WRITERS[writer]
    rng = np.random.default_rng(1000 * bits + 10 * len(writer) + seed + (500 if rms else 0)
                                + (7 if family == "sat" else 0))
    K = make_rows(rng, L, bits, family, rms)
    V = make_rows(rng, L, bits, family, rms)
    dc = _cache(bits, G, io, R, F, rms, L)
    eye = torch.eye(D, dtype=torch.float32).repeat(N_KV, 1, 1).contiguous().cuda()
    print(f"[edges] {writer} {bits}-bit {family} {'rms' if rms else 'percentile'} L={L}",
          flush=True)
    if writer == "rank_sort":
        plan = [150, 7, 1, 1, 60, 16, 17, L - 252]
    elif writer == "prefill":
        plan = [17, 250, L - 267]
    else:
        plan = [S]
    pos = 0
    for n in plan:
        dc.append(0, [0], [n], _t(K[pos:pos + n], io), _t(V[pos:pos + n], io), eye)
        pos += n
    qrng = np.random.default_rng(77)
    while pos < L:
        if writer.startswith("step"):
            q = _t(qrng.standard_normal((1, N_KV * G, D)), io)
            dc.decode_step(0, [0], _t(K[pos:pos + 1], io), _t(V[pos:pos + 1], io), eye, q, eye)
            pos += 1
        else:
            n = min(L - pos, [16, 16, 5, 16, 1, 9][pos % 6])
            q = _t(qrng.standard_normal((n, N_KV * G, D)), io)
            dc.chunk_step(0, [0], [n], _t(K[pos:pos + n], io), _t(V[pos:pos + n], io), eye, q, eye)
            pos += n
    torch.cuda.synchronize()
    assert dc.get_len(0, 0)[0] == L
    units = {}
    for h in range(N_KV):
        orc = oracle.cache_unit(K[:, h], V[:, h], np.eye(D), S=S, R=R, F=F, bits=bits,
                                p_lo=0.01, p_hi=0.99, alpha=RMS_ALPHA[bits] if rms else None)
        gpu = read_unit(dc, 0, 0, h, L)
        check_windows(gpu, orc)
        st = check_codes(gpu, orc, bits, strict=True)
        assert st["positions"] > 0
        units[h] = orc
    if family != "sat":
        # attention over the cache just checked (values within the float range)
        qt = _t(qrng.standard_normal((1, N_KV * G, D)), io)
        out = dc.decode_attn(0, [0], qt, eye).cpu().numpy()
        qb = qt.float().cpu().numpy().astype(np.float64)   # the query values the GPU read
        Kr = np.stack([oracle.readback(units[h])[0] for h in range(N_KV)])
        Vr = np.stack([oracle.readback(units[h])[1] for h in range(N_KV)])
        check_attention(out[0], oracle.attention(qb[0], Kr, Vr))
    dc.close()


@pytest.mark.parametrize("rms", [False, True], ids=["percentile", "rms"])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("writer", list(WRITERS))
def test_quantizer_ties_constant_tiny(writer, bits, rms):
    """Exact level-boundary ties, constant groups and binary16-underflowing
    scales: codes, scale and zero identical to the oracle's."""
    _run(writer, bits, "edge", rms)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("writer", list(WRITERS))
def test_quantizer_fp16_saturation(writer, bits):
    """Clip ends beyond +-65504: the binary16 scale and zero saturate, and the
    codes follow from the saturated values, identically to the oracle."""
    _run(writer, bits, "sat", False)
