"""Precision of the decode kernels' fixed-point arithmetic on key and query
distributions far from the seeded workloads' (GPU against the fp64 oracle).

The split kernel scores quantized positions with the compensated query held
as 16-bit fixed point against exact code products, and weights a sub-chunk's
values with 16-bit fixed-point softmax weights; the chunk kernel uses 24- and
15-bit.  The error of a score grows with the key's norm times the query's
largest element, so these cases scale the keys (all channels, only the
outlier channels, or a shared offset per channel) and the queries, and each
attention output must stay within max_i |o_i - r_i| <= 2e-3 max_i |r_i|.
The parity summary prints the margin of every case.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_wushkv_amd import synth
from decode_attention_wushkv_amd.device_cache import DeviceCache

from gpu_checks import check_attention, check_codes, check_windows
from cachepack import read_unit

pytestmark = pytest.mark.gpu

SHAPES = ("keys_x30", "spikes_x100", "offset_20", "spikes_x30_queries_x4")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_wushkv_amd import build
    if build.is_stale():
        build.build()
    torch.cuda.set_device(0)


def _keys(w, shape, L, rng):
    """Keys [L, n_kv, d] (bf16) of the workload's distribution, reshaped."""
    sk, sv = synth.channel_scales(w, 0)
    k, v = synth.keys_values(w, 0, 0, 0, L, scales=(sk, sv))
    k = k.float()
    if shape == "keys_x30":
        k *= 30.0
    elif shape.startswith("spikes"):
        f = 10.0 if "x100" in shape else 3.0   # the 4 outlier channels are x10 already
        for h in range(w.n_kv):
            top = np.argsort(sk[h])[-4:]
            k[:, h, top] *= f
    elif shape == "offset_20":
        k += 20.0 * torch.from_numpy(np.sign(rng.standard_normal((w.n_kv, 128)))).float()[None]
    return k.to(w.torch_io).contiguous(), v


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("shape", SHAPES)
def test_decode_step_precision_stress(shape, G, bits):
    """Prefill 4000 positions, then two fused decode steps; every output
    against the oracle's attention over its own cache (section 4.4 order)."""
    n_kv, L0, n_steps = 2, 4000, 2
    w = synth.Workload(13, "stress", 1, n_kv * G, n_kv, 1, L0 + n_steps, (bits,), 4, 128, 1,
                       0.01, 0.99, "bf16")
    rng = np.random.default_rng(100 * SHAPES.index(shape) + 10 * G + bits)
    k, v = _keys(w, shape, L0 + n_steps, rng)
    qscale = 4.0 if "queries_x4" in shape else 1.0
    print(f"[stress] {shape} G={G} {bits}-bit", flush=True)
    T, Tq = synth.transforms(w, 0)
    tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
    dc = DeviceCache(n_layers=1, n_q_heads=w.n_q, n_kv_heads=n_kv, bits=bits, sink=4, recent=128,
                     max_batch=1, ctx_cap=L0 + n_steps, io_dtype=torch.bfloat16, device="cuda")
    dc.append(0, [0], [L0], k[:L0].cuda(), v[:L0].cuda(), tk)
    for st in range(n_steps):
        p = L0 + st
        q = (synth.queries(w, 0, st, 1).float() * qscale).to(torch.bfloat16)
        out = dc.decode_step(0, [0], k[p:p + 1].cuda().contiguous(), v[p:p + 1].cuda().contiguous(),
                             tk, q.cuda(), tq).cpu().numpy()
        Ks, Vs = [], []
        for h in range(n_kv):
            unit = oracle.cache_unit(k[:p + 1, h].double().numpy(), v[:p + 1, h].double().numpy(),
                                     T[h].astype(np.float64), S=4, R=129, F=1, bits=bits,
                                     p_lo=0.01, p_hi=0.99)
            Kh, Vh = oracle.readback(unit)
            Ks.append(Kh)
            Vs.append(Vh)
        qc = np.concatenate([oracle.compensate(T[h].astype(np.float64),
                                               q[0, h * G:(h + 1) * G].double().numpy())
                             for h in range(n_kv)])
        check_attention(out[0], oracle.attention(qc, np.stack(Ks), np.stack(Vs)))
    torch.cuda.synchronize()
    for h in range(n_kv):
        orc = oracle.cache_unit(k[:, h].double().numpy(), v[:, h].double().numpy(),
                                T[h].astype(np.float64), S=4, R=128, F=1, bits=bits,
                                p_lo=0.01, p_hi=0.99)
        gpu = read_unit(dc, 0, 0, h, L0 + n_steps)
        check_windows(gpu, orc)
        check_codes(gpu, orc, bits)
    dc.close()
