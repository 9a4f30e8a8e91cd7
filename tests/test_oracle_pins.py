"""Pins of the CPU reference against facts fixed outside itself: library
conversions, closed forms, brute force on tiny inputs, identities the method
states, and worked values derived by hand from the method's definitions.

Sources: WUSH-KV paper page, sections 4.1, 4.2, 4.4, 5.3, appendices B.1, B.3,
D.1; the blog page's cache-footprint arithmetic.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from decode_attention_wushkv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- formats

def test_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000),
        rng.standard_normal(2000).astype(np.float32),
        (np.float32(1.0) + np.arange(512, dtype=np.float32) * np.float32(2.0 ** -9)),  # ties
        np.array([1e-39, -3e-41, 1.4e-45, 3.38e38, -3.38e38], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = oracle.bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_ties_and_overflow_by_hand():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even -> 1 + 2^-6.
    got = oracle.bf16([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2.0 ** 128, 1e39])
    assert list(got[:3]) == [1.0, 1 + 2 ** -6, -1.0]
    assert np.isinf(got[3]) and np.isinf(got[4])


def test_fp16_matches_numpy_double_to_half():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 4.7, 20000),
        np.arange(-2048, 2049) * 2.0 ** -11 + 1.0,          # exact ties near 1
        np.array([2 ** -24, 2 ** -25, 3 * 2 ** -26, 6.1e-5, 65504.0, -65504.0]),
    ])
    x = x[np.abs(x) <= 65504.0]
    ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.fp16(x), ref)


def test_fp16_saturates():
    got = oracle.fp16([65520.0, 1e6, -7e4])
    assert list(got) == [65504.0, 65504.0, -65504.0]


# ---------------------------------------------------------------- transform

def _hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(n)


def test_transform_identity_and_hadamard():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((50, 128)) * rng.lognormal(0, 1, 128)
    y, _ = oracle.transform(np.eye(128), k)
    assert np.array_equal(y, k)
    H = _hadamard(128)                   # normalized Hadamard: H H = I
    y, _ = oracle.transform(H, k)
    back, _ = oracle.transform(H, y)
    assert np.allclose(back, k, rtol=0, atol=1e-12 * np.abs(k).max())
    # against the library matmul
    assert np.allclose(y, k @ H.T, rtol=1e-13, atol=1e-13)


def test_score_invariance_under_compensation():
    """q.k = (T^{-T} q).(T k): section 4.2 / appendix B.1, fp64 to 1e-9."""
    w = synth.WORKLOADS[1]
    T, Tq = synth.transforms(w, layer=0)
    rng = np.random.default_rng(4)
    for h in range(3):
        k = rng.standard_normal((40, 128)) * 3
        q = rng.standard_normal((5, 128))
        kt, _ = oracle.transform(T[h].astype(np.float64), k)
        qc = oracle.compensate(T[h].astype(np.float64), q)
        ref = q @ k.T
        got = qc @ kt.T
        assert np.max(np.abs(got - ref)) <= 1e-9 * np.max(np.abs(ref))
        # the closed-form inverse transpose of Q diag(delta) is Q diag(1/delta)
        qc2 = q @ Tq[h].astype(np.float64).T
        assert np.max(np.abs(qc - qc2)) <= 1e-5 * np.max(np.abs(qc))  # fp32 storage of Tq


def test_ambiguity_band_flags_midpoints_only():
    # A value sitting exactly on a bf16 midpoint is ambiguous; one far away is not.
    y = np.array([1 + 2 ** -8, 1 + 2 ** -9, 3.0])
    absy = np.array([1.0, 1.0, 3.0])
    assert list(oracle.bf16_ambiguous(y, absy)) == [True, False, False]


# ---------------------------------------------------------------- percentile

def _order_stat_bruteforce(x, k):
    """k-th smallest (0-based) by rank counting, no sort."""
    for v in x:
        less = sum(1 for t in x if t < v)
        leq = sum(1 for t in x if t <= v)
        if less <= k < leq:
            return v
    raise AssertionError


@pytest.mark.parametrize("n", [1, 2, 3, 5, 6])
def test_percentile_bruteforce_small(n):
    ps = [0.0, 0.01, 0.25, 0.5, 0.73, 0.99, 1.0]
    for vals in itertools.product([0.0, 1.0, 2.5], repeat=n):
        x = np.array(vals)
        for p in ps:
            h = p * (n - 1)
            j = int(np.floor(h))
            f = h - j
            lo = _order_stat_bruteforce(vals, j)
            ref = lo if j >= n - 1 else lo + f * (_order_stat_bruteforce(vals, j + 1) - lo)
            got = oracle.percentile(x, p)
            assert abs(got - ref) <= 1e-12, (vals, p, got, ref)
            assert abs(got - np.percentile(x, 100 * p, method="linear")) <= 1e-12


def test_percentile_matches_numpy_groups():
    rng = np.random.default_rng(5)
    for _ in range(200):
        x = rng.standard_normal(128) * rng.lognormal(0, 1)
        for p in (0.01, 0.99, 0.05, 0.5):
            ref = np.percentile(x, 100 * p, method="linear")
            assert abs(oracle.percentile(x, p) - ref) <= 4e-16 * max(1.0, np.abs(x).max())


# ---------------------------------------------------------------- quantizer

def test_quantizer_ramp_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "quantizer_ramp.json")))
    x = np.arange(128, dtype=np.float64)
    q = oracle.quantize(x[None], 2, 0.01, 0.99)
    assert q["s16"][0] == g["s16"] and q["z16"][0] == g["z16"]
    expect = np.empty(128, dtype=np.uint8)
    for a, b, c in g["code_runs"]:
        expect[a:b + 1] = c
    assert np.array_equal(q["codes"][0], expect)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantizer_idempotent_on_grid(bits):
    """Values already on the grid z16 + s16 c, with >= 3 copies of each extreme
    code (so both 1% / 99% percentile ends land on grid points), come back with
    the same codes and x_hat == x exactly."""
    rng = np.random.default_rng(6 + bits)
    top = (1 << bits) - 1
    for _ in range(100):
        s16 = float(np.float16(rng.uniform(0.01, 4.0)))
        z16 = float(np.float16(rng.uniform(-8.0, 1.0)))
        c = rng.integers(0, top + 1, size=128)
        c[:3] = 0
        c[3:6] = top
        rng.shuffle(c)
        x = z16 + s16 * c
        q = oracle.quantize(x[None], bits, 0.01, 0.99)
        assert q["s16"][0] == s16 and q["z16"][0] == z16
        assert np.array_equal(q["codes"][0], c.astype(np.uint8))
        assert np.array_equal(oracle.dequantize(q["codes"], q["s16"], q["z16"])[0], x)


@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_properties(bits):
    """Monotone in x, codes in range, |x - x_hat| <= s16/2 inside the clip range,
    and every reconstruction is one of 2^b equally spaced levels (B.3)."""
    rng = np.random.default_rng(10 + bits)
    top = (1 << bits) - 1
    x = oracle.bf16(rng.standard_normal((300, 128)) * rng.lognormal(0, 1, (300, 1)))
    q = oracle.quantize(x, bits, 0.01, 0.99)
    xh = oracle.dequantize(q["codes"], q["s16"], q["z16"])
    for g in range(x.shape[0]):
        order = np.argsort(x[g], kind="stable")
        assert np.all(np.diff(q["codes"][g][order].astype(int)) >= 0)
        assert q["codes"][g].max() <= top
        s, z = q["s16"][g], q["z16"][g]
        inside = (x[g] >= z) & (x[g] <= z + top * s)
        assert np.all(np.abs(x[g] - xh[g])[inside] <= s / 2 * (1 + 1e-12))
        levels = (xh[g] - z) / s
        assert np.allclose(levels, np.round(levels), atol=1e-9)


def test_quantizer_degenerate_constant_group():
    q = oracle.quantize(np.full((1, 128), 1.5), 2, 0.01, 0.99)
    assert q["s16"][0] == 0.0 and q["z16"][0] == 1.5
    assert not q["codes"].any()
    assert np.all(oracle.dequantize(q["codes"], q["s16"], q["z16"]) == 1.5)


def test_quantizer_plants_caught():
    """A planted mistake in the clip (percentile 0.02 instead of 0.01) changes
    the zero point on ordinary data, so the ramp/idempotence pins above would
    fail for such a mistake."""
    x = np.arange(128, dtype=np.float64)
    assert oracle.quantize(x[None], 2, 0.02, 0.99)["z16"][0] != 1.26953125


# ---------------------------------------------------------------- regions

def test_squant_by_hand():
    assert oracle.squant(10, 4, 32, 1) == 4
    assert oracle.squant(36, 4, 32, 1) == 4
    assert oracle.squant(37, 4, 32, 1) == 5
    assert oracle.squant(1024, 4, 32, 1) == 992
    assert oracle.squant(300, 16, 128, 16) == 160    # 156 outside -> 9 * 16
    assert oracle.squant(2, 4, 32, 1) == 4           # L < S: nothing quantized


def test_squant_window_invariant():
    """Section 4.4: once the windows no longer overlap, S + R entries stay in full
    precision plus fewer than S_flush temporary ones."""
    for S, R, F in [(4, 32, 1), (16, 128, 16), (0, 8, 3), (4, 0, 1)]:
        prev = S
        for L in range(0, 600):
            sq = oracle.squant(L, S, R, F)
            assert sq >= S and sq >= prev
            prev = sq
            if L >= S + R:
                assert 0 <= L - sq - R < F
                assert (sq - S) % F == 0
            else:
                assert sq == S


# ---------------------------------------------------------------- attention

def _sdpa(q, k, v):
    """torch SDPA in fp64 with GQA head repetition: q [n_q, d], k, v [n_kv, L, d]."""
    n_q = q.shape[0]
    G = n_q // k.shape[0]
    kk = torch.from_numpy(np.repeat(k, G, axis=0))
    vv = torch.from_numpy(np.repeat(v, G, axis=0))
    qq = torch.from_numpy(q)[:, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0, :].numpy()


def test_attention_matches_sdpa_gqa():
    rng = np.random.default_rng(20)
    n_kv, G, L = 2, 4, 300
    q = rng.standard_normal((n_kv * G, 128))
    k = rng.standard_normal((n_kv, L, 128))
    v = rng.standard_normal((n_kv, L, 128))
    assert np.allclose(oracle.attention(q, k, v), _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_unquantized_pipeline_equals_plain_attention():
    """With fp64 windows and nothing quantized, attention of the compensated query
    over transformed keys equals plain attention over raw keys (transform
    invariance, section 4.2), to 1e-12."""
    w = synth.WORKLOADS[0]
    T, _ = synth.transforms(w, 0)
    T = T[0].astype(np.float64)
    rng = np.random.default_rng(21)
    L = 200
    k = rng.standard_normal((L, 128)) * 2
    v = rng.standard_normal((L, 128))
    q = rng.standard_normal((4, 128))
    kt, _ = oracle.transform(T, k)
    qc = oracle.compensate(T, q)
    got = oracle.attention(qc, kt[None], v[None])
    ref = _sdpa(q, k[None], v[None])
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())


def test_attention_linear_in_v_and_wo_fold():
    """V fold (section 4.2 / 4.5): the cache and output live in the T_V basis;
    W_o o = (W_o T_V^{-1})(T_V o), and attention output is T_V times the output
    over untransformed V.  fp64 to 1e-9."""
    rng = np.random.default_rng(22)
    L, d = 150, 128
    qc = rng.standard_normal((4, d))
    k = rng.standard_normal((1, L, d))
    v = rng.standard_normal((1, L, d))
    Tv = rng.standard_normal((d, d)) + 3 * np.eye(d)
    Wo = rng.standard_normal((64, d))
    o = oracle.attention(qc, k, v)
    o_t = oracle.attention(qc, k, (v[0] @ Tv.T)[None])
    assert np.max(np.abs(o_t - o @ Tv.T)) <= 1e-9 * np.abs(o_t).max()
    folded = Wo @ np.linalg.inv(Tv)
    assert np.max(np.abs(o_t @ folded.T - o @ Wo.T)) <= 1e-9 * np.abs(o @ Wo.T).max()


def test_split_merge_identity():
    """Log-sum-exp merge of attention over random partitions of the positions
    equals the one-shot softmax (the identity split-K decoding relies on)."""
    rng = np.random.default_rng(23)
    L, d = 500, 128
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, L, d)) * 2
    v = rng.standard_normal((1, L, d))
    ref = oracle.attention(q, k, v)[0]
    cuts = np.sort(rng.choice(np.arange(1, L), size=7, replace=False))
    ms, ls, os_ = [], [], []
    for a, b in zip(np.r_[0, cuts], np.r_[cuts, L]):
        e = (k[0, a:b] @ q[0]) / np.sqrt(d)
        m = e.max()
        p = np.exp(e - m)
        ms.append(m)
        ls.append(p.sum())
        os_.append(p @ v[0, a:b])
    M = max(ms)
    lsum = sum(l * np.exp(m - M) for m, l in zip(ms, ls))
    o = sum(oo * np.exp(m - M) for m, oo in zip(ms, os_)) / lsum
    assert np.max(np.abs(o - ref)) <= 1e-12 * np.abs(ref).max()


# ---------------------------------------------------------------- cache unit

def test_cache_unit_regions_and_inputs():
    w = synth.WORKLOADS[0]
    T, _ = synth.transforms(w, 0)
    k, v = synth.keys_values(w, 0, 0, 0, 300)
    unit = oracle.cache_unit(k[:, 0].double().numpy(), v[:, 0].double().numpy(),
                             T[0].astype(np.float64), S=4, R=32, F=1, bits=2,
                             p_lo=0.01, p_hi=0.99)
    assert unit["squant"] == 300 - 32
    assert np.array_equal(unit["qpos"], np.arange(4, 268))
    # window entries are the bf16 roundings of T k and v
    # (library matmul; a transposed T would fail this since T is not symmetric)
    kt = k[:, 0].double().numpy() @ T[0].astype(np.float64).T
    ok = ~unit["k_ambiguous"]
    assert ok.mean() > 0.999
    assert np.array_equal(unit["k_bf16"][ok], oracle.bf16(kt)[ok])
    assert np.array_equal(unit["v_bf16"], torch.from_numpy(v[:, 0].float().numpy())
                          .to(torch.bfloat16).double().numpy())
    # window positions keep no codes
    assert (unit["kcodes"][:4] == 255).all() and (unit["kcodes"][268:] == 255).all()
    K, V = oracle.readback(unit)
    assert np.array_equal(K[:4], unit["k_bf16"][:4]) and np.array_equal(V[268:], unit["v_bf16"][268:])
    # a quantized entry is within half a step of its bf16 value when inside the clip range
    x = unit["v_bf16"][100]
    s, z = unit["vs16"][100], unit["vz16"][100]
    inside = (x >= z) & (x <= z + 3 * s)
    assert np.all(np.abs(V[100] - x)[inside] <= s / 2 + 1e-12)


def test_cache_unit_nothing_quantized_equals_sdpa_on_bf16():
    w = synth.WORKLOADS[0]
    T, _ = synth.transforms(w, 0)
    T = T[0].astype(np.float64)
    k, v = synth.keys_values(w, 0, 0, 0, 64)
    q = synth.queries(w, 0, 0, 1)[0].double().numpy()
    unit = oracle.cache_unit(k[:, 0].double().numpy(), v[:, 0].double().numpy(), T,
                             S=4, R=64, F=1, bits=2, p_lo=0.01, p_hi=0.99)
    assert unit["squant"] == 4 and unit["qpos"].size == 0
    K, V = oracle.readback(unit)
    qc = oracle.compensate(T, q)
    got = oracle.attention(qc, K[None], V[None])
    ref = _sdpa(qc, K[None], V[None])
    assert np.max(np.abs(got - ref)) <= 1e-12


# ------------------------------------------------------------ RMS (QuEST-style) codec

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("alpha", [0.7, 1.5, 2.5])
def test_gaussian_grid_mse_matches_numeric_integration(bits, alpha):
    """Closed-form E[(z - Q_alpha(z))^2] against direct quadrature of the
    integrand over each decision interval (appendix B.3's grid of 2^b levels
    from -alpha to alpha)."""
    from scipy import integrate
    from scipy.stats import norm
    n = 1 << bits
    levels = np.linspace(-alpha, alpha, n)
    edges = np.concatenate([[-np.inf], (levels[:-1] + levels[1:]) / 2, [np.inf]])
    total = 0.0
    for k, y in enumerate(levels):
        val, _ = integrate.quad(lambda z: (z - y) ** 2 * norm.pdf(z), edges[k], edges[k + 1],
                                epsabs=1e-14, epsrel=1e-13, limit=200)
        total += val
    assert abs(oracle.gaussian_grid_mse(alpha, bits) - total) <= 1e-10


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_gaussian_alpha_optimal_and_monte_carlo(bits):
    a = oracle.quest_alpha(bits)
    f = oracle.gaussian_grid_mse(a, bits)
    for d in (1e-3, -1e-3, 1e-2, -1e-2):
        assert oracle.gaussian_grid_mse(a + d, bits) > f
    # the error of that grid on Gaussian samples
    z = np.random.default_rng(7 + bits).standard_normal(1_000_000)
    n = 1 << bits
    delta = 2 * a / (n - 1)
    c = np.clip(np.rint((z + a) / delta), 0, n - 1)
    mse = np.mean((z - (-a + delta * c)) ** 2)
    assert abs(mse - f) <= 0.01 * f
    # more levels, wider optimal endpoint and smaller error
    if bits > 2:
        assert a > oracle.quest_alpha(bits - 1)
        assert f < oracle.gaussian_grid_mse(oracle.quest_alpha(bits - 1), bits - 1)


@pytest.mark.parametrize("bits", [2, 4])
def test_quantize_rms_brute_force(bits):
    """Clip ends -alpha rms, +alpha rms; binary16 scale and zero; each code is
    the nearest level z16 + c s16 (ties to the even level), by exhaustive
    search over the levels."""
    rng = np.random.default_rng(40 + bits)
    x = rng.standard_normal((64, 128)) * rng.lognormal(0, 1, (1, 128))
    x = oracle.bf16(x)
    alpha = 1.7
    r = oracle.quantize_rms(x, bits, alpha)
    n = 1 << bits
    for g in range(x.shape[0]):
        rms = np.sqrt(np.sum(x[g] ** 2) / 128)
        lo, hi = -alpha * rms, alpha * rms
        s16 = oracle.fp16((hi - lo) / (n - 1))
        z16 = oracle.fp16(lo)
        assert r["s16"][g] == s16 and r["z16"][g] == z16
        levels = z16 + s16 * np.arange(n)
        for i in range(128):
            d = np.abs(x[g, i] - levels)
            best = np.flatnonzero(d == d.min())
            want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert r["codes"][g, i] == want


def test_quantize_rms_worked_examples():
    """Clip ends of the RMS codec pinned by hand-worked groups whose RMS is
    exactly 2 (tests/golden/quantizer_rms.json; appendix B.3's grid from
    -alpha to alpha scaled by the group's RMS).  A mean-centred deviation, a
    divisor of n - 1 or a missing square root changes the stored scale of
    group A; group C puts every even value on a level boundary (ties to the
    even level)."""
    import json
    spec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quantizer_rms.json")))
    rng = np.random.default_rng(12)
    for g in spec["groups"]:
        x = np.concatenate([np.full(n, v) for v, n in g["values"]])
        assert x.size == 128
        x = x[rng.permutation(128)]
        r = oracle.quantize_rms(x, g["bits"], g["alpha"])
        assert r["s16"] == g["s16"] and r["z16"] == g["z16"], g["name"]
        want = dict((float(v), c) for v, c in g["codes"])
        assert all(r["codes"][i] == want[float(x[i])] for i in range(128)), g["name"]
