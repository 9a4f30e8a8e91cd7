"""fp64 CPU reference ("the oracle") for the WUSH-KV transformed low-bit KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library and the GPU library never imports it.

The arithmetic lives in ``wko.c`` (scalar fp64 loops, built with
``-ffp-contract=off``); this module loads it with ctypes and composes the steps
for one (sequence, KV head) unit.  Library primitives used as steps: numpy's
linear solve for the query compensation ``T^{-T} q``.

Sources are the web pages on "WUSH-KV: KV Cache Quantization with
Data-Adaptive Transforms" (the paper's own text):
  * section 4.1 (GQA cache layout; query head (h, g) reads KV head h; keys are
    cached after RoPE),
  * section 4.2 (full d x d key transform after RoPE plus query compensation),
  * section 4.4 (sink / recent windows, S_flush batches, S_quant boundary),
  * section 5.3 (percentile-clipped asymmetric affine quantizer with adaptive
    zero point),
  * appendix B.1 (each column is one quantization group; B_T = T^{-T} H T^{-1},
    i.e. the compensation is T^{-T}),
  * appendix B.3 (2^b equally spaced levels, spacing range / (2^b - 1)),
  * appendix D.1 (softmax with the model's native scaling).

Parity pins live in ``tests/test_oracle_pins.py``; every function here has at
least one pin that does not re-type its own formula.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wko.c")
_LIB_PATH = os.path.join(_HERE, "libwko.so")
_lib = None

# Band for "the bfloat16 rounding of T k is not decided by fp64": any
# summation order of the same 128 fp64 products differs from the exact sum by
# at most n * 2^-53 * sum|T_ij k_j| = 2^-46 sum|.| for n = 128; use 2^-44.
AMBIGUITY_BAND_LOG2 = -44


def build(force: bool = True) -> str:
    """Compile wko.c into libwko.so next to it (gcc, fp64, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", _LIB_PATH, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    i64 = ctypes.c_int64
    lib.wko_bf16.restype = ctypes.c_double
    lib.wko_bf16.argtypes = [ctypes.c_double]
    lib.wko_fp16.restype = ctypes.c_double
    lib.wko_fp16.argtypes = [ctypes.c_double]
    lib.wko_bf16_array.argtypes = [dp, dp, i64]
    lib.wko_fp16_array.argtypes = [dp, dp, i64]
    lib.wko_transform.argtypes = [dp, dp, i64, ctypes.c_int, dp, dp]
    lib.wko_percentile.restype = ctypes.c_double
    lib.wko_percentile.argtypes = [dp, ctypes.c_int, ctypes.c_double, dp]
    lib.wko_quantize.restype = ctypes.c_int
    lib.wko_quantize.argtypes = [dp, i64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_double, ctypes.c_double, u8p, dp, dp, dp]
    lib.wko_quantize_rms.restype = ctypes.c_int
    lib.wko_quantize_rms.argtypes = [dp, i64, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                     u8p, dp, dp, dp]
    lib.wko_dequantize.argtypes = [u8p, dp, dp, i64, ctypes.c_int, dp]
    lib.wko_squant.restype = i64
    lib.wko_squant.argtypes = [i64, i64, i64, i64]
    lib.wko_attention.restype = ctypes.c_int
    lib.wko_attention.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, i64,
                                  ctypes.c_int, dp]
    _lib = lib
    return lib


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16(x) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even), returned as float64."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().wko_bf16_array(_dp(x), _dp(y), x.size)
    return y


def fp16(x) -> np.ndarray:
    """Round to IEEE binary16 (nearest, ties to even, saturating at +-65504)."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().wko_fp16_array(_dp(x), _dp(y), x.size)
    return y


# --------------------------------------------------------------------------
# Steps of the method
# --------------------------------------------------------------------------

def transform(T, keys):
    """k'_t = T k_t for every row of ``keys`` (section 4.2, appendix B.1).

    Returns (k', sum_j |T_ij k_j|), both float64 with the shape of ``keys``.
    """
    T = _f64(T)
    keys = _f64(keys)
    d = T.shape[0]
    assert T.shape == (d, d) and keys.shape[-1] == d
    flat = keys.reshape(-1, d)
    out = np.empty_like(flat)
    aout = np.empty_like(flat)
    _load().wko_transform(_dp(T), _dp(flat), flat.shape[0], d, _dp(out), _dp(aout))
    return out.reshape(keys.shape), aout.reshape(keys.shape)


def bf16_ambiguous(y, absy) -> np.ndarray:
    """True where the bfloat16 rounding of the exact T k is not decided by the
    fp64 value ``y`` within the error band 2^-44 sum|T_ij k_j|: both bfloat16
    neighbours are then correct results for any implementation."""
    y = _f64(y)
    band = np.ldexp(_f64(absy), AMBIGUITY_BAND_LOG2)
    return bf16(y - band) != bf16(y + band)


def percentile(x, p: float) -> float:
    """Linear-interpolation percentile of a 1-D sample (sort based)."""
    x = _f64(x).ravel()
    scratch = np.empty_like(x)
    return _load().wko_percentile(_dp(x), x.size, float(p), _dp(scratch))


def quantize(groups, bits: int, p_lo: float, p_hi: float):
    """Per-group percentile-clipped affine quantizer (section 5.3, B.1, B.3).

    ``groups``: [..., n]; each row is one group (one token of one KV head).
    Returns dict(codes uint8 [..., n], s16 [...], z16 [...], u [..., n]).
    """
    g = _f64(groups)
    n = g.shape[-1]
    flat = g.reshape(-1, n)
    ng = flat.shape[0]
    codes = np.empty((ng, n), dtype=np.uint8)
    s16 = np.empty(ng)
    z16 = np.empty(ng)
    u = np.empty((ng, n))
    rc = _load().wko_quantize(_dp(flat), ng, n, int(bits), float(p_lo), float(p_hi),
                              codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                              _dp(s16), _dp(z16), _dp(u))
    if rc != 0:
        raise ValueError("wko_quantize: bad arguments")
    lead = g.shape[:-1]
    return dict(codes=codes.reshape(g.shape), s16=s16.reshape(lead),
                z16=z16.reshape(lead), u=u.reshape(g.shape))


def quantize_rms(groups, bits: int, alpha: float):
    """Symmetric quantizer on the RMS-normalized group (appendix B.3's grid of
    2^b levels from -alpha to alpha, scaled by the group's RMS).  Same outputs
    as quantize()."""
    g = _f64(groups)
    n = g.shape[-1]
    flat = g.reshape(-1, n)
    ng = flat.shape[0]
    codes = np.empty((ng, n), dtype=np.uint8)
    s16 = np.empty(ng)
    z16 = np.empty(ng)
    u = np.empty((ng, n))
    rc = _load().wko_quantize_rms(_dp(flat), ng, n, int(bits), float(alpha),
                                  codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                  _dp(s16), _dp(z16), _dp(u))
    if rc != 0:
        raise ValueError("wko_quantize_rms: bad arguments")
    lead = g.shape[:-1]
    return dict(codes=codes.reshape(g.shape), s16=s16.reshape(lead),
                z16=z16.reshape(lead), u=u.reshape(g.shape))


def gaussian_grid_mse(alpha: float, bits: int) -> float:
    """E[(zeta - Q_alpha(zeta))^2] for zeta ~ N(0, 1), Q_alpha rounding to the
    nearest of 2^b equally spaced levels from -alpha to alpha (appendix B.3).
    Closed form per decision interval [a, b] with level y:
    (1 + y^2)(Phi(b) - Phi(a)) - (b phi(b) - a phi(a)) + 2 y (phi(b) - phi(a))."""
    from scipy.stats import norm
    nlev = 1 << bits
    delta = 2.0 * alpha / (nlev - 1)
    levels = -alpha + delta * np.arange(nlev)
    edges = np.concatenate([[-np.inf], (levels[:-1] + levels[1:]) / 2.0, [np.inf]])
    total = 0.0
    for k, y in enumerate(levels):
        a, b = edges[k], edges[k + 1]
        Pa, Pb = norm.cdf(a), norm.cdf(b)
        pa = 0.0 if np.isinf(a) else norm.pdf(a)
        pb = 0.0 if np.isinf(b) else norm.pdf(b)
        apa = 0.0 if np.isinf(a) else a * pa
        bpb = 0.0 if np.isinf(b) else b * pb
        total += (1.0 + y * y) * (Pb - Pa) - (bpb - apa) + 2.0 * y * (pb - pa)
    return float(total)


def quest_alpha(bits: int) -> float:
    """The endpoint alpha_b minimizing gaussian_grid_mse (appendix B.3's
    optimal endpoint), by bounded scalar minimization."""
    from scipy.optimize import minimize_scalar
    r = minimize_scalar(lambda a: gaussian_grid_mse(a, bits), bounds=(0.3, 6.0),
                        method="bounded", options={"xatol": 1e-12, "maxiter": 500})
    return float(r.x)


def dequantize(codes, s16, z16) -> np.ndarray:
    """xhat = z16 + s16 * code."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    c = codes.reshape(-1, n)
    s = _f64(s16).ravel()
    z = _f64(z16).ravel()
    out = np.empty(c.shape)
    _load().wko_dequantize(c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                           _dp(s), _dp(z), c.shape[0], n, _dp(out))
    return out.reshape(codes.shape)


def squant(L: int, S: int, R: int, F: int) -> int:
    """End of the quantized region [S, S_quant) at cache length L (section 4.4)."""
    return int(_load().wko_squant(int(L), int(S), int(R), int(F)))


def compensate(T, q) -> np.ndarray:
    """q' = T^{-T} q (appendix B.1), by solving T^T q' = q in fp64."""
    T = _f64(T)
    q = _f64(q)
    return np.linalg.solve(T.T, q.reshape(-1, T.shape[0]).T).T.reshape(q.shape)


def attention(qc, K, V) -> np.ndarray:
    """Decode attention of compensated queries over a read-back cache.

    qc: [n_q, d]; K, V: [n_kv, L, d].  Returns [n_q, d] (transformed V basis).
    """
    qc = _f64(qc)
    K = _f64(K)
    V = _f64(V)
    n_q, d = qc.shape
    n_kv, L, d2 = K.shape
    assert d2 == d and V.shape == K.shape
    out = np.empty((n_q, d))
    rc = _load().wko_attention(_dp(qc), _dp(K), _dp(V), n_q, n_kv, L, d, _dp(out))
    if rc != 0:
        raise ValueError("wko_attention: bad arguments")
    return out


# --------------------------------------------------------------------------
# One (sequence, KV head) unit of the cache after it reached length L
# --------------------------------------------------------------------------

def cache_unit(keys, values, T, *, S: int, R: int, F: int, bits: int,
               p_lo: float, p_hi: float, positions=None, alpha=None):
    """State of one (sequence, KV head) cache unit at length L = len(keys).

    keys: [L, d] post-RoPE keys; values: [L, d] values already in the value
    transform's basis; T: [d, d] key transform.

    By section 4.4 the state depends only on L: positions [0, S) are the sink,
    [S, S_quant) are quantized, [S_quant, L) are the recent window.  Every
    entry is first rounded to bfloat16 (window precision); the quantizer takes
    those bfloat16 values (reading: entries are "first appended in full
    precision").  ``positions`` (optional) restricts the quantizer to a subset
    of the quantized positions (the rest of the arrays are then left as NaN /
    255) so that large units can be sampled.  ``alpha`` (optional) selects the
    symmetric RMS-normalized quantizer with that endpoint instead of the
    percentile clip.
    """
    keys = _f64(keys)
    values = _f64(values)
    L, d = keys.shape
    ktr, kabs = transform(T, keys)
    kb = bf16(ktr)
    vb = bf16(values)
    amb = bf16_ambiguous(ktr, kabs)
    # where the rounding is undecided, the other bfloat16 neighbour of T k is
    # an equally correct stored value (NaN elsewhere)
    band = np.ldexp(kabs, AMBIGUITY_BAND_LOG2)
    lo_b, hi_b = bf16(ktr - band), bf16(ktr + band)
    k_alt = np.where(amb, np.where(lo_b == kb, hi_b, lo_b), np.nan)
    sq = squant(L, S, R, F)
    qpos = np.arange(S, sq) if positions is None else np.asarray(positions)
    kcodes = np.full((L, d), 255, dtype=np.uint8)
    vcodes = np.full((L, d), 255, dtype=np.uint8)
    ks = np.full(L, np.nan)
    kz = np.full(L, np.nan)
    vs = np.full(L, np.nan)
    vz = np.full(L, np.nan)
    ku = np.full((L, d), np.nan)
    vu = np.full((L, d), np.nan)
    if qpos.size:
        if alpha is None:   # percentile clip ends
            qk = quantize(kb[qpos], bits, p_lo, p_hi)
            qv = quantize(vb[qpos], bits, p_lo, p_hi)
        else:               # symmetric, RMS-normalized grid with endpoint alpha
            qk = quantize_rms(kb[qpos], bits, alpha)
            qv = quantize_rms(vb[qpos], bits, alpha)
        kcodes[qpos], ks[qpos], kz[qpos], ku[qpos] = qk["codes"], qk["s16"], qk["z16"], qk["u"]
        vcodes[qpos], vs[qpos], vz[qpos], vu[qpos] = qv["codes"], qv["s16"], qv["z16"], qv["u"]
    return dict(L=L, S=S, squant=sq, k_bf16=kb, v_bf16=vb, k_ambiguous=amb, k_alt=k_alt,
                kcodes=kcodes, ks16=ks, kz16=kz, ku=ku,
                vcodes=vcodes, vs16=vs, vz16=vz, vu=vu, qpos=qpos,
                bits=bits, p_lo=p_lo, p_hi=p_hi, alpha=alpha)


def readback(unit) -> tuple[np.ndarray, np.ndarray]:
    """The cache a decode step reads: window entries as stored in bfloat16,
    quantized entries dequantized.  Returns (K [L, d], V [L, d])."""
    K = unit["k_bf16"].copy()
    V = unit["v_bf16"].copy()
    q = np.arange(min(unit["S"], unit["squant"]), unit["squant"])
    if not np.array_equal(np.asarray(unit["qpos"]), q):
        raise ValueError("readback needs every quantized position (no sampling)")
    if q.size:
        K[q] = dequantize(unit["kcodes"][q], unit["ks16"][q], unit["kz16"][q])
        V[q] = dequantize(unit["vcodes"][q], unit["vs16"][q], unit["vz16"][q])
    return K, V
