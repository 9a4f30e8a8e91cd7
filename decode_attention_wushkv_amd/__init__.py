"""Python binding of libwushkv (the WUSH-KV transformed low-bit KV cache for
MI355X).  Argument marshalling only: every step of the method runs in the HIP
kernels behind the C ABI declared in ``include/wushkv.h``.  PyTorch is used by
callers for device memory and streams; the binding takes raw addresses.

There is no CPU fallback: importing works anywhere, but every call needs the
built ``libwushkv.so`` (``python -m decode_attention_wushkv_amd.build``) and,
for ``wushkv_append`` / ``wushkv_decode_attn``, a gfx950 GPU.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwushkv.so")

WUSHKV_OK, WUSHKV_EINVAL, WUSHKV_ECAPACITY, WUSHKV_EWORKSPACE, WUSHKV_EUNSUPPORTED, \
    WUSHKV_EDEVICE = range(6)
WUSHKV_IO_FP32, WUSHKV_IO_BF16 = 0, 1
WUSHKV_CODEC_PERCENTILE, WUSHKV_CODEC_RMS = 0, 1
WUSHKV_MAX_SEQ_PER_CALL = 128

# Symbols the header declares (checked by the test-suite against the .so).
EXPORTS = (
    "wushkv_config_check", "wushkv_layout", "wushkv_cache_create", "wushkv_cache_destroy",
    "wushkv_reset_seq", "wushkv_get_len", "wushkv_quantized_range", "wushkv_append", "wushkv_decode_workspace_bytes",
    "wushkv_decode_attn", "wushkv_decode_step", "wushkv_decode_step_noalloc", "wushkv_set_split_events", "wushkv_set_combine_events",
    "wushkv_stream_read_probe", "wushkv_gaussian_alpha", "wushkv_set_block_table",
    "wushkv_chunk_workspace_bytes", "wushkv_chunk_step", "wushkv_status_str",
)
WUSHKV_MAX_CHUNK = 16


class wushkv_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("bits", ctypes.c_int32), ("sink", ctypes.c_int32), ("recent", ctypes.c_int32),
        ("flush", ctypes.c_int32), ("p_lo", ctypes.c_double), ("p_hi", ctypes.c_double),
        ("max_batch", ctypes.c_int32), ("ctx_cap", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("codec", ctypes.c_int32), ("clip_alpha", ctypes.c_double),
        ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32),
    ]


_U64 = ctypes.c_uint64


class wushkv_layout_t(ctypes.Structure):
    _fields_ = [("total_bytes", _U64)] + [
        (f"off_{n}", _U64) for n in ("kcode", "vcode", "ksz", "vsz", "ksink", "vsink", "kring", "vring")
    ] + [
        (f"bytes_{n}", _U64) for n in ("kcode", "vcode", "ksz", "vsz", "ksink", "vsink", "kring", "vring")
    ] + [(n, ctypes.c_int32) for n in ("code_bytes", "vblock", "ctx_blocks", "cpos", "ring_slots", "units",
                                       "page_size", "n_pages", "pages_per_seq")]


class WushkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {wushkv_status_str(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libwushkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m decode_attention_wushkv_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    i32p = ctypes.POINTER(ctypes.c_int32)
    cfgp = ctypes.POINTER(wushkv_config)
    L.wushkv_config_check.restype = ctypes.c_int
    L.wushkv_config_check.argtypes = [cfgp]
    L.wushkv_layout.restype = ctypes.c_int
    L.wushkv_layout.argtypes = [cfgp, ctypes.POINTER(wushkv_layout_t)]
    L.wushkv_cache_create.restype = ctypes.c_int
    L.wushkv_cache_create.argtypes = [cfgp, P, _U64, ctypes.POINTER(P)]
    L.wushkv_cache_destroy.restype = None
    L.wushkv_cache_destroy.argtypes = [P]
    L.wushkv_reset_seq.restype = ctypes.c_int
    L.wushkv_reset_seq.argtypes = [P, i32]
    L.wushkv_get_len.restype = ctypes.c_int
    L.wushkv_get_len.argtypes = [P, i32, i32, i32p, i32p]
    L.wushkv_quantized_range.restype = ctypes.c_int
    L.wushkv_quantized_range.argtypes = [P, i32, i32p, i32p]
    L.wushkv_append.restype = ctypes.c_int
    L.wushkv_append.argtypes = [P, i32, i32, i32p, i32p, P, P, P, P]
    L.wushkv_decode_workspace_bytes.restype = _U64
    L.wushkv_decode_workspace_bytes.argtypes = [P, i32]
    L.wushkv_decode_attn.restype = ctypes.c_int
    L.wushkv_decode_attn.argtypes = [P, i32, i32, i32p, P, P, P, P, _U64, P]
    L.wushkv_decode_step.restype = ctypes.c_int
    L.wushkv_decode_step.argtypes = [P, i32, i32, i32p, P, P, P, P, P, P, P, _U64, P]
    L.wushkv_decode_step_noalloc.restype = ctypes.c_int
    L.wushkv_decode_step_noalloc.argtypes = [P, i32, i32, i32p, P, P, P, P, P, P, P]
    L.wushkv_chunk_workspace_bytes.restype = _U64
    L.wushkv_chunk_workspace_bytes.argtypes = [P, i32, i32]
    L.wushkv_chunk_step.restype = ctypes.c_int
    L.wushkv_chunk_step.argtypes = [P, i32, i32, i32p, i32p, P, P, P, P, P, P, P, _U64, P]
    L.wushkv_set_block_table.restype = ctypes.c_int
    L.wushkv_set_block_table.argtypes = [P, P]
    L.wushkv_set_split_events.restype = ctypes.c_int
    L.wushkv_set_split_events.argtypes = [P, P, P]
    L.wushkv_set_combine_events.restype = ctypes.c_int
    L.wushkv_set_combine_events.argtypes = [P, P, P]
    L.wushkv_gaussian_alpha.restype = ctypes.c_double
    L.wushkv_gaussian_alpha.argtypes = [i32]
    L.wushkv_stream_read_probe.restype = ctypes.c_int
    L.wushkv_stream_read_probe.argtypes = [P, _U64, i32, P, P]
    L.wushkv_status_str.restype = ctypes.c_char_p
    L.wushkv_status_str.argtypes = [ctypes.c_int]
    _lib = L
    return L


def _check(st: int, where: str):
    if st != WUSHKV_OK:
        raise WushkvError(st, where)


def _i32_array(xs):
    xs = [int(x) for x in xs]
    return (ctypes.c_int32 * max(1, len(xs)))(*xs), len(xs)


def make_config(*, n_layers, n_q_heads, n_kv_heads, bits, sink, recent, flush=1, p_lo=0.01,
                p_hi=0.99, max_batch, ctx_cap, io_dtype, head_dim=128, codec=WUSHKV_CODEC_PERCENTILE,
                clip_alpha=0.0, page_size=0, n_pages=0) -> wushkv_config:
    return wushkv_config(n_layers, n_q_heads, n_kv_heads, head_dim, bits, sink, recent, flush,
                         p_lo, p_hi, max_batch, ctx_cap, io_dtype, codec, clip_alpha, page_size,
                         n_pages)


# ------------------------------------------------------------- C-ABI mirrors

def wushkv_status_str(status: int) -> str:
    return lib().wushkv_status_str(int(status)).decode()


def wushkv_config_check(cfg: wushkv_config) -> int:
    return lib().wushkv_config_check(ctypes.byref(cfg))


def wushkv_layout(cfg: wushkv_config) -> wushkv_layout_t:
    out = wushkv_layout_t()
    _check(lib().wushkv_layout(ctypes.byref(cfg), ctypes.byref(out)), "wushkv_layout")
    return out


def wushkv_cache_create(cfg: wushkv_config, arena_ptr: int, arena_bytes: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().wushkv_cache_create(ctypes.byref(cfg), ctypes.c_void_p(arena_ptr),
                                     int(arena_bytes), ctypes.byref(h)), "wushkv_cache_create")
    return h.value


def wushkv_cache_destroy(cache: int) -> None:
    lib().wushkv_cache_destroy(ctypes.c_void_p(cache))


def wushkv_reset_seq(cache: int, slot: int) -> None:
    _check(lib().wushkv_reset_seq(ctypes.c_void_p(cache), int(slot)), "wushkv_reset_seq")


def wushkv_get_len(cache: int, layer: int, slot: int):
    L = ctypes.c_int32()
    sq = ctypes.c_int32()
    _check(lib().wushkv_get_len(ctypes.c_void_p(cache), int(layer), int(slot), ctypes.byref(L),
                                ctypes.byref(sq)), "wushkv_get_len")
    return L.value, sq.value


def wushkv_quantized_range(cache: int, length: int):
    """(begin, end): the positions quantized at sequence length `length`."""
    b = ctypes.c_int32()
    e = ctypes.c_int32()
    _check(lib().wushkv_quantized_range(ctypes.c_void_p(cache), int(length), ctypes.byref(b),
                                        ctypes.byref(e)), "wushkv_quantized_range")
    return b.value, e.value


def wushkv_append(cache: int, layer: int, slots, n_new, k_ptr: int, v_ptr: int, tk_ptr: int,
                  stream: int = 0, *, check: bool = True) -> int:
    s, n = _i32_array(slots)
    nn, n2 = _i32_array(n_new)
    assert n == n2
    st = lib().wushkv_append(ctypes.c_void_p(cache), int(layer), n, s, nn, ctypes.c_void_p(k_ptr),
                             ctypes.c_void_p(v_ptr), ctypes.c_void_p(tk_ptr), ctypes.c_void_p(stream))
    if check:
        _check(st, "wushkv_append")
    return st


def wushkv_decode_workspace_bytes(cache: int, n_seq: int) -> int:
    return int(lib().wushkv_decode_workspace_bytes(ctypes.c_void_p(cache), int(n_seq)))


def wushkv_decode_attn(cache: int, layer: int, slots, q_ptr: int, tq_ptr: int, out_ptr: int,
                       ws_ptr: int, ws_bytes: int, stream: int = 0, *, check: bool = True) -> int:
    s, n = _i32_array(slots)
    st = lib().wushkv_decode_attn(ctypes.c_void_p(cache), int(layer), n, s, ctypes.c_void_p(q_ptr),
                                  ctypes.c_void_p(tq_ptr), ctypes.c_void_p(out_ptr),
                                  ctypes.c_void_p(ws_ptr), int(ws_bytes), ctypes.c_void_p(stream))
    if check:
        _check(st, "wushkv_decode_attn")
    return st


def wushkv_decode_step(cache: int, layer: int, slots, k_ptr: int, v_ptr: int, tk_ptr: int,
                       q_ptr: int, tq_ptr: int, out_ptr: int, ws_ptr: int, ws_bytes: int,
                       stream: int = 0, *, check: bool = True) -> int:
    s, n = _i32_array(slots)
    vp = ctypes.c_void_p
    st = lib().wushkv_decode_step(vp(cache), int(layer), n, s, vp(k_ptr), vp(v_ptr), vp(tk_ptr),
                                  vp(q_ptr), vp(tq_ptr), vp(out_ptr), vp(ws_ptr), int(ws_bytes),
                                  vp(stream))
    if check:
        _check(st, "wushkv_decode_step")
    return st


WUSHKV_NOALLOC_SCRATCH_BYTES = 16 << 20


def wushkv_decode_step_noalloc(cache: int, layer: int, slots, k_ptr: int, v_ptr: int, tk_ptr: int,
                               q_ptr: int, tq_ptr: int, out_ptr: int, stream: int = 0, *,
                               check: bool = True) -> int:
    """wushkv_decode_step with the library's own per-GPU scratch as workspace
    (no allocation); calls that overlap on one GPU race."""
    s, n = _i32_array(slots)
    vp = ctypes.c_void_p
    st = lib().wushkv_decode_step_noalloc(vp(cache), int(layer), n, s, vp(k_ptr), vp(v_ptr),
                                          vp(tk_ptr), vp(q_ptr), vp(tq_ptr), vp(out_ptr),
                                          vp(stream))
    if check:
        _check(st, "wushkv_decode_step_noalloc")
    return st


def wushkv_chunk_workspace_bytes(cache: int, n_seq: int, max_new: int) -> int:
    return int(lib().wushkv_chunk_workspace_bytes(ctypes.c_void_p(cache), int(n_seq), int(max_new)))


def wushkv_chunk_step(cache: int, layer: int, slots, n_new, k_ptr: int, v_ptr: int, tk_ptr: int,
                      q_ptr: int, tq_ptr: int, out_ptr: int, ws_ptr: int, ws_bytes: int,
                      stream: int = 0, *, check: bool = True) -> int:
    s, n = _i32_array(slots)
    nn, n2 = _i32_array(n_new)
    assert n == n2
    vp = ctypes.c_void_p
    st = lib().wushkv_chunk_step(vp(cache), int(layer), n, s, nn, vp(k_ptr), vp(v_ptr), vp(tk_ptr),
                                 vp(q_ptr), vp(tq_ptr), vp(out_ptr), vp(ws_ptr), int(ws_bytes),
                                 vp(stream))
    if check:
        _check(st, "wushkv_chunk_step")
    return st


def wushkv_gaussian_alpha(bits: int) -> float:
    return float(lib().wushkv_gaussian_alpha(int(bits)))


def wushkv_stream_read_probe(buf_ptr: int, nbytes: int, blocks: int, out_ptr: int,
                             stream: int = 0) -> None:
    """Instrumentation: one grid-stride streaming read of nbytes at buf_ptr."""
    _check(lib().wushkv_stream_read_probe(ctypes.c_void_p(buf_ptr), int(nbytes), int(blocks),
                                          ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream)),
           "wushkv_stream_read_probe")


def wushkv_set_block_table(cache: int, table_ptr: int) -> None:
    _check(lib().wushkv_set_block_table(ctypes.c_void_p(cache), ctypes.c_void_p(table_ptr)),
           "wushkv_set_block_table")


def wushkv_set_split_events(cache: int, ev_start: int | None, ev_stop: int | None) -> None:
    _check(lib().wushkv_set_split_events(ctypes.c_void_p(cache), ctypes.c_void_p(ev_start or 0),
                                         ctypes.c_void_p(ev_stop or 0)), "wushkv_set_split_events")


def wushkv_set_combine_events(cache: int, ev_start: int | None, ev_stop: int | None) -> None:
    _check(lib().wushkv_set_combine_events(ctypes.c_void_p(cache), ctypes.c_void_p(ev_start or 0),
                                           ctypes.c_void_p(ev_stop or 0)), "wushkv_set_combine_events")
