"""Host-side checks of the C ABI (no GPU needed): the library loads and
exports every function include/wushkv.h declares, configs are validated, the
arena layout reproduces the pages' footprint arithmetic, and invalid calls
fail before any launch without changing state."""
import ctypes
import json
import os
import re

import pytest

import decode_attention_wushkv_amd as wk
from decode_attention_wushkv_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(wk.LIB_PATH):
        build.build()


def header_functions():
    src = open(os.path.join(ROOT, "include", "wushkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wushkv_[a-z_]+)\s*\(", src)))


def test_exports_every_header_function():
    names = header_functions()
    assert set(names) == set(wk.EXPORTS)
    lib = ctypes.CDLL(wk.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _cfg(**kw):
    base = dict(n_layers=32, n_q_heads=32, n_kv_heads=32, bits=2, sink=4, recent=128, flush=1,
                p_lo=0.01, p_hi=0.99, max_batch=1, ctx_cap=131072, io_dtype=wk.WUSHKV_IO_BF16)
    base.update(kw)
    return wk.make_config(**base)


def test_footprint_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "footprint.json")))
    cfg = _cfg(n_layers=g["n_layers"], n_kv_heads=g["n_kv_heads"], n_q_heads=g["n_kv_heads"],
               ctx_cap=g["context"])
    lay = wk.wushkv_layout(cfg)
    # values per token: 2 (K, V) x layers x KV heads x head_dim
    vals = 2 * cfg.n_layers * cfg.n_kv_heads * cfg.head_dim
    assert vals == g["values_per_token"]
    assert vals * 2 == g["fp16_bytes_per_token"]
    assert vals * 2 * g["context"] == g["fp16_bytes_per_sequence"]
    # the 2-bit code planes hold exactly 2 bits per cached value
    assert lay.bytes_kcode + lay.bytes_vcode == g["two_bit_code_bytes_per_sequence"]
    # scale/zero overhead, reported separately: 4 B per (token, layer, KV head) per K/V
    assert lay.bytes_ksz + lay.bytes_vsz == 2 * 4 * cfg.n_layers * cfg.n_kv_heads * g["context"]
    assert lay.bytes_ksz + lay.bytes_vsz == 1 << 30
    # windows: bf16 sink + ring per unit
    units = cfg.n_layers * cfg.n_kv_heads
    assert lay.bytes_ksink == units * 4 * 128 * 2
    assert lay.bytes_kring == units * 128 * 128 * 2
    assert lay.total_bytes % 256 == 0
    for n in ("kcode", "vcode", "ksz", "vsz", "ksink", "vsink", "kring", "vring"):
        assert getattr(lay, f"off_{n}") % 256 == 0


def test_footprint_4bit():
    lay = wk.wushkv_layout(_cfg(bits=4))
    assert lay.bytes_kcode + lay.bytes_vcode == 2 * 8589934592
    assert lay.vblock == 32 and lay.code_bytes == 64


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), wk.WUSHKV_EUNSUPPORTED),
    (dict(bits=5), wk.WUSHKV_EUNSUPPORTED),
    (dict(bits=1), wk.WUSHKV_EUNSUPPORTED),
    (dict(bits=3), wk.WUSHKV_OK),
    (dict(n_q_heads=30, n_kv_heads=8), wk.WUSHKV_EINVAL),
    (dict(n_q_heads=24, n_kv_heads=8), wk.WUSHKV_EUNSUPPORTED),
    (dict(p_lo=0.5, p_hi=0.5), wk.WUSHKV_EINVAL),
    (dict(p_lo=-0.1), wk.WUSHKV_EINVAL),
    (dict(flush=0), wk.WUSHKV_EINVAL),
    (dict(recent=-1), wk.WUSHKV_EINVAL),
    (dict(ctx_cap=0), wk.WUSHKV_EINVAL),
    (dict(io_dtype=7), wk.WUSHKV_EINVAL),
    (dict(recent=1100), wk.WUSHKV_EUNSUPPORTED),
    (dict(), wk.WUSHKV_OK),
])
def test_config_check(kw, status):
    assert wk.wushkv_config_check(_cfg(**kw)) == status


FAKE_ARENA = 1 << 40   # an aligned address that is never dereferenced by these host-only calls


def _fake_cache(**kw):
    cfg = _cfg(n_layers=2, n_q_heads=8, n_kv_heads=2, max_batch=4, ctx_cap=100, **kw)
    lay = wk.wushkv_layout(cfg)
    return wk.wushkv_cache_create(cfg, FAKE_ARENA, lay.total_bytes), lay


def test_cache_create_checks_arena():
    cfg = _cfg(n_layers=1, max_batch=1, ctx_cap=100)
    lay = wk.wushkv_layout(cfg)
    with pytest.raises(wk.WushkvError):
        wk.wushkv_cache_create(cfg, FAKE_ARENA + 16, lay.total_bytes)
    with pytest.raises(wk.WushkvError):
        wk.wushkv_cache_create(cfg, FAKE_ARENA, lay.total_bytes - 1)
    h = wk.wushkv_cache_create(cfg, FAKE_ARENA, lay.total_bytes)
    assert wk.wushkv_get_len(h, 0, 0) == (0, 4)
    wk.wushkv_cache_destroy(h)


def test_append_errors_leave_state_unchanged():
    h, _ = _fake_cache()
    P = 1 << 41
    assert wk.wushkv_append(h, 0, [0, 0], [1, 1], P, P, P, check=False) == wk.WUSHKV_EINVAL  # duplicate
    assert wk.wushkv_append(h, 0, [5], [1], P, P, P, check=False) == wk.WUSHKV_EINVAL        # slot range
    assert wk.wushkv_append(h, 2, [0], [1], P, P, P, check=False) == wk.WUSHKV_EINVAL        # layer range
    assert wk.wushkv_append(h, 0, [0], [-1], P, P, P, check=False) == wk.WUSHKV_EINVAL
    assert wk.wushkv_append(h, 0, [0, 1], [50, 101], P, P, P, check=False) == wk.WUSHKV_ECAPACITY
    assert wk.wushkv_append(h, 0, [0], [1], 0, P, P, check=False) == wk.WUSHKV_EINVAL        # null k
    assert wk.wushkv_append(h, 0, [0], [1], P + 1, P, P, check=False) == wk.WUSHKV_EINVAL    # misaligned
    assert wk.wushkv_append(h, 0, list(range(4)) * 40, [0] * 160, P, P, P, check=False) == \
        wk.WUSHKV_EUNSUPPORTED
    assert wk.wushkv_append(h, 0, [0, 1], [0, 0], P, P, P, check=False) == wk.WUSHKV_OK      # no-op
    for s in range(4):
        assert wk.wushkv_get_len(h, 0, s) == (0, 4)
    wk.wushkv_cache_destroy(h)


def test_decode_errors():
    h, _ = _fake_cache()
    P = 1 << 41
    need = wk.wushkv_decode_workspace_bytes(h, 2)
    assert need > 0
    # empty sequences cannot be decoded
    assert wk.wushkv_decode_attn(h, 0, [0], P, P, P, P, need, check=False) == wk.WUSHKV_EINVAL
    assert wk.wushkv_decode_attn(h, 0, [0, 1], P, P, P, P, need - 1, check=False) == wk.WUSHKV_EWORKSPACE
    assert wk.wushkv_decode_attn(h, 0, [1, 1], P, P, P, P, need, check=False) == wk.WUSHKV_EINVAL
    assert wk.wushkv_decode_attn(h, 0, [0], 0, P, P, P, need, check=False) == wk.WUSHKV_EINVAL
    assert wk.wushkv_decode_attn(h, 0, [0], P, P, P + 4, P, need, check=False) == wk.WUSHKV_EINVAL
    wk.wushkv_cache_destroy(h)


def test_decode_step_errors():
    h, _ = _fake_cache()
    P = 1 << 41
    need = wk.wushkv_decode_workspace_bytes(h, 2)
    step = lambda slots, k=P, tk=P, out=P, ws=need: wk.wushkv_decode_step(
        h, 0, slots, k, P, tk, P, P, out, P, ws, check=False)
    assert step([0, 1], ws=need - 1) == wk.WUSHKV_EWORKSPACE
    assert step([1, 1]) == wk.WUSHKV_EINVAL                  # duplicate slot
    assert step([0], k=0) == wk.WUSHKV_EINVAL                # null key
    assert step([0], tk=P + 4) == wk.WUSHKV_EINVAL           # misaligned T_K
    assert step([0], out=P + 4) == wk.WUSHKV_EINVAL          # misaligned output
    assert wk.wushkv_decode_step(h, 2, [0], P, P, P, P, P, P, P, need, check=False) == \
        wk.WUSHKV_EINVAL                                     # layer range
    for s in range(4):
        assert wk.wushkv_get_len(h, 0, s) == (0, 4)
    wk.wushkv_cache_destroy(h)
    # a window of sink + recent + flush = 1025 entries passes the config check
    # (the append path needs one fewer) but not the fused step
    h, _ = _fake_cache(recent=1020)
    assert wk.wushkv_decode_step(h, 0, [0], P, P, P, P, P, P, P, need, check=False) == \
        wk.WUSHKV_EUNSUPPORTED
    wk.wushkv_cache_destroy(h)


def test_reset_and_status_strings():
    h, _ = _fake_cache()
    wk.wushkv_reset_seq(h, 3)
    with pytest.raises(wk.WushkvError):
        wk.wushkv_reset_seq(h, 4)
    wk.wushkv_cache_destroy(h)
    for s in range(6):
        assert wk.wushkv_status_str(s)
    assert wk.wushkv_status_str(99) == "unknown status"


def test_gaussian_alpha_matches_oracle():
    """The library's own endpoint computation agrees with the oracle's
    (independent implementations of the same minimization)."""
    import oracle
    for bits in (2, 3, 4):
        a = wk.wushkv_gaussian_alpha(bits)
        assert abs(a - oracle.quest_alpha(bits)) <= 1e-6 * a
    assert wk.wushkv_gaussian_alpha(0) == 0.0 and wk.wushkv_gaussian_alpha(9) == 0.0


def test_codec_config_check():
    assert wk.wushkv_config_check(_cfg(codec=wk.WUSHKV_CODEC_RMS)) == wk.WUSHKV_OK
    assert wk.wushkv_config_check(_cfg(codec=wk.WUSHKV_CODEC_RMS, clip_alpha=2.0)) == wk.WUSHKV_OK
    assert wk.wushkv_config_check(_cfg(codec=2)) == wk.WUSHKV_EINVAL
    assert wk.wushkv_config_check(_cfg(clip_alpha=-1.0)) == wk.WUSHKV_EINVAL
    assert wk.wushkv_config_check(_cfg(clip_alpha=float("nan"))) == wk.WUSHKV_EINVAL


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=128, n_pages=10), wk.WUSHKV_OK),
    (dict(page_size=4096, n_pages=1), wk.WUSHKV_OK),
    (dict(page_size=64, n_pages=10), wk.WUSHKV_EINVAL),     # below one decode sub-chunk
    (dict(page_size=384, n_pages=10), wk.WUSHKV_EINVAL),    # not a power of two
    (dict(page_size=128, n_pages=0), wk.WUSHKV_EINVAL),     # empty pool
    (dict(page_size=0, n_pages=3), wk.WUSHKV_EINVAL),       # pool size without paging
    (dict(page_size=1 << 21, n_pages=1), wk.WUSHKV_EINVAL),
])
def test_paged_config_check(kw, status):
    assert wk.wushkv_config_check(_cfg(**kw)) == status


def test_paged_layout():
    """Paged planes hold n_pages pages of page_size positions per (layer, KV
    head); windows stay per slot; the block-table row covers ctx_cap."""
    cfg = _cfg(n_layers=3, n_kv_heads=8, n_q_heads=32, max_batch=5, ctx_cap=1000,
               page_size=256, n_pages=7)
    lay = wk.wushkv_layout(cfg)
    rows = 3 * 7 * 8 * 256
    assert (lay.page_size, lay.n_pages, lay.pages_per_seq) == (256, 7, 4)
    assert lay.bytes_kcode == rows * 32 and lay.bytes_vcode == rows * 32
    assert lay.bytes_ksz == rows * 4 and lay.bytes_vsz == rows * 4
    assert lay.bytes_ksink == 3 * 5 * 8 * 4 * 256
    assert lay.bytes_kring == 3 * 5 * 8 * 128 * 256
    flat = wk.wushkv_layout(_cfg(n_layers=3, n_kv_heads=8, n_q_heads=32, max_batch=5, ctx_cap=1000))
    assert (flat.page_size, flat.n_pages, flat.pages_per_seq) == (0, 0, 0)
    assert flat.bytes_ksink == lay.bytes_ksink


def test_block_table_binding():
    P = 1 << 41
    h, _ = _fake_cache()
    with pytest.raises(wk.WushkvError):      # contiguous cache
        wk.wushkv_set_block_table(h, P)
    wk.wushkv_cache_destroy(h)
    h, _ = _fake_cache(page_size=128, n_pages=4)
    need = wk.wushkv_decode_workspace_bytes(h, 1)
    # no table bound yet: appends and decodes are refused before any launch
    assert wk.wushkv_append(h, 0, [0], [1], P, P, P, check=False) == wk.WUSHKV_EINVAL
    assert wk.wushkv_decode_step(h, 0, [0], P, P, P, P, P, P, P, need, check=False) == \
        wk.WUSHKV_EINVAL
    with pytest.raises(wk.WushkvError):
        wk.wushkv_set_block_table(h, 0)
    with pytest.raises(wk.WushkvError):
        wk.wushkv_set_block_table(h, P + 2)
    wk.wushkv_set_block_table(h, P)
    assert wk.wushkv_append(h, 0, [0], [0], P, P, P, check=False) == wk.WUSHKV_OK
    assert wk.wushkv_get_len(h, 0, 0) == (0, 4)
    wk.wushkv_cache_destroy(h)


def test_layout_3bit():
    """3-bit planes: 48 bytes per position and head for K and for V (the
    scope's non-power-of-two packing), value blocks of 128 positions."""
    lay = wk.wushkv_layout(_cfg(bits=3))
    assert lay.code_bytes == 48 and lay.vblock == 128
    assert lay.bytes_kcode == lay.bytes_vcode == 32 * 32 * 131072 * 48
    assert lay.bytes_ksz == 32 * 32 * 131072 * 4


def test_3bit_high_plane_order():
    """The documented high-plane order: a bijection on the 128 elements, and
    (word >> k) & 0x11111111 yields, nibble for nibble, the elements whose low
    bits the 2-bit unpacking (w & 0x33333333, (w >> 2) & 0x33333333) of word
    2 j + (k >> 1) yields."""
    import numpy as np
    from cachepack import HI, pack3, unpack3
    assert sorted(HI.tolist()) == list(range(128))
    for j in range(4):
        for k in range(4):
            w = 2 * j + (k >> 1)
            for n in range(8):
                lo_elem = 16 * w + 2 * n + (k & 1)     # nibble n of the 2-bit unpacking
                assert HI[lo_elem] == 32 * j + 4 * n + k
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 8, size=(37, 128), dtype=np.uint8)
    lo, hi = pack3(codes)
    assert lo.shape == (37, 32) and hi.shape == (37, 16)
    assert np.array_equal(unpack3(lo, hi), codes)


def test_chunk_step_errors():
    """Argument checks of wushkv_chunk_step fail before any launch and leave
    the lengths unchanged."""
    P = 1 << 41
    h, _ = _fake_cache()
    need = wk.wushkv_chunk_workspace_bytes(h, 2, 16)
    assert need > 0 and wk.wushkv_chunk_workspace_bytes(h, 2, 17) == 0
    assert wk.wushkv_chunk_workspace_bytes(h, 2, 0) == 0
    step = lambda slots, nn, ws=need, q=P, k=P: wk.wushkv_chunk_step(
        h, 0, slots, nn, k, P, P, q, P, P, P, ws, check=False)
    assert step([0, 1], [16, 16], ws=need - 1) == wk.WUSHKV_EWORKSPACE
    assert step([0, 1], [17, 1]) == wk.WUSHKV_EINVAL          # chunk too long
    assert step([0, 1], [0, 1]) == wk.WUSHKV_EINVAL           # empty chunk
    assert step([1, 1], [1, 1]) == wk.WUSHKV_EINVAL           # duplicate slot
    assert step([0], [1], q=0) == wk.WUSHKV_EINVAL            # null query
    assert step([0], [1], k=P + 1) == wk.WUSHKV_EINVAL        # misaligned key
    for s in range(4):
        assert wk.wushkv_get_len(h, 0, s) == (0, 4)
    wk.wushkv_cache_destroy(h)
    # 3- and 4-bit caches take the same argument checks (no launch here)
    for bits in (3, 4):
        h, _ = _fake_cache(bits=bits)
        assert wk.wushkv_chunk_step(h, 0, [0], [17], P, P, P, P, P, P, P, need, check=False) == \
            wk.WUSHKV_EINVAL
        small = wk.wushkv_chunk_workspace_bytes(h, 1, 1)
        assert wk.wushkv_chunk_step(h, 0, [0], [1], P, P, P, P, P, P, P, small - 1, check=False) == \
            wk.WUSHKV_EWORKSPACE
        wk.wushkv_cache_destroy(h)


def test_quantized_range():
    """The quantized positions [sink, S_quant(L)) by length, from section 4.4
    (sink 4, recent 128, flush 1 / 16), computed by hand; the binding and
    the device plumbing take the window rule from this call."""
    import ctypes
    h, _ = _fake_cache()
    for L, want in [(0, 4), (1, 4), (132, 4), (133, 5), (1000, 872)]:
        assert wk.wushkv_quantized_range(h, L) == (4, want)
    b, e = ctypes.c_int32(), ctypes.c_int32()
    assert wk.lib().wushkv_quantized_range(ctypes.c_void_p(h), -1, ctypes.byref(b),
                                           ctypes.byref(e)) == wk.WUSHKV_EINVAL
    assert wk.lib().wushkv_quantized_range(ctypes.c_void_p(h), 5, None,
                                           ctypes.byref(e)) == wk.WUSHKV_EINVAL
    wk.wushkv_cache_destroy(h)
    h, _ = _fake_cache(sink=16, flush=16)
    # 16 + 16 * floor((L - 128 - 16) / 16)
    for L, want in [(144, 16), (159, 16), (160, 32), (1000, 864)]:
        assert wk.wushkv_quantized_range(h, L) == (16, want)
    wk.wushkv_cache_destroy(h)


def test_decode_step_noalloc_limits():
    """The no-allocation decode step checks its arguments and the size of the
    workspace it needs against its fixed scratch before touching the device:
    a step whose workspace exceeds the scratch (8 sequences with 64 query
    heads: 17.6 MB of split partials) is refused with EWORKSPACE, invalid
    arguments with EINVAL, and lengths stay unchanged."""
    P = 1 << 41
    cfg = _cfg(n_layers=1, n_q_heads=64, n_kv_heads=8, max_batch=8, ctx_cap=1000)
    lay = wk.wushkv_layout(cfg)
    h = wk.wushkv_cache_create(cfg, FAKE_ARENA, lay.total_bytes)
    assert wk.wushkv_decode_workspace_bytes(h, 8) > wk.WUSHKV_NOALLOC_SCRATCH_BYTES
    step = lambda slots, q=P: wk.wushkv_decode_step_noalloc(h, 0, slots, P, P, P, q, P, P,
                                                            check=False)
    assert step(list(range(8))) == wk.WUSHKV_EWORKSPACE
    assert step([]) == wk.WUSHKV_OK
    for s in range(8):
        assert wk.wushkv_get_len(h, 0, s) == (0, 4)
    wk.wushkv_cache_destroy(h)
    h, _ = _fake_cache()   # groups of 4: a small workspace
    step = lambda slots, q=P: wk.wushkv_decode_step_noalloc(h, 0, slots, P, P, P, q, P, P,
                                                            check=False)
    assert step([0, 0]) == wk.WUSHKV_EINVAL       # duplicate slot
    assert step([0], q=0) == wk.WUSHKV_EINVAL     # null query
    assert step([7]) == wk.WUSHKV_EINVAL          # slot out of range
    for s in range(4):
        assert wk.wushkv_get_len(h, 0, s) == (0, 4)
    wk.wushkv_cache_destroy(h)


def test_event_hooks_check_arguments():
    """Both instrumentation hooks take two events or none (host-only calls)."""
    h, _ = _fake_cache()
    E = 1 << 41
    for fn in (wk.wushkv_set_split_events, wk.wushkv_set_combine_events):
        with pytest.raises(wk.WushkvError):
            fn(h, E, None)
        with pytest.raises(wk.WushkvError):
            fn(h, None, E)
        with pytest.raises(wk.WushkvError):
            fn(0, E, E)
        fn(h, E, E)
        fn(h, None, None)
    wk.wushkv_cache_destroy(h)
