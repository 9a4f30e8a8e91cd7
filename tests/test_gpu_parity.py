"""GPU parity of libwushkv against the fp64 CPU oracle (small and medium sizes).

Stages, each with its own tolerance:
  T  transformed keys as stored in the bfloat16 windows: bit-exact except where
     the oracle flags the bfloat16 rounding of T k as undecided by fp64.
  Q  codes: >= 99.99 % equal and every mismatch one level off with the
     oracle's code coordinate within 1e-5 of a rounding boundary; binary16
     scale and zero within 1e-6 relative.
  A  attention output per (sequence, query head):
     max_i |o_i - r_i| <= 2e-3 * max_i |r_i|.
All inputs come from the seeded synthetic generator; nothing the oracle reads
comes from the GPU path.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_wushkv_amd import synth
from decode_attention_wushkv_amd.device_cache import DeviceCache

from cachepack import read_unit, write_unit
from gpu_checks import ATOL_REL, check_attention, check_codes, check_windows, reference_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_wushkv_amd import build
    if build.is_stale():
        build.build()
    torch.cuda.set_device(0)


def _cache(w: synth.Workload, *, bits=None, S=None, R=None, F=None, max_batch=None, ctx_cap=None,
           p_lo=None, p_hi=None, n_layers=None, rms_alpha=None, page=0):
    """page > 0: a paged cache with pages of that many positions, a pool of
    every slot's worth plus three, handed out in a seeded shuffled order (so
    consecutive pages of a sequence are scattered through the pool)."""
    codec = {} if rms_alpha is None else dict(codec=1, clip_alpha=rms_alpha)
    if page:
        nb, cap = max_batch or w.batch, ctx_cap or max(w.lengths())
        codec.update(page_size=page, n_pages=nb * ((cap + page - 1) // page) + 3,
                     page_seed=1234 + page)
    return DeviceCache(n_layers=n_layers or 1, n_q_heads=w.n_q, n_kv_heads=w.n_kv,
                       bits=bits or w.bits[0], sink=w.sink if S is None else S,
                       recent=w.recent if R is None else R, flush=F or w.flush,
                       p_lo=p_lo or w.p_lo, p_hi=p_hi or w.p_hi,
                       max_batch=max_batch or w.batch, ctx_cap=ctx_cap or max(w.lengths()),
                       io_dtype=w.torch_io, device="cuda", **codec)


def _alpha_of(dc):
    """The oracle's argument for the cache's codec: None (percentile clip) or
    the RMS codec's endpoint."""
    return dc.cfg.clip_alpha if dc.cfg.codec == 1 else None


def _inputs(w, layer, seq, L):
    k, v = synth.keys_values(w, layer, seq, 0, L)
    return k, v


def _append_all(dc, layer, slots, ks, vs, T, plan):
    """Append each sequence's tokens following plan = list of chunk sizes
    (applied to every sequence in the call, clipped to what remains)."""
    pos = [0] * len(slots)
    tk = torch.from_numpy(T).cuda()
    for n in plan:
        nn = [min(n, ks[i].shape[0] - pos[i]) for i in range(len(slots))]
        if sum(nn) == 0:
            continue
        kk = torch.cat([ks[i][pos[i]:pos[i] + nn[i]] for i in range(len(slots))]).cuda().contiguous()
        vv = torch.cat([vs[i][pos[i]:pos[i] + nn[i]] for i in range(len(slots))]).cuda().contiguous()
        dc.append(layer, slots, nn, kk, vv, tk)
        pos = [p + n_ for p, n_ in zip(pos, nn)]
    assert all(p == k.shape[0] for p, k in zip(pos, ks))


def _oracle_units(w, ks, vs, T, dc):
    c = dc.cfg
    units = {}
    for si, (k, v) in enumerate(zip(ks, vs)):
        for h in range(w.n_kv):
            units[(si, h)] = oracle.cache_unit(
                k[:, h].double().numpy(), v[:, h].double().numpy(), T[h].astype(np.float64),
                S=c.sink, R=c.recent, F=c.flush, bits=c.bits, p_lo=c.p_lo, p_hi=c.p_hi,
                alpha=_alpha_of(dc))
    return units


def _check_state(dc, w, ks, vs, T):
    """T and Q stages for every (sequence, KV head) of layer 0 against the
    oracle's cache at the sequences' full lengths; returns the oracle units."""
    units = _oracle_units(w, ks, vs, T, dc)
    for (si, h), orc in units.items():
        assert dc.get_len(0, si) == (orc["L"], orc["squant"])
        gpu = read_unit(dc, 0, si, h, orc["L"])
        check_windows(gpu, orc)
        check_codes(gpu, orc, dc.cfg.bits)
    return units


def _run_e2e(w, plan, *, bits=None, S=None, R=None, F=None, p_lo=None, p_hi=None, lengths=None,
             check_attn=True, rms_alpha=None, page=0):
    lengths = lengths or w.lengths()
    dc = _cache(w, bits=bits, S=S, R=R, F=F, p_lo=p_lo, p_hi=p_hi, max_batch=len(lengths),
                ctx_cap=max(lengths), rms_alpha=rms_alpha, page=page)
    T, Tq = synth.transforms(w, 0)
    ks, vs = zip(*[_inputs(w, 0, si, L) for si, L in enumerate(lengths)])
    slots = list(range(len(lengths)))
    _append_all(dc, 0, slots, ks, vs, T, plan)
    torch.cuda.synchronize()
    units = _check_state(dc, w, ks, vs, T)
    if not check_attn:
        return dc
    q = synth.queries(w, 0, 0, len(lengths))
    out = dc.decode_attn(0, slots, q.cuda(), torch.from_numpy(Tq).cuda()).cpu().numpy()
    for si in range(len(lengths)):
        ref = reference_attention(w, T, q[si], {h: units[(si, h)] for h in range(w.n_kv)})
        check_attention(out[si], ref)
    return dc


# ------------------------------------------------------------------ tests

def test_cfg0_prefill_then_decode_steps():
    """1 layer, 1 KV head, 4 query heads, fp32 io, 1024 positions: a prefill of
    1000 positions then 24 one-token appends (ring evictions each step)."""
    w = synth.WORKLOADS[0]
    _run_e2e(w, [1000] + [1] * 24)


def test_cfg0_token_by_token_small():
    w = synth.WORKLOADS[0]
    _run_e2e(w, [1] * 300, lengths=[300])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_cfg0_bits(bits):
    w = synth.WORKLOADS[0]
    _run_e2e(w, [700, 5, 300, 19], bits=bits)


def test_transform_stage_nothing_quantized():
    """T stage: with S + R >= L every entry stays in bfloat16."""
    w = synth.WORKLOADS[0]
    _run_e2e(w, [999, 1], R=1000, lengths=[1000])


def test_cfg1_llama_layer_32k():
    """32 query / 8 KV heads, bf16, 32768 positions: prefill 32767 + one decode
    append, full parity on all 8 KV heads."""
    w = synth.WORKLOADS[1]
    _run_e2e(w, [32767, 1])


def test_prefill_equals_token_by_token():
    """Section 4.4's state depends only on the length: a single prefill and a
    ragged sequence of appends give bit-identical caches."""
    w = synth.WORKLOADS[1]
    L = 1500
    dc = _cache(w, max_batch=2, ctx_cap=L)
    T, _ = synth.transforms(w, 0)
    k, v = _inputs(w, 0, 0, L)
    tk = torch.from_numpy(T).cuda()
    dc.append(0, [0], [L], k.cuda(), v.cuda(), tk)
    pos = 0
    for n in [1, 3, 17, 300, 1, 1, 64, 600, 1, 2, 255, 129, 130]:
        n = min(n, L - pos)
        dc.append(0, [1], [n], k[pos:pos + n].cuda().contiguous(), v[pos:pos + n].cuda().contiguous(), tk)
        pos += n
    if pos < L:
        dc.append(0, [1], [L - pos], k[pos:].cuda().contiguous(), v[pos:].cuda().contiguous(), tk)
    torch.cuda.synchronize()
    for h in range(w.n_kv):
        a = read_unit(dc, 0, 0, h, L)
        b = read_unit(dc, 0, 1, h, L)
        sq = a["squant"]
        for key in ("kcodes", "vcodes"):
            assert np.array_equal(a[key][4:sq], b[key][4:sq])
        for key in ("ks16", "kz16", "vs16", "vz16"):
            assert np.array_equal(a[key][4:sq], b[key][4:sq])
        for key in ("kwin", "vwin"):
            assert np.array_equal(np.nan_to_num(a[key], nan=7.0), np.nan_to_num(b[key], nan=7.0))


def test_ragged_batch_gqa():
    """Three sequences of different lengths in one call; a zero-length append
    for one of them mid-way."""
    w = synth.WORKLOADS[1]
    _run_e2e(w, [700, 3, 1, 1, 600, 5], lengths=[1310, 2, 907])


@pytest.mark.parametrize("S,R,F", [(0, 32, 1), (4, 0, 1), (16, 128, 16), (1, 5, 3)])
def test_window_variants(S, R, F):
    w = synth.WORKLOADS[0]
    _run_e2e(w, [513, 1, 1, 70, 1], S=S, R=R, F=F, lengths=[586])


def _bf16_workload(L, *, bits=2, S=4, R=128, F=1, p_lo=0.01, p_hi=0.99, n_kv=2, G=4):
    return synth.Workload(11, "prefill-bf16", 1, n_kv * G, n_kv, 1, L, (bits,), S, R, F, p_lo, p_hi,
                          "bf16")


@pytest.mark.parametrize("S,R,F", [(0, 32, 1), (4, 0, 1), (16, 128, 16), (1, 5, 3)])
def test_prefill_bf16_window_variants(S, R, F):
    """bfloat16 inputs take the matrix-core prefill kernel: tiles that start
    and end mid-block, sink and ring positions inside tiles, flush > 1."""
    w = _bf16_workload(2900, S=S, R=R, F=F)
    _run_e2e(w, [37, 2000, 1, 700, 150, 1, 11])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_prefill_bf16_bits(bits):
    w = _bf16_workload(3000, bits=bits)
    _run_e2e(w, [1100, 1900])


@pytest.mark.parametrize("p_lo,p_hi", [(0.0, 1.0), (0.0157, 0.985), (0.01, 0.995), (0.05, 0.9)])
def test_prefill_bf16_percentiles(p_lo, p_hi):
    """Clip percentiles at the ends of what the selection kernel covers (min and
    max; interpolation between the 2nd and 3rd smallest / 3rd and 2nd largest),
    and one that falls back to the rank-sort kernel (0.05 / 0.9)."""
    w = _bf16_workload(1500, p_lo=p_lo, p_hi=p_hi)
    _run_e2e(w, [1500])


def test_short_sequences_sink_only():
    w = synth.WORKLOADS[0]
    _run_e2e(w, [1, 1, 1], lengths=[3])


def test_other_percentiles():
    w = synth.WORKLOADS[0]
    _run_e2e(w, [600], p_lo=0.05, p_hi=0.9, lengths=[600])


@pytest.mark.parametrize("bits,G,L", [(2, 1, 3001), (2, 4, 2048), (4, 8, 1500), (4, 2, 5),
                                      (2, 8, 1027), (3, 1, 2111), (3, 2, 700), (3, 4, 1500),
                                      (3, 8, 333)])
def test_decode_on_identical_contents(bits, G, L):
    """Decode attention alone: arbitrary stored contents written into the arena
    (codes, binary16 scale/zero, bfloat16 windows) are read identically by the
    GPU and by the oracle."""
    n_kv = 2
    w = synth.Workload(9, "decode-only", 1, n_kv * G, n_kv, 1, L, (bits,), 4, 64, 1, 0.01, 0.99, "bf16")
    dc = _cache(w, ctx_cap=L)
    T, Tq = synth.transforms(w, 0)
    k, v = _inputs(w, 0, 0, L)
    dc.append(0, [0], [L], k.cuda(), v.cuda(), torch.from_numpy(T).cuda())   # sets the length
    torch.cuda.synchronize()
    rng = np.random.default_rng(100 + bits + G)
    K, V = [], []
    for h in range(n_kv):
        cont = synth.random_cache_contents(rng, L, bits)
        write_unit(dc, 0, 0, h, L, cont)
        sq = dc.get_len(0, 0)[1]
        Kh = cont["k_bf16"].astype(np.float64).copy()
        Vh = cont["v_bf16"].astype(np.float64).copy()
        qp = np.arange(4, sq)
        Kh[qp] = oracle.dequantize(cont["kcodes"][qp], cont["ks16"][qp], cont["kz16"][qp])
        Vh[qp] = oracle.dequantize(cont["vcodes"][qp], cont["vs16"][qp], cont["vz16"][qp])
        K.append(Kh)
        V.append(Vh)
    torch.cuda.synchronize()
    q = synth.queries(w, 0, 0, 1)
    out = dc.decode_attn(0, [0], q.cuda(), torch.from_numpy(Tq).cuda()).cpu().numpy()
    qc = np.concatenate([oracle.compensate(T[h].astype(np.float64), q[0, h * G:(h + 1) * G].double().numpy())
                         for h in range(n_kv)])
    ref = oracle.attention(qc, np.stack(K), np.stack(V))
    check_attention(out[0], ref)


def test_decode_twice_bitwise_deterministic():
    w = synth.WORKLOADS[0]
    dc = _run_e2e(w, [1024], check_attn=False)
    _, Tq = synth.transforms(w, 0)
    q = synth.queries(w, 0, 0, 1).cuda()
    tq = torch.from_numpy(Tq).cuda()
    a = dc.decode_attn(0, [0], q, tq).clone()
    b = dc.decode_attn(0, [0], q, tq).clone()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ decode step

def _run_steps(w, L0s, n_steps, *, bits=None, S=None, R=None, F=None, check_every=1,
               rms_alpha=None, page=0):
    """Prefill L0s[i] positions per sequence with wushkv_append, then n_steps
    fused decode steps.  Each step's output is checked against the oracle's
    attention over the state before the flush (section 4.4: the new entry
    joins the bfloat16 window, flushed after the attention) -- the oracle cache
    at length L + 1 with recent + 1 -- and the final cache against the oracle
    cache at its length."""
    lengths = [L0 + n_steps for L0 in L0s]
    dc = _cache(w, bits=bits, S=S, R=R, F=F, max_batch=len(lengths), ctx_cap=max(lengths),
                rms_alpha=rms_alpha, page=page)
    c = dc.cfg
    T, Tq = synth.transforms(w, 0)
    ks, vs = zip(*[_inputs(w, 0, si, L) for si, L in enumerate(lengths)])
    slots = list(range(len(lengths)))
    tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
    if any(L0s):
        kk = torch.cat([ks[i][:L0s[i]] for i in slots]).cuda().contiguous()
        vv = torch.cat([vs[i][:L0s[i]] for i in slots]).cuda().contiguous()
        dc.append(0, slots, list(L0s), kk, vv, tk)
    for st in range(n_steps):
        pos = [L0 + st for L0 in L0s]
        k1 = torch.stack([ks[i][pos[i]] for i in slots]).cuda().contiguous()
        v1 = torch.stack([vs[i][pos[i]] for i in slots]).cuda().contiguous()
        q = synth.queries(w, 0, st, len(slots))
        out = dc.decode_step(0, slots, k1, v1, tk, q.cuda(), tq)
        if st % check_every and st != n_steps - 1:
            continue
        out = out.cpu().numpy()
        for si in slots:
            Lq = pos[si] + 1
            units = {h: oracle.cache_unit(ks[si][:Lq, h].double().numpy(),
                                          vs[si][:Lq, h].double().numpy(),
                                          T[h].astype(np.float64), S=c.sink, R=c.recent + 1,
                                          F=c.flush, bits=c.bits, p_lo=c.p_lo, p_hi=c.p_hi,
                                          alpha=_alpha_of(dc))
                     for h in range(w.n_kv)}
            check_attention(out[si], reference_attention(w, T, q[si], units))
    torch.cuda.synchronize()
    _check_state(dc, w, ks, vs, T)
    return dc


def test_decode_step_cfg0_after_prefill():
    """fp32 io, 4 query heads on 1 KV head: prefill 900, then 24 steps (one
    ring entry quantized after each attention)."""
    _run_steps(synth.WORKLOADS[0], [900], 24)


@pytest.mark.parametrize("S,R,F", [(4, 8, 1), (0, 6, 1), (4, 0, 1), (2, 5, 3), (16, 32, 16)])
def test_decode_step_from_empty(S, R, F):
    """Steps from an empty sequence through the sink, the ring filling, and the
    first flushes (batched for flush > 1; the new entry itself quantized right
    after its attention when recent = 0)."""
    _run_steps(synth.WORKLOADS[0], [0], 60, S=S, R=R, F=F)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_decode_step_gqa_ragged(bits):
    """bf16 io, 32 query / 8 KV heads, three sequences of different lengths
    (one starting empty) in each call."""
    _run_steps(synth.WORKLOADS[1], [1500, 0, 777], 5, bits=bits, check_every=2)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_decode_step_prepared_query_blocks(bits):
    """Contexts past 2K positions with little cache traffic: the launcher
    prepares each unit's query (and the step's new entry) once in the prep
    kernel and oversubscribes the split grid; parity as for the in-workgroup
    preparation."""
    _run_steps(synth.WORKLOADS[1], [2600, 0, 2301], 3, bits=bits, check_every=1)


@pytest.mark.parametrize("G", [1, 2])
def test_decode_step_one_workgroup_per_cu_fp32_paged(G):
    """Few units at G <= 2: one quantized workgroup per CU on a contiguous run
    (workgroup 0 of each unit lighter), window workgroups last; with fp32
    inputs and on a paged cache with shuffled pages."""
    _run_steps(_gqa_workload(4000, G=G, io="fp32"), [3500, 2200], 3, check_every=1)
    _run_steps(_gqa_workload(4000, G=G), [3500, 2200], 3, check_every=1, page=128)


@pytest.mark.parametrize("G", [1, 2])
def test_decode_step_one_workgroup_per_cu_short(G):
    """Short contexts in the one-workgroup-per-CU layout: a single quantized
    workgroup per unit, and runs of a sub-chunk or none."""
    _run_steps(_gqa_workload(800, G=G), [400, 130, 0], 4, check_every=1)


@pytest.mark.parametrize("G", [1, 2])
def test_decode_step_prep_kernel_many_units(G):
    """More units than half the CUs at G <= 2 (72 KV heads x 2 sequences): the
    query is prepared once per unit in the prep kernel and the grid is
    oversubscribed instead."""
    _run_steps(_gqa_workload(3000, G=G, n_kv=72), [2600, 2100], 2, check_every=1)


def test_decode_step_same_cache_as_append():
    """The cache a decode step leaves equals the one wushkv_append (n_new = 1)
    leaves, bit for bit, over steps that quantize and steps that do not."""
    w = synth.WORKLOADS[1]
    L0, n = 400, 40
    dc = _cache(w, S=4, R=16, F=4, max_batch=2, ctx_cap=L0 + n)
    T, Tq = synth.transforms(w, 0)
    k, v = _inputs(w, 0, 0, L0 + n)
    tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
    dc.append(0, [0, 1], [L0, L0], torch.cat([k[:L0], k[:L0]]).cuda(),
              torch.cat([v[:L0], v[:L0]]).cuda(), tk)
    for st in range(n):
        p = L0 + st
        k1 = k[p:p + 1].cuda().contiguous()
        v1 = v[p:p + 1].cuda().contiguous()
        q = synth.queries(w, 0, st, 1).cuda()
        dc.decode_step(0, [0], k1, v1, tk, q, tq)
        dc.append(0, [1], [1], k1, v1, tk)
        dc.decode_attn(0, [1], q, tq)
    torch.cuda.synchronize()
    L = L0 + n
    assert dc.get_len(0, 0) == dc.get_len(0, 1)
    for h in range(w.n_kv):
        a = read_unit(dc, 0, 0, h, L)
        b = read_unit(dc, 0, 1, h, L)
        sq = a["squant"]
        for key in ("kcodes", "vcodes", "ks16", "kz16", "vs16", "vz16"):
            assert np.array_equal(a[key][4:sq], b[key][4:sq]), key
        for key in ("kwin", "vwin"):
            assert np.array_equal(np.nan_to_num(a[key], nan=7.0), np.nan_to_num(b[key], nan=7.0))


# ------------------------------------------------------------------ RMS codec

@pytest.mark.parametrize("bits", [2, 4])
def test_rms_codec_fp32_path(bits):
    """The RMS (QuEST-style) codec through the rank-sort kernel (fp32 inputs):
    prefill, token appends, decode; endpoint = the Gaussian-optimal alpha."""
    w = synth.WORKLOADS[0]
    _run_e2e(w, [700, 1, 1, 300, 22], bits=bits, rms_alpha=oracle.quest_alpha(bits))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_rms_codec_prefill_kernel(bits):
    """bf16 inputs: the matrix-core prefill kernel with RMS clip ends, then
    token appends through the one-position path (both sum squares in the same
    order)."""
    w = _bf16_workload(2600, bits=bits)
    _run_e2e(w, [2000, 1, 1, 598], bits=bits, rms_alpha=oracle.quest_alpha(bits))


def test_rms_codec_decode_step():
    _run_steps(synth.WORKLOADS[0], [500], 12, rms_alpha=1.9)


# ------------------------------------------------------------------ paged cache

def test_paged_fp32_path():
    """Paged quantized planes (128-position pages, shuffled pool) through the
    rank-sort append kernel: prefill, token appends, decode attention."""
    _run_e2e(synth.WORKLOADS[0], [700, 1, 1, 300, 22], page=128)


@pytest.mark.parametrize("page,bits", [(128, 2), (256, 4), (1024, 2), (128, 3)])
def test_paged_prefill_kernel(page, bits):
    """The matrix-core prefill kernel writing paged planes: tiles that start
    mid-page, pages shared out across a ragged GQA batch."""
    w = synth.WORKLOADS[1]
    _run_e2e(w, [700, 3, 1, 1, 600, 5], bits=bits, lengths=[1310, 2, 907], page=page)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_paged_decode_steps_batched_flush(bits):
    """Fused decode steps on a paged cache with the paper's evaluation windows
    (sink 16, recent 128, flush 16): pages mapped as the quantized region
    grows, 16 ring entries quantized every 16th step."""
    _run_steps(synth.WORKLOADS[1], [1500, 0, 777], 40, bits=bits, S=16, R=128, F=16,
               check_every=8, page=128)


def test_paged_equals_contiguous():
    """A paged cache and a contiguous one fed the same inputs store the same
    codes, scale/zero and windows and produce bit-identical attention."""
    w = synth.WORKLOADS[1]
    lengths = [1310, 2, 907]
    slots = list(range(3))
    T, Tq = synth.transforms(w, 0)
    tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
    ks, vs = zip(*[_inputs(w, 0, si, L + 20) for si, L in enumerate(lengths)])
    outs = []
    caches = []
    for page in (0, 128):
        dc = _cache(w, max_batch=3, ctx_cap=max(lengths) + 20, page=page)
        kk = torch.cat([ks[i][:lengths[i]] for i in slots]).cuda().contiguous()
        vv = torch.cat([vs[i][:lengths[i]] for i in slots]).cuda().contiguous()
        dc.append(0, slots, lengths, kk, vv, tk)
        o = []
        for st in range(20):
            k1 = torch.stack([ks[i][lengths[i] + st] for i in slots]).cuda().contiguous()
            v1 = torch.stack([vs[i][lengths[i] + st] for i in slots]).cuda().contiguous()
            q = synth.queries(w, 0, st, 3).cuda()
            o.append(dc.decode_step(0, slots, k1, v1, tk, q, tq).cpu())
        outs.append(torch.stack(o))
        caches.append(dc)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    for si, L in enumerate(lengths):
        for h in range(w.n_kv):
            a = read_unit(caches[0], 0, si, h, L + 20)
            b = read_unit(caches[1], 0, si, h, L + 20)
            sq = a["squant"]
            for key in ("kcodes", "vcodes", "ks16", "kz16", "vs16", "vz16"):
                assert np.array_equal(a[key][4:sq], b[key][4:sq]), key
            for key in ("kwin", "vwin"):
                assert np.array_equal(np.nan_to_num(a[key], nan=7.0), np.nan_to_num(b[key], nan=7.0))


def test_paged_pages_reused_after_reset():
    """Pages returned by a finished sequence are handed to a new one: its
    results depend only on its own entries (stale codes in reused pages are
    overwritten before they are read)."""
    w = _bf16_workload(1800)
    dc = _cache(w, max_batch=2, ctx_cap=1800, page=128)
    T, Tq = synth.transforms(w, 0)
    tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
    k, v = _inputs(w, 0, 0, 1800)
    dc.append(0, [0], [1800], k.cuda(), v.cuda(), tk)
    used = dc.pages_in_use()
    dc.reset_seq(0)
    assert dc.pages_in_use() == 0
    k2, v2 = synth.keys_values(w, 0, 1, 0, 1500)
    dc.append(0, [1], [1200], k2[:1200].contiguous().cuda(), v2[:1200].contiguous().cuda(), tk)
    dc.append(0, [1], [300], k2[1200:].contiguous().cuda(), v2[1200:].contiguous().cuda(), tk)
    assert 0 < dc.pages_in_use() <= used
    q = synth.queries(w, 0, 0, 1)
    out = dc.decode_attn(0, [1], q.cuda(), tq).cpu().numpy()
    torch.cuda.synchronize()
    units = {}
    for h in range(w.n_kv):
        orc = oracle.cache_unit(k2[:, h].double().numpy(), v2[:, h].double().numpy(),
                                T[h].astype(np.float64), S=w.sink, R=w.recent, F=w.flush,
                                bits=2, p_lo=w.p_lo, p_hi=w.p_hi)
        gpu = read_unit(dc, 0, 1, h, 1500)
        check_windows(gpu, orc)
        check_codes(gpu, orc, 2)
        units[h] = orc
    check_attention(out[0], reference_attention(w, T, q[0], units))


# ------------------------------------------------------------------ 3-bit cache

def test_3bit_window_variants_fp32_path():
    """3-bit codes (two bit planes) through the rank-sort kernel with flush
    batches: prefill, one-token appends, decode attention."""
    w = synth.WORKLOADS[0]
    _run_e2e(w, [513, 1, 1, 70, 1, 414], bits=3, S=16, R=128, F=16, lengths=[1000])


def test_3bit_prefill_tiles_mid_block():
    """bf16 prefill at 3 bits: appends that start and end inside 128-position
    blocks, so tiles write one half of a block's high-plane row each, across
    separate calls and workgroups."""
    w = _bf16_workload(3100, bits=3)
    _run_e2e(w, [37, 1050, 1, 64, 1000, 3, 945], bits=3)


# ------------------------------------------------------------------ chunked steps

def _run_chunks(w, L0s, plan, *, bits=None, S=None, R=None, F=None, page=0, check_every=1):
    """Prefill L0s[i] positions per sequence, then one wushkv_chunk_step per
    entry of plan (a list of per-sequence chunk sizes).  Each new position's
    output is checked against the oracle's causal attention over the cache of
    section 4.4 at that moment: the quantized boundary of the length before
    the chunk (the oracle cache with recent + chunk at the chunk's end), the
    chunk's entries in bfloat16, positions up to the query's own.  The final
    cache is checked against the oracle cache at its length."""
    lengths = [L0 + sum(step[i] for step in plan) for i, L0 in enumerate(L0s)]
    dc = _cache(w, bits=bits, S=S, R=R, F=F, max_batch=len(lengths), ctx_cap=max(lengths), page=page)
    c = dc.cfg
    T, Tq = synth.transforms(w, 0)
    ks, vs = zip(*[_inputs(w, 0, si, L) for si, L in enumerate(lengths)])
    slots = list(range(len(lengths)))
    tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
    if any(L0s):
        kk = torch.cat([ks[i][:L0s[i]] for i in slots]).cuda().contiguous()
        vv = torch.cat([vs[i][:L0s[i]] for i in slots]).cuda().contiguous()
        dc.append(0, slots, list(L0s), kk, vv, tk)
    pos = list(L0s)
    G = w.group
    for st, nn in enumerate(plan):
        kk = torch.cat([ks[i][pos[i]:pos[i] + nn[i]] for i in slots]).cuda().contiguous()
        vv = torch.cat([vs[i][pos[i]:pos[i] + nn[i]] for i in slots]).cuda().contiguous()
        q = synth.queries(w, 0, st, sum(nn))
        out = dc.chunk_step(0, slots, nn, kk, vv, tk, q.cuda(), tq)
        if st % check_every == 0 or st == len(plan) - 1:
            out = out.cpu().numpy()
            tok = 0
            for si in slots:
                L, n = pos[si], nn[si]
                KV = []
                for h in range(w.n_kv):
                    unit = oracle.cache_unit(ks[si][:L + n, h].double().numpy(),
                                             vs[si][:L + n, h].double().numpy(),
                                             T[h].astype(np.float64), S=c.sink, R=c.recent + n,
                                             F=c.flush, bits=c.bits, p_lo=c.p_lo, p_hi=c.p_hi)
                    KV.append(oracle.readback(unit))
                for cc in range(n):
                    qc = np.concatenate([oracle.compensate(T[h].astype(np.float64),
                                                           q[tok + cc, h * G:(h + 1) * G].double().numpy())
                                         for h in range(w.n_kv)])
                    K = np.stack([KV[h][0][:L + cc + 1] for h in range(w.n_kv)])
                    V = np.stack([KV[h][1][:L + cc + 1] for h in range(w.n_kv)])
                    check_attention(out[tok + cc], oracle.attention(qc, K, V))
                tok += n
        pos = [p + n for p, n in zip(pos, nn)]
    torch.cuda.synchronize()
    _check_state(dc, w, ks, vs, T)
    return dc


def _gqa_workload(L, *, G, n_kv=2, io="bf16"):
    return synth.Workload(12, "chunk", 1, n_kv * G, n_kv, 1, L, (2,), 4, 128, 1, 0.01, 0.99, io)


@pytest.mark.parametrize("bits", [2, 3])
def test_chunk_step_new_entries_leave_at_once(bits):
    """A recent window smaller than the chunk (S 4, R 4, F 2): ring entries
    leave the window in the prep launch, and most of each chunk's own entries
    are quantized in the same step by the flush launch after the prep."""
    _run_chunks(synth.WORKLOADS[1], [300, 40], [[16, 16], [16, 9], [5, 16], [1, 2]], S=4, R=4, F=2,
                bits=bits)


def test_chunk_step_fp32_inputs():
    """fp32 inputs, 4 query heads on 1 KV head: prefill 700, then 16-position
    chunks and a short one (every chunk crosses quantized flushes)."""
    _run_chunks(synth.WORKLOADS[0], [700], [[16]] * 5 + [[7], [1], [16]])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_chunk_step_gqa_ragged(bits):
    """32 query / 8 KV heads, three sequences (one starting empty) with ragged
    chunk sizes in each call, at every bit width (3 bits: low and high planes
    unpacked into one operand byte; 4 bits: two code words per 16 elements)."""
    _run_chunks(synth.WORKLOADS[1], [1500, 0, 777], [[16, 5, 16], [3, 16, 1], [16, 16, 16], [1, 2, 9]],
                bits=bits)


@pytest.mark.parametrize("G,bits", [(1, 2), (2, 2), (8, 2), (8, 4), (1, 3), (8, 3)])
def test_chunk_step_groups(G, bits):
    """Row tiles of 16 query rows: 16 positions x G heads (one tile at G = 1,
    eight at G = 8)."""
    _run_chunks(_gqa_workload(3000, G=G), [2100, 1333], [[16, 16], [16, 11], [4, 16]], bits=bits)


@pytest.mark.parametrize("G,plan,bits", [(1, [[8, 3], [5, 8], [1, 1]], 2), (2, [[4, 4], [3, 1]], 2),
                                         (4, [[2, 1], [2, 2]], 2), (2, [[4, 4], [3, 1]], 4),
                                         (4, [[2, 1], [2, 2]], 3)])
def test_chunk_step_paired_rows(G, plan, bits):
    """Chunks of at most 8 query rows per KV head (n_new G <= 8).  At 2 bits
    the second half of the row tile repeats the queries against the other
    column blocks of each sub-chunk and the halves merge per row; at 3 and 4
    bits the same small tiles run unpaired."""
    _run_chunks(_gqa_workload(3000, G=G), [2100, 1333], plan, bits=bits)


def test_chunk_step_paper_windows_from_empty():
    """The paper's evaluation windows (sink 16, recent 128, flush 16) from
    empty sequences in 16-position chunks: the sink fills inside a chunk, the
    ring fills, flushes of 16 follow."""
    _run_chunks(synth.WORKLOADS[1], [0, 0], [[16, 16]] * 14 + [[5, 16]], S=16, R=128, F=16,
                check_every=3)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_chunk_step_paged(bits):
    _run_chunks(synth.WORKLOADS[1], [1100, 300], [[16, 16], [16, 3], [9, 16]], page=128, bits=bits)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_chunk_step_same_cache_as_append(bits):
    """The cache a chunk step leaves equals the one wushkv_append of the same
    positions leaves, bit for bit (3 bits: the flush's word atomics on both
    value planes)."""
    w = synth.WORKLOADS[1]
    L0, steps = 600, [16, 16, 7, 16, 1, 16]
    n = sum(steps)
    dc = _cache(w, bits=bits, S=4, R=32, F=4, max_batch=2, ctx_cap=L0 + n)
    T, Tq = synth.transforms(w, 0)
    k, v = _inputs(w, 0, 0, L0 + n)
    tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
    dc.append(0, [0, 1], [L0, L0], torch.cat([k[:L0], k[:L0]]).cuda(), torch.cat([v[:L0], v[:L0]]).cuda(), tk)
    p = L0
    for st, m in enumerate(steps):
        kk = k[p:p + m].cuda().contiguous()
        vv = v[p:p + m].cuda().contiguous()
        dc.chunk_step(0, [0], [m], kk, vv, tk, synth.queries(w, 0, st, m).cuda(), tq)
        dc.append(0, [1], [m], kk, vv, tk)
        p += m
    torch.cuda.synchronize()
    L = L0 + n
    assert dc.get_len(0, 0) == dc.get_len(0, 1)
    for h in range(w.n_kv):
        a = read_unit(dc, 0, 0, h, L)
        b = read_unit(dc, 0, 1, h, L)
        sq = a["squant"]
        for key in ("kcodes", "vcodes", "ks16", "kz16", "vs16", "vz16"):
            assert np.array_equal(a[key][4:sq], b[key][4:sq]), key
        for key in ("kwin", "vwin"):
            assert np.array_equal(np.nan_to_num(a[key], nan=7.0), np.nan_to_num(b[key], nan=7.0))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_decode_step_group8(bits):
    """Groups of 8 query heads: wushkv_decode_step on the split kernel's int8
    matrix-core path (two four-head tiles sharing one value product); steps
    from a prefill and from an empty sequence, with flush batches."""
    w = _gqa_workload(2000, G=8)
    _run_steps(w, [1500, 0], 20, bits=bits, S=4, R=32, F=4, check_every=4)


def test_chunk_step_rms_codec():
    """The RMS codec through chunk steps: the flush kernel quantizes with the
    Gaussian-optimal endpoint, leaving the oracle's RMS-codec cache."""
    w = _bf16_workload(1200)
    lengths = [1200 + 16 * 3]
    alpha = oracle.quest_alpha(2)
    dc = _cache(w, max_batch=1, ctx_cap=lengths[0], rms_alpha=alpha)
    T, Tq = synth.transforms(w, 0)
    k, v = _inputs(w, 0, 0, lengths[0])
    tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
    dc.append(0, [0], [1200], k[:1200].cuda().contiguous(), v[:1200].cuda().contiguous(), tk)
    for st in range(3):
        p = 1200 + 16 * st
        dc.chunk_step(0, [0], [16], k[p:p + 16].cuda().contiguous(), v[p:p + 16].cuda().contiguous(),
                      tk, synth.queries(w, 0, st, 16).cuda(), tq)
    torch.cuda.synchronize()
    for h in range(w.n_kv):
        orc = oracle.cache_unit(k[:, h].double().numpy(), v[:, h].double().numpy(), T[h].astype(np.float64),
                                S=w.sink, R=w.recent, F=w.flush, bits=2, p_lo=w.p_lo, p_hi=w.p_hi,
                                alpha=alpha)
        gpu = read_unit(dc, 0, 0, h, lengths[0])
        check_windows(gpu, orc)
        check_codes(gpu, orc, 2)
