"""Parity at the full sizes of the three large workloads, on sampled units, in
the launch configuration the benchmark times:

  * qwen3-8b-36L-b32-ragged4k-16k  36 layers, 32 sequences of lengths
    U[4096, 16384], 32 query / 8 KV heads, 2-bit: 64 units over two layers;
  * mha-32L-32kv-128k              32 layers x 32 KV heads, 131072 positions:
    every KV head of two layers at 2 bits (64 units), every KV head of the
    last layer at 3 and 4 bits;
  * qwen3-32b-64L-b8-prefill64k    64 layers, 8 sequences x 65536 prefill
    positions, 64 query / 8 KV heads: every unit of the last layer (64) at 2
    and 4 bits.

Each test allocates the whole cache (every layer, full batch and capacity) and
fills the sampled layers through the library: one prefill wushkv_append of all
sequences at their full lengths (inputs drawn on the device by the seeded
generator), then one fused wushkv_decode_step.  Sampled (layer, sequence, KV
head) units are then checked completely against the oracle: every window
entry, every code and binary16 scale/zero after the step (the state at L + 1,
flushed entry included), and the attention output of the unit's G query heads
against the oracle's attention over its own cache before the flush (section
4.4 of the paper page: the new entry is attended in full precision).  Layers
that are not sampled stay empty: each layer is an independent launch of the
same geometry, and the last layer, the one at the largest arena offsets, is
always sampled.  The oracle units run on a pool of host threads (its C calls
release the interpreter lock).
"""
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from decode_attention_wushkv_amd import synth
from decode_attention_wushkv_amd.device_cache import DeviceCache

from cachepack import read_unit
from gpu_checks import check_attention, check_codes, check_windows

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_wushkv_amd import build
    if build.is_stale():
        build.build()
    torch.cuda.set_device(0)


def _run(wid, bits, layers, units_per_layer, seed):
    w = synth.WORKLOADS[wid]
    lengths = w.lengths()
    B = len(lengths)
    slots = list(range(B))
    dc = DeviceCache(n_layers=w.n_layers, n_q_heads=w.n_q, n_kv_heads=w.n_kv, bits=bits,
                     sink=w.sink, recent=w.recent, flush=w.flush, p_lo=w.p_lo, p_hi=w.p_hi,
                     max_batch=B, ctx_cap=max(lengths) + 1, io_dtype=w.torch_io, device="cuda")
    rng = np.random.default_rng(seed)
    G, S, R, F = w.group, w.sink, w.recent, w.flush
    readback_lock = threading.Lock()
    total = 0
    for layer in layers:
        all_units = [(si, h) for si in slots for h in range(w.n_kv)]
        if units_per_layer >= len(all_units):
            sample = all_units
        else:
            pick = rng.choice(len(all_units), size=units_per_layer, replace=False)
            sample = [all_units[i] for i in sorted(pick)]
        seqs = sorted({si for si, _ in sample})
        print(f"[full] {w.name} {bits}-bit layer {layer}: {len(sample)} units over "
              f"{len(seqs)} sequences", flush=True)
        T, Tq = synth.transforms(w, layer)
        tk, tq = torch.from_numpy(T).cuda(), torch.from_numpy(Tq).cuda()
        scales = synth.channel_scales(w, layer)
        host = {}
        parts_k, parts_v = [], []
        for si in slots:
            k, v = synth.keys_values(w, layer, si, 0, lengths[si], device="cuda", scales=scales)
            if si in seqs:
                k1, v1 = synth.keys_values(w, layer, si, lengths[si], 1, device="cuda",
                                           scales=scales)
                host[si] = (torch.cat([k, k1]).cpu(), torch.cat([v, v1]).cpu())
            parts_k.append(k)
            parts_v.append(v)
        kk, vv = torch.cat(parts_k), torch.cat(parts_v)
        del parts_k, parts_v
        dc.append(layer, slots, lengths, kk, vv, tk)
        del kk, vv
        new = [synth.keys_values(w, layer, si, lengths[si], 1, device="cuda", scales=scales)
               for si in slots]
        k1 = torch.cat([x[0] for x in new]).contiguous()
        v1 = torch.cat([x[1] for x in new]).contiguous()
        q = synth.queries(w, layer, 0, B, device="cuda")
        out = dc.decode_step(layer, slots, k1, v1, tk, q, tq).cpu().numpy()
        torch.cuda.synchronize()
        qh = q.double().cpu().numpy()

        def check_unit(unit):
            si, h = unit
            keys = host[si][0][:, h].double().numpy()
            values = host[si][1][:, h].double().numpy()
            L1 = lengths[si] + 1
            assert dc.get_len(layer, si)[0] == L1
            # cache after the step: the oracle state at L + 1
            orc = oracle.cache_unit(keys, values, T[h].astype(np.float64), S=S, R=R, F=F,
                                    bits=bits, p_lo=w.p_lo, p_hi=w.p_hi)
            with readback_lock:
                gpu = read_unit(dc, layer, si, h, L1)
            check_windows(gpu, orc)
            check_codes(gpu, orc, bits)
            # attention before the flush: boundary squant(L), new entry in bf16
            sq0 = oracle.squant(L1 - 1, S, R, F)
            K = orc["k_bf16"].copy()
            V = orc["v_bf16"].copy()
            qp = np.arange(S, sq0)
            K[qp] = oracle.dequantize(orc["kcodes"][qp], orc["ks16"][qp], orc["kz16"][qp])
            V[qp] = oracle.dequantize(orc["vcodes"][qp], orc["vs16"][qp], orc["vz16"][qp])
            qc = oracle.compensate(T[h].astype(np.float64), qh[si, h * G:(h + 1) * G])
            ref = oracle.attention(qc, K[None], V[None])
            check_attention(out[si, h * G:(h + 1) * G], ref)
            return unit

        with ThreadPoolExecutor(max_workers=THREADS) as ex:
            for _ in ex.map(check_unit, sample):
                pass
        total += len(sample)
        del host
    print(f"[full] {w.name} {bits}-bit: {total} units checked", flush=True)
    del dc
    torch.cuda.empty_cache()
    return total


def test_full_ragged_batch_36_layers():
    """Ragged batch of 32 at 4K-16K: 32 sampled units in each of two layers."""
    w = synth.WORKLOADS[2]
    assert _run(2, 2, [5, w.n_layers - 1], 32, seed=21) >= 64


def test_full_mha_128k():
    """32 KV heads at 131072 positions: every unit of the first and the last
    layer."""
    w = synth.WORKLOADS[3]
    assert _run(3, 2, [0, w.n_layers - 1], w.n_kv, seed=31) >= 64


@pytest.mark.parametrize("bits", [3, 4])
def test_full_mha_128k_wider_codes(bits):
    """The 128K MHA workload at 3 and 4 bits (64-position sub-chunks, one
    quantized workgroup per CU): every unit of the last layer."""
    w = synth.WORKLOADS[3]
    assert _run(3, bits, [w.n_layers - 1], w.n_kv, seed=33 + bits) == w.n_kv


@pytest.mark.parametrize("bits", [2, 4])
def test_full_prefill_64k(bits):
    """8 sequences x 65536 prefill positions, G = 8: every unit of the last
    layer (one full layer, 64 units)."""
    w = synth.WORKLOADS[4]
    assert _run(4, bits, [w.n_layers - 1], w.batch * w.n_kv, seed=41 + bits) == 64
