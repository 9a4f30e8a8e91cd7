#!/usr/bin/env python3
"""Decode-step benchmark of the WUSH-KV 2-bit transformed KV cache on one MI355X.

A step is one pass of the whole hot path over one batch: for every layer, one
wushkv_decode_step call per batch (key transform of the new position, query
compensation, split-K scan over the packed codes and the bfloat16 windows with
the new entry included, then the flush of the ring entry that leaves the
window: percentile clip, quantize, pack -- and the log-sum-exp merge).  With
--path append+attn the same step runs as wushkv_append followed by
wushkv_decode_attn (three launches per layer instead of two; the flush then
precedes the attention).  The cache is built beforehand through the same
library (prefill appends) from seeded synthetic inputs and is resident in HBM
when the timed region starts.

Default workload: 32 layers x 32 KV heads x head_dim 128 (MHA, 32 query heads),
batch 1, context 131072, 2-bit, sink 4, recent 128 -- the cache whose 2-bit
footprint is ~8 GiB of codes (+1 GiB of fp16 scale/zero).

Prints one JSON line.  value = cache bytes the attention reads (algorithmic:
72 B per quantized token-head, 512 B per bfloat16 window token-head) per second
of whole-step time (appends included).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def squant(L, S, R, F):
    return S + F * (max(0, L - R - S) // F)


def unit_bytes(L, S, R, F, bits, step=True):
    """Algorithmic bytes the attention reads for one (sequence, KV head) at
    length L (new position included).  A fused step attends before the flush:
    its quantized boundary is that of length L - 1."""
    sq = squant(L - 1 if step else L, S, R, F)
    quant = max(0, sq - S)
    window = min(S, L) + max(0, L - sq)
    return quant * (2 * (128 * bits // 8) + 8) + window * 512


def cpu_baseline(w, bits, seconds, max_units):
    """The CPU reference's decode attention (dequantize + naive softmax attention,
    fp64, one thread) on a bounded sample of (layer, KV head) units of the same
    workload, with arbitrary stored contents of the same shape."""
    import numpy as np

    import oracle
    from decode_attention_wushkv_amd import synth

    rng = np.random.default_rng(12345)
    L = max(w.lengths())
    S, R, F = w.sink, w.recent, w.flush
    sq = squant(L, S, R, F)
    done, elapsed = 0, 0.0
    while done < max_units and elapsed < seconds:
        cont = synth.random_cache_contents(rng, L, bits)
        q = rng.standard_normal((w.group, 128))
        t0 = time.perf_counter()
        K = cont["k_bf16"].astype(np.float64)
        V = cont["v_bf16"].astype(np.float64)
        qp = slice(S, sq)
        K[qp] = oracle.dequantize(cont["kcodes"][qp], cont["ks16"][qp], cont["kz16"][qp])
        V[qp] = oracle.dequantize(cont["vcodes"][qp], cont["vs16"][qp], cont["vz16"][qp])
        oracle.attention(q, K[None], V[None])
        elapsed += time.perf_counter() - t0
        done += 1
    gbs = done * unit_bytes(L, S, R, F, bits, step=False) / elapsed / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (layer, KV head) units of {w.group} query head(s) at context {L}, "
                      f"dequantize + fp64 softmax attention, {elapsed:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=3, help="workload id in synth.WORKLOADS")
    ap.add_argument("--bits", type=int, default=None)
    ap.add_argument("--path", choices=("step", "append+attn"), default="step",
                    help="fused wushkv_decode_step, or wushkv_append then wushkv_decode_attn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device-to-device copy of this size first (hardware-counter "
                         "calibration: bytes fetched/written by a copy of known size)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path is a per-GPU "
                                   "kernel (head or context sharding across GPUs is not built)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import decode_attention_wushkv_amd as wk
    from decode_attention_wushkv_amd import synth
    from decode_attention_wushkv_amd.device_cache import DeviceCache

    wk.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    bits = args.bits or w.bits[0]
    K, W = args.steps, args.warmup
    targets = w.lengths()
    B = len(targets)
    L0 = [t - (W + 2 * K) for t in targets]
    S, R, F = w.sink, w.recent, w.flush
    slots = list(range(B))

    dc = DeviceCache(n_layers=w.n_layers, n_q_heads=w.n_q, n_kv_heads=w.n_kv, bits=bits, sink=S,
                     recent=R, flush=F, p_lo=w.p_lo, p_hi=w.p_hi, max_batch=B,
                     ctx_cap=max(targets), io_dtype=w.torch_io, device=dev)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- build the cache through the library (prefill appends), layer by layer
    t_build = time.perf_counter()
    tks, tqs = [], []
    for layer in range(w.n_layers):
        T, Tq = synth.transforms(w, layer)
        tks.append(torch.from_numpy(T).to(dev))
        tqs.append(torch.from_numpy(Tq).to(dev))
        scales = synth.channel_scales(w, layer)
        parts_k, parts_v = [], []
        for s in range(B):
            k, v = synth.keys_values(w, layer, s, 0, L0[s], device=dev, scales=scales)
            parts_k.append(k)
            parts_v.append(v)
        kk = torch.cat(parts_k) if B > 1 else parts_k[0]
        vv = torch.cat(parts_v) if B > 1 else parts_v[0]
        del parts_k, parts_v
        dc.append(layer, slots, L0, kk, vv, tks[layer])
        del kk, vv
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t_build
    print(f"[bench] cache built: {w.name}, {bits}-bit, {dc.layout.total_bytes / 2**30:.2f} GiB arena, "
          f"{build_s:.1f} s", file=sys.stderr, flush=True)

    # ---- per-step inputs, resident before timing
    layer_scales = [synth.channel_scales(w, layer) for layer in range(w.n_layers)]
    steps_in = []
    for st in range(W + 2 * K):
        per_layer = []
        for layer in range(w.n_layers):
            scales = layer_scales[layer]
            ks, vs = [], []
            for s in range(B):
                k, v = synth.keys_values(w, layer, s, L0[s] + st, 1, device=dev, scales=scales)
                ks.append(k)
                vs.append(v)
            q = synth.queries(w, layer, st, B, device=dev)
            per_layer.append((torch.cat(ks).contiguous(), torch.cat(vs).contiguous(), q))
        steps_in.append(per_layer)
    out = torch.empty((B, w.n_q, 128), dtype=torch.float32, device=dev)
    dc.workspace(B)
    stream = torch.cuda.current_stream(dev)

    fused = args.path == "step"

    def layer_call(st, layer):
        k1, v1, q = steps_in[st][layer]
        if fused:
            dc.decode_step(layer, slots, k1, v1, tks[layer], q, tqs[layer], out)
        else:
            dc.append(layer, slots, [1] * B, k1, v1, tks[layer])
            dc.decode_attn(layer, slots, q, tqs[layer], out)

    # HIP events bracketing every split launch of pass B, created and recorded
    # once beforehand so that the timed loop only records them
    ev_pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(K * w.n_layers)]
    for e0, e1 in ev_pairs:
        e0.record(stream)
        e1.record(stream)
    torch.cuda.synchronize()

    for st in range(W):
        for layer in range(w.n_layers):
            layer_call(st, layer)

    def timed_pass(first, instrument):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        i = 0
        for st in range(first, first + K):
            for layer in range(w.n_layers):
                if instrument:
                    e0, e1 = ev_pairs[i]
                    i += 1
                    wk.wushkv_set_split_events(dc.handle, e0.cuda_event, e1.cuda_event)
                layer_call(st, layer)
                if instrument:
                    wk.wushkv_set_split_events(dc.handle, None, None)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    # pass A: the step metric, no instrumentation in the stream
    total_ms = timed_pass(W, False)
    ms_per_step = total_ms / K
    # pass B: the same steps continued, split kernel bracketed by HIP events
    total_b_ms = timed_pass(W + K, True)
    split_ms = [a.elapsed_time(b) for a, b in ev_pairs]

    # algorithmic bytes of the attention reads over the timed steps of pass A
    bytes_total = 0
    for st in range(W, W + K):
        for s in range(B):
            Lnow = L0[s] + st + 1
            bytes_total += w.n_layers * w.n_kv * unit_bytes(Lnow, S, R, F, bits, fused)
    bytes_per_step = bytes_total / K
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    # per split launch of pass B (the same sequences, K positions longer)
    bytes_b = 0
    for st in range(W + K, W + 2 * K):
        for s in range(B):
            bytes_b += w.n_layers * w.n_kv * unit_bytes(L0[s] + st + 1, S, R, F, bits, fused)
    bytes_per_launch = bytes_b / (K * w.n_layers)
    split_avg_ms = float(np.mean(split_ms))
    achieved = bytes_per_launch / (split_avg_ms * 1e-3) / 1e9
    append_tok_s = B * w.n_layers * K / (total_ms * 1e-3)

    res = {
        "metric": "2-bit KV decode attn: cache GB/s & % HBM peak; append tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "n_layers": w.n_layers, "n_q_heads": w.n_q,
                   "n_kv_heads": w.n_kv, "head_dim": 128, "batch": B,
                   "context": targets if B > 1 and len(set(targets)) > 1 else targets[0],
                   "bits": bits, "sink": S, "recent": R, "flush": F,
                   "p_lo": w.p_lo, "p_hi": w.p_hi, "io": w.io},
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "path": args.path,
        "append": {"tokens_per_s": round(append_tok_s, 1),
                   "note": "one-token appends per (sequence, layer) inside the timed steps"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "split_kernel (split-K scan over codes + windows"
                               + (", fused one-token append)" if fused else ")"),
                     "bytes_per_launch": int(bytes_per_launch),
                     "avg_launch_ms": round(split_avg_ms, 5), "launches": len(split_ms),
                     "timing": "HIP events around every split launch of a second timed pass of "
                               f"{K} steps ({round(total_b_ms / K, 4)} ms/step with the events)"},
        "cache_build_s": round(build_s, 2),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, bits, args.cpu_seconds, max_units=400)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
