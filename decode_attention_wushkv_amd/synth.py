"""Seeded synthetic workloads for the WUSH-KV cache path.

This module only draws inputs: post-RoPE keys, values (already in the value
transform's basis), decode queries, the per-KV-head key transform T_K and its
inverse transpose.  It holds none of the method's arithmetic and is the only
module that both the GPU path's tests/benchmark and the CPU reference read.

Workload shapes follow the five configurations of the benchmark plan; the
distributions stand in for calibrated Qwen3/Llama caches, which are not
available here:

* K: per (layer, KV head) channel scales sigma_c ~ LogNormal(0, 1), 4 channels
  chosen uniformly get sigma x 10 (single-coordinate key spikes), entries
  N(0, 1) * sigma_c, then RoPE (theta = 10000, rotate-half pairing (c, c+64),
  inv_freq_i = theta^(-2i/d)) at the token's position.
* V: N(0, 1) * sigma_c with sigma_c ~ LogNormal(0, 0.5).
* Q: N(0, 1).
* T_K = Q diag(delta), Q from the QR factorisation of a Gaussian matrix with
  diag(R) > 0, delta ~ LogNormal(0, 0.3); T_K^{-T} = Q diag(1 / delta) in fp64,
  both handed over as float32.
* bf16 inputs are float32 draws rounded to bfloat16 by torch.
* Seeds: seed = 1000 + config id; per tensor numpy.random.SeedSequence
  ([seed, layer, head/seq, tag]) on the CPU, torch.Generator seeded from the
  same tuple for device-side draws.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np
import torch

D = 128
THETA = 10000.0

TAG_T, TAG_KSCALE, TAG_VSCALE, TAG_K, TAG_V, TAG_Q, TAG_LEN, TAG_CACHE = range(1, 9)


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    n_layers: int
    n_q: int
    n_kv: int
    batch: int
    ctx: int | tuple           # int, or (lo, hi) inclusive for ragged batches
    bits: tuple
    sink: int
    recent: int
    flush: int
    p_lo: float
    p_hi: float
    io: str                    # "fp32" or "bf16"

    @property
    def seed(self) -> int:
        return 1000 + self.cid

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv

    @property
    def torch_io(self):
        return torch.float32 if self.io == "fp32" else torch.bfloat16

    def lengths(self) -> list:
        if isinstance(self.ctx, tuple):
            rng = np.random.default_rng(np.random.SeedSequence([self.seed, 0, 0, TAG_LEN]))
            return [int(x) for x in rng.integers(self.ctx[0], self.ctx[1], size=self.batch,
                                                 endpoint=True)]
        return [int(self.ctx)] * self.batch


WORKLOADS = {
    0: Workload(0, "tiny-1kv-gqa4-1k", 1, 4, 1, 1, 1024, (2,), 4, 32, 1, 0.01, 0.99, "fp32"),
    1: Workload(1, "llama3-8b-layer-32k", 1, 32, 8, 1, 32768, (2,), 4, 128, 1, 0.01, 0.99, "bf16"),
    2: Workload(2, "qwen3-8b-36L-b32-ragged4k-16k", 36, 32, 8, 32, (4096, 16384), (2,), 4, 128, 1,
                0.01, 0.99, "bf16"),
    3: Workload(3, "mha-32L-32kv-128k", 32, 32, 32, 1, 131072, (2,), 4, 128, 1, 0.01, 0.99, "bf16"),
    4: Workload(4, "qwen3-32b-64L-b8-prefill64k", 64, 64, 8, 8, 65536, (2, 4), 4, 128, 1,
                0.01, 0.99, "bf16"),
}


def _ss(*key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def _torch_seed(*key) -> int:
    h = hashlib.sha256(repr(tuple(int(k) for k in key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(*key))
    return g


def transforms(w: Workload, layer: int):
    """(T_K, T_K^{-T}) per KV head, float32 numpy arrays [n_kv, d, d], row-major
    so that k'_i = sum_j T[i, j] k_j."""
    T = np.empty((w.n_kv, D, D), dtype=np.float32)
    Tq = np.empty((w.n_kv, D, D), dtype=np.float32)
    for h in range(w.n_kv):
        rng = _ss(w.seed, layer, h, TAG_T)
        a = rng.standard_normal((D, D))
        qm, rm = np.linalg.qr(a)
        qm = qm * np.sign(np.diag(rm))[None, :]
        delta = rng.lognormal(0.0, 0.3, size=D)
        T[h] = (qm * delta[None, :]).astype(np.float32)
        Tq[h] = (qm / delta[None, :]).astype(np.float32)
    return T, Tq


def channel_scales(w: Workload, layer: int):
    """Per (KV head, channel) standard deviations of K (with 4 outlier channels
    x10) and V.  float64 numpy [n_kv, d] each."""
    sk = np.empty((w.n_kv, D))
    sv = np.empty((w.n_kv, D))
    for h in range(w.n_kv):
        rng = _ss(w.seed, layer, h, TAG_KSCALE)
        s = rng.lognormal(0.0, 1.0, size=D)
        spikes = rng.choice(D, size=4, replace=False)
        s[spikes] *= 10.0
        sk[h] = s
        sv[h] = _ss(w.seed, layer, h, TAG_VSCALE).lognormal(0.0, 0.5, size=D)
    return sk, sv


def rope(x: torch.Tensor, positions: torch.Tensor) -> torch.Tensor:
    """Rotate-half RoPE, theta = 10000, on the last dim.  x: [n, ..., d] fp32/64,
    positions: [n]."""
    half = x.shape[-1] // 2
    inv = THETA ** (-torch.arange(half, dtype=torch.float64, device=x.device) * 2.0 / x.shape[-1])
    ang = positions.to(torch.float64)[:, None] * inv[None, :]
    shape = [x.shape[0]] + [1] * (x.dim() - 2) + [half]
    cos = torch.cos(ang).reshape(shape).to(x.dtype)
    sin = torch.sin(ang).reshape(shape).to(x.dtype)
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


def keys_values(w: Workload, layer: int, seq: int, start: int, count: int,
                device="cpu", scales=None):
    """Post-RoPE keys and values for positions [start, start + count) of one
    sequence: torch tensors [count, n_kv, d] in the workload's io dtype."""
    sk, sv = scales if scales is not None else channel_scales(w, layer)
    gk = _gen(device, w.seed, layer, seq, start, TAG_K)
    gv = _gen(device, w.seed, layer, seq, start, TAG_V)
    k = torch.randn((count, w.n_kv, D), generator=gk, device=device, dtype=torch.float32)
    v = torch.randn((count, w.n_kv, D), generator=gv, device=device, dtype=torch.float32)
    k = k * torch.as_tensor(sk, dtype=torch.float32, device=device)[None]
    v = v * torch.as_tensor(sv, dtype=torch.float32, device=device)[None]
    pos = torch.arange(start, start + count, device=device)
    k = rope(k, pos)
    return k.to(w.torch_io).contiguous(), v.to(w.torch_io).contiguous()


def queries(w: Workload, layer: int, step: int, n_seq: int, device="cpu"):
    """Decode queries [n_seq, n_q, d] in the io dtype (post-RoPE is irrelevant for
    the distribution: N(0, 1))."""
    g = _gen(device, w.seed, layer, step, n_seq, TAG_Q)
    q = torch.randn((n_seq, w.n_q, D), generator=g, device=device, dtype=torch.float32)
    return q.to(w.torch_io).contiguous()


def random_cache_contents(rng: np.random.Generator, n_pos: int, bits: int,
                          scale_range=(0.05, 3.0), zero_range=(-6.0, 0.0)):
    """Arbitrary but valid stored cache contents for n_pos positions of one unit:
    codes uint8 [n_pos, d] in [0, 2^bits), binary16 scale/zero (as float64),
    and bfloat16 window values (as float32).  Used to exercise decode attention
    on contents both sides read identically."""
    codes_k = rng.integers(0, 1 << bits, size=(n_pos, D), dtype=np.uint8)
    codes_v = rng.integers(0, 1 << bits, size=(n_pos, D), dtype=np.uint8)
    f16 = lambda a: a.astype(np.float16).astype(np.float64)
    ks = f16(rng.uniform(*scale_range, size=n_pos))
    kz = f16(rng.uniform(*zero_range, size=n_pos))
    vs = f16(rng.uniform(*scale_range, size=n_pos))
    vz = f16(rng.uniform(*zero_range, size=n_pos))
    kw = torch.from_numpy(rng.standard_normal((n_pos, D)).astype(np.float32) * 2).to(
        torch.bfloat16).float().numpy()
    vw = torch.from_numpy(rng.standard_normal((n_pos, D)).astype(np.float32)).to(
        torch.bfloat16).float().numpy()
    return dict(kcodes=codes_k, vcodes=codes_v, ks16=ks, kz16=kz, vs16=vs, vz16=vz,
                k_bf16=kw, v_bf16=vw)
