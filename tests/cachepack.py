"""Test-side reader/writer of the documented cache arena layout (include/wushkv.h).

Reads one (layer, slot, KV head) unit of a DeviceCache back to numpy in
canonical form, or writes arbitrary canonical contents into it.  Pure data
movement and bit (un)packing; no arithmetic of the method.
"""
from __future__ import annotations

import numpy as np
import torch


def _unit(dc, layer, slot, head):
    c = dc.cfg
    return (layer * c.max_batch + slot) * c.n_kv_heads + head


def _slice(dc, name, start, nbytes):
    off = getattr(dc.layout, f"off_{name}") + start
    return dc.arena[off:off + nbytes]


def unpack_bits(raw: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Little-endian b-bit fields of a byte array [..., nbytes] -> [..., n]."""
    per = 8 // bits
    idx = np.arange(n)
    byte = raw[..., idx // per]
    return (byte >> ((idx % per) * bits)) & ((1 << bits) - 1)


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    per = 8 // bits
    n = codes.shape[-1]
    out = np.zeros(codes.shape[:-1] + (n // per,), dtype=np.uint8)
    for e in range(per):
        out |= (codes[..., e::per].astype(np.uint8) << (e * bits)).astype(np.uint8)
    return out


def f16_pair(u32: np.ndarray):
    s = (u32 & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    z = (u32 >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    return s, z


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def read_unit(dc, layer: int, slot: int, head: int, L: int) -> dict:
    """Canonical contents of one unit at length L: codes [L, 128] (uint8; rows
    outside the quantized region are garbage), s/z [L], window values [L, 128]
    (NaN outside the windows), plus the region bounds."""
    c, lay = dc.cfg, dc.layout
    u = _unit(dc, layer, slot, head)
    bits, S, W = c.bits, c.sink, lay.ring_slots
    cb, cpos, VB = lay.code_bytes, lay.cpos, lay.vblock
    n = max(L, 1)
    kraw = _slice(dc, "kcode", u * cpos * cb, cpos * cb).cpu().numpy().reshape(cpos, cb)[:n]
    kcodes = unpack_bits(kraw, bits, 128).astype(np.uint8)
    vraw = _slice(dc, "vcode", u * lay.ctx_blocks * 128 * 16, lay.ctx_blocks * 128 * 16)
    vraw = vraw.cpu().numpy().reshape(lay.ctx_blocks, 128, 16)
    vc = unpack_bits(vraw, bits, VB)                     # [blocks, 128 dims, VB]
    vcodes = vc.transpose(0, 2, 1).reshape(-1, 128)[:n].astype(np.uint8)
    ksz = _slice(dc, "ksz", u * cpos * 4, cpos * 4).cpu().numpy().view(np.uint32)[:n]
    vsz = _slice(dc, "vsz", u * cpos * 4, cpos * 4).cpu().numpy().view(np.uint32)[:n]
    ks, kz = f16_pair(ksz)
    vs, vz = f16_pair(vsz)
    sq = S + c.flush * (max(0, L - c.recent - S) // c.flush)
    kwin = np.full((n, 128), np.nan)
    vwin = np.full((n, 128), np.nan)
    if S:
        ksink = _slice(dc, "ksink", u * S * 256, S * 256).cpu().numpy().view(np.uint16).reshape(S, 128)
        vsink = _slice(dc, "vsink", u * S * 256, S * 256).cpu().numpy().view(np.uint16).reshape(S, 128)
        m = min(S, L)
        kwin[:m] = bf16_to_f64(ksink[:m])
        vwin[:m] = bf16_to_f64(vsink[:m])
    if W and L > sq:
        kring = _slice(dc, "kring", u * W * 256, W * 256).cpu().numpy().view(np.uint16).reshape(W, 128)
        vring = _slice(dc, "vring", u * W * 256, W * 256).cpu().numpy().view(np.uint16).reshape(W, 128)
        for p in range(max(sq, S), L):
            kwin[p] = bf16_to_f64(kring[(p - S) % W])
            vwin[p] = bf16_to_f64(vring[(p - S) % W])
    return dict(kcodes=kcodes, vcodes=vcodes, ks16=ks, kz16=kz, vs16=vs, vz16=vz,
                kwin=kwin, vwin=vwin, squant=sq, L=L)


def write_unit(dc, layer: int, slot: int, head: int, L: int, contents: dict) -> None:
    """Write canonical contents for positions [0, L) of one unit: codes and s/z
    for the quantized region, bfloat16 window values for sink and ring."""
    c, lay = dc.cfg, dc.layout
    u = _unit(dc, layer, slot, head)
    bits, S, W = c.bits, c.sink, lay.ring_slots
    cb, cpos, VB = lay.code_bytes, lay.cpos, lay.vblock
    dev = dc.device
    kc = np.zeros((cpos, 128), dtype=np.uint8)
    vcd = np.zeros((cpos, 128), dtype=np.uint8)
    kc[:L] = contents["kcodes"][:L]
    vcd[:L] = contents["vcodes"][:L]
    kraw = pack_bits(kc, bits)
    vblk = vcd.reshape(lay.ctx_blocks, VB, 128).transpose(0, 2, 1)    # [blocks, dims, VB]
    vraw = pack_bits(np.ascontiguousarray(vblk), bits)                  # [blocks, dims, 16]
    _slice(dc, "kcode", u * cpos * cb, cpos * cb).copy_(torch.from_numpy(kraw.reshape(-1)).to(dev))
    _slice(dc, "vcode", u * lay.ctx_blocks * 2048, lay.ctx_blocks * 2048).copy_(
        torch.from_numpy(vraw.reshape(-1)).to(dev))

    def sz(s, z):
        out = np.zeros(cpos, dtype=np.uint32)
        su = np.asarray(s[:L], dtype=np.float16).view(np.uint16).astype(np.uint32)
        zu = np.asarray(z[:L], dtype=np.float16).view(np.uint16).astype(np.uint32)
        out[:L] = su | (zu << 16)
        return torch.from_numpy(out.view(np.uint8)).to(dev)

    _slice(dc, "ksz", u * cpos * 4, cpos * 4).copy_(sz(contents["ks16"], contents["kz16"]))
    _slice(dc, "vsz", u * cpos * 4, cpos * 4).copy_(sz(contents["vs16"], contents["vz16"]))

    def bf(x):
        return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.uint8)

    if S:
        m = min(S, L)
        ks = torch.zeros((S, 128), dtype=torch.bfloat16)
        vs = torch.zeros((S, 128), dtype=torch.bfloat16)
        ks[:m] = torch.from_numpy(np.asarray(contents["k_bf16"][:m], dtype=np.float32)).to(torch.bfloat16)
        vs[:m] = torch.from_numpy(np.asarray(contents["v_bf16"][:m], dtype=np.float32)).to(torch.bfloat16)
        _slice(dc, "ksink", u * S * 256, S * 256).copy_(ks.view(torch.uint8).reshape(-1).to(dev))
        _slice(dc, "vsink", u * S * 256, S * 256).copy_(vs.view(torch.uint8).reshape(-1).to(dev))
    sq = S + c.flush * (max(0, L - c.recent - S) // c.flush)
    if W:
        kr = torch.zeros((W, 128), dtype=torch.bfloat16)
        vr = torch.zeros((W, 128), dtype=torch.bfloat16)
        for p in range(max(sq, S), L):
            kr[(p - S) % W] = torch.from_numpy(np.asarray(contents["k_bf16"][p], dtype=np.float32)).to(torch.bfloat16)
            vr[(p - S) % W] = torch.from_numpy(np.asarray(contents["v_bf16"][p], dtype=np.float32)).to(torch.bfloat16)
        _slice(dc, "kring", u * W * 256, W * 256).copy_(kr.view(torch.uint8).reshape(-1).to(dev))
        _slice(dc, "vring", u * W * 256, W * 256).copy_(vr.view(torch.uint8).reshape(-1).to(dev))
