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


def hi_bit(e):
    """Bit of element e (0..127) in the 128-bit high plane of 3-bit codes
    (include/wushkv.h): bit 4 n + k of word j holds element
    32 j + 16 (k >> 1) + 2 n + (k & 1)."""
    e = np.asarray(e)
    return 32 * (e >> 5) + 4 * ((e & 15) >> 1) + ((((e & 31) >> 4) << 1) | (e & 1))


HI = hi_bit(np.arange(128))


def unpack3(lo_raw: np.ndarray, hi_raw: np.ndarray) -> np.ndarray:
    """3-bit codes of 128 elements from their low plane ([..., 32] bytes, 2-bit
    packing) and high plane ([..., 16] bytes)."""
    lo = unpack_bits(lo_raw, 2, 128)
    hb = hi_raw[..., HI >> 3] >> (HI & 7) & 1
    return lo | (hb << 2)


def pack3(codes: np.ndarray):
    """Inverse of unpack3: (low plane [..., 32], high plane [..., 16]) bytes."""
    lo = pack_bits(codes & 3, 2)
    hb = (codes >> 2) & 1
    hi = np.zeros(codes.shape[:-1] + (16,), dtype=np.uint8)
    for e in range(128):
        b = int(HI[e])
        hi[..., b >> 3] |= (hb[..., e] << (b & 7)).astype(np.uint8)
    return lo, hi


def f16_pair(u32: np.ndarray):
    s = (u32 & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    z = (u32 >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    return s, z


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def row_runs(dc, layer: int, slot: int, head: int, n: int):
    """Runs (first position, first row or None when unmapped, positions) of the
    quantized-plane rows holding positions [0, n) of one unit, per the
    documented contiguous or paged layout (the block table read back from the
    device)."""
    c, lay = dc.cfg, dc.layout
    if lay.page_size == 0:
        return [(0, _unit(dc, layer, slot, head) * lay.cpos, lay.cpos)]
    P = lay.page_size
    table = dc.table[slot].cpu().numpy()
    runs = []
    for i in range((max(n, 1) + P - 1) // P):
        pg = int(table[i])
        row0 = ((layer * lay.n_pages + pg) * c.n_kv_heads + head) * P if 0 <= pg < lay.n_pages else None
        runs.append((i * P, row0, P))
    return runs


def _read_rows(dc, runs, name, row_bytes, rows_per_unit=1):
    """Concatenate plane bytes of the runs ([positions, row_bytes]; zeros for
    unmapped runs); rows_per_unit > 1 reads whole value-code blocks."""
    parts = []
    for _, row0, cnt in runs:
        nb = cnt // rows_per_unit * row_bytes
        if row0 is None:
            parts.append(np.zeros(nb, dtype=np.uint8))
        else:
            parts.append(_slice(dc, name, row0 // rows_per_unit * row_bytes, nb).cpu().numpy())
    return np.concatenate(parts)


def read_unit(dc, layer: int, slot: int, head: int, L: int) -> dict:
    """Canonical contents of one unit at length L: codes [L, 128] (uint8; rows
    outside the quantized region are garbage), s/z [L], window values [L, 128]
    (NaN outside the windows), plus the region bounds."""
    c, lay = dc.cfg, dc.layout
    u = _unit(dc, layer, slot, head)
    bits, S, W = c.bits, c.sink, lay.ring_slots
    cb, VB = lay.code_bytes, lay.vblock
    n = max(L, 1)
    runs = row_runs(dc, layer, slot, head, n)
    kraw = _read_rows(dc, runs, "kcode", cb).reshape(-1, cb)[:n]
    if bits == 3:
        kcodes = unpack3(kraw[:, :32], kraw[:, 32:]).astype(np.uint8)
        # block of 128 positions: low-plane rows for positions [0, 64) and
        # [64, 128), then the high-plane row, each [128 dims][16 B]
        vraw = _read_rows(dc, runs, "vcode", 3 * 128 * 16, 128).reshape(-1, 3, 128, 16)
        lo = np.concatenate([vraw[:, 0], vraw[:, 1]], axis=-1)      # [blocks, dims, 32]
        vc = unpack3(lo, vraw[:, 2])                                 # [blocks, dims, 128]
        vcodes = vc.transpose(0, 2, 1).reshape(-1, 128)[:n].astype(np.uint8)
    else:
        kcodes = unpack_bits(kraw, bits, 128).astype(np.uint8)
        vraw = _read_rows(dc, runs, "vcode", 128 * 16, VB).reshape(-1, 128, 16)
        vc = unpack_bits(vraw, bits, VB)                     # [blocks, 128 dims, VB]
        vcodes = vc.transpose(0, 2, 1).reshape(-1, 128)[:n].astype(np.uint8)
    ksz = _read_rows(dc, runs, "ksz", 4).view(np.uint32)[:n]
    vsz = _read_rows(dc, runs, "vsz", 4).view(np.uint32)[:n]
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
    cb, VB = lay.code_bytes, lay.vblock
    dev = dc.device
    runs = row_runs(dc, layer, slot, head, L)
    npos = sum(cnt for _, _, cnt in runs)
    kc = np.zeros((npos, 128), dtype=np.uint8)
    vcd = np.zeros((npos, 128), dtype=np.uint8)
    kc[:L] = contents["kcodes"][:L]
    vcd[:L] = contents["vcodes"][:L]
    vblk = np.ascontiguousarray(vcd.reshape(npos // VB, VB, 128).transpose(0, 2, 1))  # [blocks, dims, VB]
    if bits == 3:
        klo, khi = pack3(kc)
        kraw = np.concatenate([klo, khi], axis=-1)                      # [positions, 48]
        vlo, vhi = pack3(vblk)                                          # [blocks, dims, 32 / 16]
        vraw = np.stack([vlo[..., :16], vlo[..., 16:], vhi], axis=1)    # [blocks, 3, dims, 16]
        vrow_bytes = 3 * 2048
    else:
        kraw = pack_bits(kc, bits)                                      # [positions, cb]
        vraw = pack_bits(vblk, bits)                                    # [blocks, dims, 16]
        vrow_bytes = 2048

    def sz(s, z):
        out = np.zeros(npos, dtype=np.uint32)
        su = np.asarray(s[:L], dtype=np.float16).view(np.uint16).astype(np.uint32)
        zu = np.asarray(z[:L], dtype=np.float16).view(np.uint16).astype(np.uint32)
        out[:L] = su | (zu << 16)
        return out

    ksz = sz(contents["ks16"], contents["kz16"])
    vsz = sz(contents["vs16"], contents["vz16"])
    for p0, row0, cnt in runs:
        if row0 is None:
            continue
        planes = (("kcode", kraw[p0:p0 + cnt], row0 * cb),
                  ("vcode", vraw[p0 // VB:(p0 + cnt) // VB], row0 // VB * vrow_bytes),
                  ("ksz", ksz[p0:p0 + cnt].view(np.uint8), row0 * 4),
                  ("vsz", vsz[p0:p0 + cnt].view(np.uint8), row0 * 4))
        for name, arr, off in planes:
            arr = np.ascontiguousarray(arr).reshape(-1)
            _slice(dc, name, off, arr.size).copy_(torch.from_numpy(arr).to(dev))

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
