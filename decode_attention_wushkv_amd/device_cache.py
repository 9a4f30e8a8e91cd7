"""PyTorch plumbing around the C ABI: allocate the cache arena, the decode
workspace and the output on a HIP device and pass raw addresses and the
current stream to libwushkv.  For paged caches it also keeps the block table
(a host-side free list of physical pages, mirrored to the device table the
kernels read).  No arithmetic of the method happens here: which positions are
quantized comes from the library (wushkv_quantized_range).

Two debugging aids, off by default (the test-suite turns them on through the
class attributes): guard bands of a known byte pattern around the arena and
the workspaces, verified by check_guards(), and outputs and workspaces filled
with NaN bytes before every call, so that a kernel that skips a write shows."""
from __future__ import annotations

import weakref

import numpy as np
import torch

from . import (WUSHKV_IO_BF16, WUSHKV_IO_FP32, make_config, wushkv_append, wushkv_cache_create,
               wushkv_cache_destroy, wushkv_chunk_step, wushkv_chunk_workspace_bytes,
               wushkv_decode_attn, wushkv_decode_step,
               wushkv_decode_workspace_bytes, wushkv_get_len, wushkv_layout,
               wushkv_quantized_range, wushkv_reset_seq, wushkv_set_block_table)

GUARD_BYTE = 0xA5


class DeviceCache:
    """page_size > 0 makes the quantized planes paged: a pool of n_pages pages
    per layer, handed out from a free list in the order given by page_seed (a
    seeded shuffle; None keeps ascending order) as sequences grow."""

    guard_bytes = 0        # bytes of guard pattern before and after each buffer
    poison = False         # NaN-fill outputs and workspaces before every call
    live = weakref.WeakSet()
    guard_failures = []    # descriptions of corrupted guards found at close()

    def __init__(self, *, n_layers, n_q_heads, n_kv_heads, bits, sink, recent, flush=1,
                 p_lo=0.01, p_hi=0.99, max_batch, ctx_cap, io_dtype: torch.dtype,
                 device="cuda", codec=0, clip_alpha=0.0, page_size=0, n_pages=0,
                 page_seed=None):
        io = WUSHKV_IO_BF16 if io_dtype == torch.bfloat16 else WUSHKV_IO_FP32
        if io_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("io dtype must be bfloat16 or float32")
        self.io_dtype = io_dtype
        self.cfg = make_config(n_layers=n_layers, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                               bits=bits, sink=sink, recent=recent, flush=flush, p_lo=p_lo,
                               p_hi=p_hi, max_batch=max_batch, ctx_cap=ctx_cap, io_dtype=io, codec=codec,
                               clip_alpha=clip_alpha, page_size=page_size, n_pages=n_pages)
        self.layout = wushkv_layout(self.cfg)
        device = torch.device(device)
        if device.type == "cuda" and device.index is None:
            device = torch.device("cuda", torch.cuda.current_device())
        self.device = device
        self._guarded = []  # (name, buffer, payload bytes) with guard bands
        self.arena = self._alloc("arena", self.layout.total_bytes)
        self.handle = wushkv_cache_create(self.cfg, self.arena.data_ptr(), self.layout.total_bytes)
        self._ws = None
        self._cws = None
        DeviceCache.live.add(self)
        self.table = None
        if page_size:
            pps = self.layout.pages_per_seq
            self.table_host = np.full((max_batch, pps), -1, dtype=np.int32)
            self.table = torch.full((max_batch, pps), -1, dtype=torch.int32, device=self.device)
            order = np.arange(n_pages, dtype=np.int64)
            if page_seed is not None:
                order = np.random.default_rng(page_seed).permutation(n_pages)
            self._free = [int(x) for x in order[::-1]]   # pop() takes the front of `order`
            self._mapped = [0] * max_batch                 # logical pages [0, n) examined per slot
            wushkv_set_block_table(self.handle, self.table.data_ptr())

    def _alloc(self, name: str, nbytes: int) -> torch.Tensor:
        """A device byte buffer of nbytes (256-byte aligned), inside guard bands
        when guard_bytes > 0."""
        g = (self.guard_bytes + 255) // 256 * 256
        if g == 0:
            return torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        buf = torch.empty(nbytes + 2 * g, dtype=torch.uint8, device=self.device)
        buf[:g].fill_(GUARD_BYTE)
        buf[g + nbytes:].fill_(GUARD_BYTE)
        self._guarded.append((name, buf, nbytes))
        return buf[g:g + nbytes]

    def check_guards(self) -> list:
        """Names of the buffers whose guard bands were overwritten."""
        g = (self.guard_bytes + 255) // 256 * 256
        bad = []
        for name, buf, n in self._guarded:
            if not (bool((buf[:g] == GUARD_BYTE).all()) and bool((buf[g + n:] == GUARD_BYTE).all())):
                bad.append(name)
        return bad

    def squant(self, L: int) -> int:
        return wushkv_quantized_range(self.handle, L)[1]

    def reserve(self, slot: int, length: int):
        """Map every page that holds a quantized position of slot at `length`
        (the library's quantized range at that length); no-op for contiguous
        caches."""
        if self.table is None:
            return
        begin, end = wushkv_quantized_range(self.handle, length)
        P = self.layout.page_size
        need = (end - 1) // P + 1 if end > begin else 0
        if need <= self._mapped[slot]:
            return
        row = self.table_host[slot]
        for i in range(max(self._mapped[slot], begin // P), need):
            if row[i] < 0:
                if not self._free:
                    raise RuntimeError("page pool exhausted")
                row[i] = self._free.pop()
        self._mapped[slot] = need
        # stream-ordered: the kernels enqueued after this copy see the new entries
        self.table[slot].copy_(torch.from_numpy(row.copy()))

    def pages_in_use(self) -> int:
        return 0 if self.table is None else int((self.table_host >= 0).sum())

    def close(self):
        if self.handle:
            if self._guarded:
                torch.cuda.synchronize(self.device)
                for name in self.check_guards():
                    DeviceCache.guard_failures.append(f"{name} of a {self.cfg.bits}-bit cache")
            wushkv_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _stream(self):
        return torch.cuda.current_stream(self.device).cuda_stream

    def plane(self, name: str) -> torch.Tensor:
        off = getattr(self.layout, f"off_{name}")
        n = getattr(self.layout, f"bytes_{name}")
        return self.arena[off:off + n]

    def reset_seq(self, slot: int):
        """Forget slot; a paged cache returns its pages to the free list."""
        wushkv_reset_seq(self.handle, slot)
        if self.table is not None:
            row = self.table_host[slot]
            self._free.extend(int(x) for x in row[row >= 0][::-1])
            row[:] = -1
            self._mapped[slot] = 0
            self.table[slot].copy_(torch.from_numpy(row.copy()))

    def get_len(self, layer: int, slot: int):
        return wushkv_get_len(self.handle, layer, slot)

    def append(self, layer: int, slots, n_new, k: torch.Tensor, v: torch.Tensor, tk: torch.Tensor):
        for t in (k, v):
            assert t.dtype == self.io_dtype and t.is_contiguous() and t.device == self.device
        assert tk.dtype == torch.float32 and tk.is_contiguous() and tk.device == self.device
        if self.table is not None:
            for s, n in zip(slots, n_new):
                self.reserve(s, self.get_len(layer, s)[0] + n)
        wushkv_append(self.handle, layer, slots, n_new, k.data_ptr(), v.data_ptr(), tk.data_ptr(),
                      self._stream())

    def workspace(self, n_seq: int) -> torch.Tensor:
        need = wushkv_decode_workspace_bytes(self.handle, n_seq)
        if self._ws is None or self._ws.numel() < need:
            self._ws = self._alloc("decode workspace", need)
        if self.poison:
            self._ws.fill_(0xFF)
        return self._ws

    def _out(self, out, rows: int) -> torch.Tensor:
        if out is None:
            out = torch.empty((rows, self.cfg.n_q_heads, 128), dtype=torch.float32,
                              device=self.device)
        if self.poison:
            out.fill_(float("nan"))
        return out

    def decode_attn(self, layer: int, slots, q: torch.Tensor, tq: torch.Tensor,
                    out: torch.Tensor | None = None) -> torch.Tensor:
        assert q.dtype == self.io_dtype and q.is_contiguous() and q.device == self.device
        assert tq.dtype == torch.float32 and tq.is_contiguous()
        n_seq = len(slots)
        out = self._out(out, n_seq)
        ws = self.workspace(n_seq)
        wushkv_decode_attn(self.handle, layer, slots, q.data_ptr(), tq.data_ptr(), out.data_ptr(),
                           ws.data_ptr(), ws.numel(), self._stream())
        return out

    def decode_step(self, layer: int, slots, k: torch.Tensor, v: torch.Tensor, tk: torch.Tensor,
                    q: torch.Tensor, tq: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        """Append one position per sequence and attend to all positions (new one
        included, flush after the attention); k, v are [n_seq][n_kv][128]."""
        for t in (k, v, q):
            assert t.dtype == self.io_dtype and t.is_contiguous() and t.device == self.device
        for t in (tk, tq):
            assert t.dtype == torch.float32 and t.is_contiguous() and t.device == self.device
        n_seq = len(slots)
        out = self._out(out, n_seq)
        ws = self.workspace(n_seq)
        if self.table is not None:
            for s in slots:
                self.reserve(s, self.get_len(layer, s)[0] + 1)
        wushkv_decode_step(self.handle, layer, slots, k.data_ptr(), v.data_ptr(), tk.data_ptr(),
                           q.data_ptr(), tq.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(),
                           self._stream())
        return out

    def chunk_step(self, layer: int, slots, n_new, k: torch.Tensor, v: torch.Tensor,
                   tk: torch.Tensor, q: torch.Tensor, tq: torch.Tensor,
                   out: torch.Tensor | None = None) -> torch.Tensor:
        """Append n_new[i] positions per sequence and attend each new position's
        queries causally (chunk entries in full precision, flush after);
        k, v are [sum(n_new)][n_kv][128], q is [sum(n_new)][n_q][128]."""
        for t in (k, v, q):
            assert t.dtype == self.io_dtype and t.is_contiguous() and t.device == self.device
        for t in (tk, tq):
            assert t.dtype == torch.float32 and t.is_contiguous() and t.device == self.device
        n_tok = int(sum(n_new))
        out = self._out(out, n_tok)
        need = wushkv_chunk_workspace_bytes(self.handle, len(slots), max(n_new))
        if self._cws is None or self._cws.numel() < need:
            self._cws = self._alloc("chunk workspace", need)
        if self.poison:
            self._cws.fill_(0xFF)
        if self.table is not None:
            for s, n in zip(slots, n_new):
                self.reserve(s, self.get_len(layer, s)[0] + n)
        wushkv_chunk_step(self.handle, layer, slots, n_new, k.data_ptr(), v.data_ptr(),
                          tk.data_ptr(), q.data_ptr(), tq.data_ptr(), out.data_ptr(),
                          self._cws.data_ptr(), self._cws.numel(), self._stream())
        return out
