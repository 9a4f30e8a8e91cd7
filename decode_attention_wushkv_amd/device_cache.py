"""PyTorch plumbing around the C ABI: allocate the cache arena, the decode
workspace and the output on a HIP device and pass raw addresses and the
current stream to libwushkv.  No arithmetic of the method happens here."""
from __future__ import annotations

import torch

from . import (WUSHKV_IO_BF16, WUSHKV_IO_FP32, make_config, wushkv_append, wushkv_cache_create,
               wushkv_cache_destroy, wushkv_decode_attn, wushkv_decode_step,
               wushkv_decode_workspace_bytes, wushkv_get_len, wushkv_layout, wushkv_reset_seq)


class DeviceCache:
    def __init__(self, *, n_layers, n_q_heads, n_kv_heads, bits, sink, recent, flush=1,
                 p_lo=0.01, p_hi=0.99, max_batch, ctx_cap, io_dtype: torch.dtype,
                 device="cuda", codec=0, clip_alpha=0.0):
        io = WUSHKV_IO_BF16 if io_dtype == torch.bfloat16 else WUSHKV_IO_FP32
        if io_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("io dtype must be bfloat16 or float32")
        self.io_dtype = io_dtype
        self.cfg = make_config(n_layers=n_layers, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                               bits=bits, sink=sink, recent=recent, flush=flush, p_lo=p_lo,
                               p_hi=p_hi, max_batch=max_batch, ctx_cap=ctx_cap, io_dtype=io, codec=codec,
                               clip_alpha=clip_alpha)
        self.layout = wushkv_layout(self.cfg)
        device = torch.device(device)
        if device.type == "cuda" and device.index is None:
            device = torch.device("cuda", torch.cuda.current_device())
        self.device = device
        self.arena = torch.empty(self.layout.total_bytes, dtype=torch.uint8, device=self.device)
        self.handle = wushkv_cache_create(self.cfg, self.arena.data_ptr(), self.layout.total_bytes)
        self._ws = None

    def close(self):
        if self.handle:
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
        wushkv_reset_seq(self.handle, slot)

    def get_len(self, layer: int, slot: int):
        return wushkv_get_len(self.handle, layer, slot)

    def append(self, layer: int, slots, n_new, k: torch.Tensor, v: torch.Tensor, tk: torch.Tensor):
        for t in (k, v):
            assert t.dtype == self.io_dtype and t.is_contiguous() and t.device == self.device
        assert tk.dtype == torch.float32 and tk.is_contiguous() and tk.device == self.device
        wushkv_append(self.handle, layer, slots, n_new, k.data_ptr(), v.data_ptr(), tk.data_ptr(),
                      self._stream())

    def workspace(self, n_seq: int) -> torch.Tensor:
        need = wushkv_decode_workspace_bytes(self.handle, n_seq)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def decode_attn(self, layer: int, slots, q: torch.Tensor, tq: torch.Tensor,
                    out: torch.Tensor | None = None) -> torch.Tensor:
        assert q.dtype == self.io_dtype and q.is_contiguous() and q.device == self.device
        assert tq.dtype == torch.float32 and tq.is_contiguous()
        n_seq = len(slots)
        if out is None:
            out = torch.empty((n_seq, self.cfg.n_q_heads, 128), dtype=torch.float32,
                              device=self.device)
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
        if out is None:
            out = torch.empty((n_seq, self.cfg.n_q_heads, 128), dtype=torch.float32,
                              device=self.device)
        ws = self.workspace(n_seq)
        wushkv_decode_step(self.handle, layer, slots, k.data_ptr(), v.data_ptr(), tk.data_ptr(),
                           q.data_ptr(), tq.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(),
                           self._stream())
        return out
