// C-ABI entry points of libwushkv: argument checks, arena layout, host-side
// sequence lengths and kernel launches.  No device memory is allocated here.
#include <string.h>
#include <cmath>

#include <new>
#include <vector>

#include "../../include/wushkv.h"
#include "common.h"
#include "chunk.h"

using namespace wkv;

struct wushkv_cache {
  wushkv_config cfg;
  wushkv_layout_t lay;
  uint8_t* arena;
  const int32_t* table = nullptr;  // paged caches: device block table [max_batch][pages_per_seq]
  std::vector<int32_t> len;  // [n_layers][max_batch]
  hipEvent_t ev_start = nullptr, ev_stop = nullptr;    // around the split-K scan launch
  hipEvent_t ev_cstart = nullptr, ev_cstop = nullptr;  // around the combine launch
};

static uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// E[(x - Q(x))^2] for x ~ N(0, 1) and Q rounding to the nearest of 2^bits
// levels -alpha + k delta, delta = 2 alpha / (2^bits - 1).  On a decision
// interval [a, b] with level y the integral of (x - y)^2 phi(x) is
// (1 + y^2)(Phi(b) - Phi(a)) - (b phi(b) - a phi(a)) + 2 y (phi(b) - phi(a)).
static double gaussian_grid_mse(double alpha, int bits) {
  const int n = 1 << bits;
  const double delta = 2.0 * alpha / (n - 1);
  const double inv_sqrt2 = 0.70710678118654752440, inv_sqrt2pi = 0.39894228040143267794;
  auto Phi = [&](double x) { return 0.5 * std::erfc(-x * inv_sqrt2); };
  auto phi = [&](double x) { return inv_sqrt2pi * std::exp(-0.5 * x * x); };
  double total = 0.0;
  for (int k = 0; k < n; ++k) {
    const double y = -alpha + delta * k;
    const bool lo_inf = k == 0, hi_inf = k == n - 1;
    const double a = y - 0.5 * delta, b = y + 0.5 * delta;
    const double Pa = lo_inf ? 0.0 : Phi(a), Pb = hi_inf ? 1.0 : Phi(b);
    const double pa = lo_inf ? 0.0 : phi(a), pb = hi_inf ? 0.0 : phi(b);
    const double apa = lo_inf ? 0.0 : a * pa, bpb = hi_inf ? 0.0 : b * pb;
    total += (1.0 + y * y) * (Pb - Pa) - (bpb - apa) + 2.0 * y * (pb - pa);
  }
  return total;
}

extern "C" double wushkv_gaussian_alpha(int32_t bits) {
  if (bits < 1 || bits > 8) return 0.0;
  // golden-section search on [0.3, 6]: the error is unimodal in alpha there
  const double r = 0.61803398874989484820;
  double lo = 0.3, hi = 6.0;
  double x1 = hi - r * (hi - lo), x2 = lo + r * (hi - lo);
  double f1 = gaussian_grid_mse(x1, bits), f2 = gaussian_grid_mse(x2, bits);
  for (int it = 0; it < 200 && hi - lo > 1e-13; ++it) {
    if (f1 < f2) {
      hi = x2;
      x2 = x1;
      f2 = f1;
      x1 = hi - r * (hi - lo);
      f1 = gaussian_grid_mse(x1, bits);
    } else {
      lo = x1;
      x1 = x2;
      f1 = f2;
      x2 = lo + r * (hi - lo);
      f2 = gaussian_grid_mse(x2, bits);
    }
  }
  return 0.5 * (lo + hi);
}

extern "C" wushkv_status wushkv_config_check(const wushkv_config* c) {
  if (!c) return WUSHKV_EINVAL;
  if (c->n_layers < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->max_batch < 1 ||
      c->ctx_cap < 1)
    return WUSHKV_EINVAL;
  if (c->n_q_heads % c->n_kv_heads != 0) return WUSHKV_EINVAL;
  if (c->sink < 0 || c->recent < 0 || c->flush < 1) return WUSHKV_EINVAL;
  if (!(c->p_lo >= 0.0 && c->p_lo < c->p_hi && c->p_hi <= 1.0)) return WUSHKV_EINVAL;
  if (c->io_dtype != WUSHKV_IO_FP32 && c->io_dtype != WUSHKV_IO_BF16) return WUSHKV_EINVAL;
  if (c->codec != WUSHKV_CODEC_PERCENTILE && c->codec != WUSHKV_CODEC_RMS) return WUSHKV_EINVAL;
  if (!(c->clip_alpha >= 0.0 && c->clip_alpha < 1e6)) return WUSHKV_EINVAL;
  if (c->head_dim != D) return WUSHKV_EUNSUPPORTED;
  if (c->bits < 2 || c->bits > 4) return WUSHKV_EUNSUPPORTED;
  {
    const int G = c->n_q_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return WUSHKV_EUNSUPPORTED;
  }
  // The window split scores all sink + ring entries in one workgroup.
  if ((int64_t)c->sink + c->recent + c->flush - 1 > WINDOW_MAX) return WUSHKV_EUNSUPPORTED;
  // Paged quantized planes: pages of a power-of-two number of positions, at
  // least one decode sub-chunk (128) and at most 2^20.
  if (c->page_size == 0) {
    if (c->n_pages != 0) return WUSHKV_EINVAL;
  } else {
    const int P = c->page_size;
    if (P < 128 || P > (1 << 20) || (P & (P - 1)) != 0 || c->n_pages < 1) return WUSHKV_EINVAL;
  }
  return WUSHKV_OK;
}

extern "C" wushkv_status wushkv_layout(const wushkv_config* c, wushkv_layout_t* out) {
  wushkv_status st = wushkv_config_check(c);
  if (st != WUSHKV_OK) return st;
  if (!out) return WUSHKV_EINVAL;
  wushkv_layout_t L;
  memset(&L, 0, sizeof(L));
  L.code_bytes = D * c->bits / 8;
  // value-code block: one 16-byte row per dimension (2, 4 bits) or two
  // low-plane rows and one high-plane row (3 bits)
  L.vblock = c->bits == 3 ? 128 : 128 / c->bits;
  // positions per unit: ctx_cap rounded up to 128 (whole decode sub-chunks)
  L.cpos = (c->ctx_cap + 127) / 128 * 128;
  L.ctx_blocks = L.cpos / L.vblock;
  L.ring_slots = c->recent + c->flush - 1;
  L.units = c->n_layers * c->max_batch * c->n_kv_heads;
  const uint64_t u = (uint64_t)L.units;
  // rows of the quantized planes (one per position and KV head)
  uint64_t rows = u * (uint64_t)L.cpos;
  if (c->page_size > 0) {
    L.page_size = c->page_size;
    L.n_pages = c->n_pages;
    L.pages_per_seq = (c->ctx_cap + c->page_size - 1) / c->page_size;
    rows = (uint64_t)c->n_layers * (uint64_t)c->n_pages * (uint64_t)c->n_kv_heads *
           (uint64_t)c->page_size;
  }
  L.bytes_kcode = rows * L.code_bytes;
  L.bytes_vcode = rows * L.code_bytes;
  L.bytes_ksz = rows * 4;
  L.bytes_vsz = L.bytes_ksz;
  L.bytes_ksink = u * (uint64_t)c->sink * D * 2;
  L.bytes_vsink = L.bytes_ksink;
  L.bytes_kring = u * (uint64_t)L.ring_slots * D * 2;
  L.bytes_vring = L.bytes_kring;
  uint64_t off = 0;
  L.off_kcode = off; off = align256(off + L.bytes_kcode);
  L.off_vcode = off; off = align256(off + L.bytes_vcode);
  L.off_ksz = off;   off = align256(off + L.bytes_ksz);
  L.off_vsz = off;   off = align256(off + L.bytes_vsz);
  L.off_ksink = off; off = align256(off + L.bytes_ksink);
  L.off_vsink = off; off = align256(off + L.bytes_vsink);
  L.off_kring = off; off = align256(off + L.bytes_kring);
  L.off_vring = off; off = align256(off + L.bytes_vring);
  L.total_bytes = off;
  *out = L;
  return WUSHKV_OK;
}

extern "C" wushkv_status wushkv_cache_create(const wushkv_config* cfg, void* arena,
                                             uint64_t arena_bytes, wushkv_cache** out) {
  if (!out) return WUSHKV_EINVAL;
  wushkv_layout_t L;
  wushkv_status st = wushkv_layout(cfg, &L);
  if (st != WUSHKV_OK) return st;
  if (!arena || ((uintptr_t)arena & 255) != 0 || arena_bytes < L.total_bytes) return WUSHKV_EINVAL;
  wushkv_cache* c = new (std::nothrow) wushkv_cache;
  if (!c) return WUSHKV_EINVAL;
  c->cfg = *cfg;
  c->lay = L;
  c->arena = (uint8_t*)arena;
  try {
    c->len.assign((size_t)cfg->n_layers * cfg->max_batch, 0);
  } catch (...) {
    delete c;
    return WUSHKV_EINVAL;
  }
  *out = c;
  return WUSHKV_OK;
}

extern "C" void wushkv_cache_destroy(wushkv_cache* c) { delete c; }

extern "C" wushkv_status wushkv_reset_seq(wushkv_cache* c, int32_t slot) {
  if (!c || slot < 0 || slot >= c->cfg.max_batch) return WUSHKV_EINVAL;
  for (int l = 0; l < c->cfg.n_layers; ++l) c->len[(size_t)l * c->cfg.max_batch + slot] = 0;
  return WUSHKV_OK;
}

extern "C" wushkv_status wushkv_get_len(const wushkv_cache* c, int32_t layer, int32_t slot,
                                        int32_t* len, int32_t* sq) {
  if (!c || layer < 0 || layer >= c->cfg.n_layers || slot < 0 || slot >= c->cfg.max_batch)
    return WUSHKV_EINVAL;
  int32_t L = c->len[(size_t)layer * c->cfg.max_batch + slot];
  if (len) *len = L;
  if (sq) *sq = squant_of(L, c->cfg.sink, c->cfg.recent, c->cfg.flush);
  return WUSHKV_OK;
}

extern "C" wushkv_status wushkv_quantized_range(const wushkv_cache* c, int32_t len,
                                                int32_t* begin, int32_t* end) {
  if (!c || !begin || !end || len < 0) return WUSHKV_EINVAL;
  *begin = c->cfg.sink;
  *end = squant_of(len, c->cfg.sink, c->cfg.recent, c->cfg.flush);
  return WUSHKV_OK;
}

static Planes planes_of(const wushkv_cache* c) {
  Planes p;
  uint8_t* a = c->arena;
  p.kcode = a + c->lay.off_kcode;
  p.vcode = a + c->lay.off_vcode;
  p.ksz = (uint32_t*)(a + c->lay.off_ksz);
  p.vsz = (uint32_t*)(a + c->lay.off_vsz);
  p.ksink = (uint16_t*)(a + c->lay.off_ksink);
  p.vsink = (uint16_t*)(a + c->lay.off_vsink);
  p.kring = (uint16_t*)(a + c->lay.off_kring);
  p.vring = (uint16_t*)(a + c->lay.off_vring);
  return p;
}

static Geometry geometry_of(const wushkv_cache* c) {
  Geometry g;
  g.n_kv = c->cfg.n_kv_heads;
  g.n_q = c->cfg.n_q_heads;
  g.G = g.n_q / g.n_kv;
  g.bits = c->cfg.bits;
  g.S = c->cfg.sink;
  g.R = c->cfg.recent;
  g.F = c->cfg.flush;
  g.W = c->lay.ring_slots;
  g.code_bytes = c->lay.code_bytes;
  g.vblock = c->lay.vblock;
  g.ctx_blocks = c->lay.ctx_blocks;
  g.cpos = c->lay.cpos;
  g.max_batch = c->cfg.max_batch;
  g.p_lo = c->cfg.p_lo;
  g.p_hi = c->cfg.p_hi;
  g.codec = c->cfg.codec;
  g.alpha = c->cfg.clip_alpha > 0.0 ? c->cfg.clip_alpha : wushkv_gaussian_alpha(c->cfg.bits);
  if (c->cfg.page_size > 0) {
    g.table = c->table;
    g.pps = c->lay.pages_per_seq;
    g.page_shift = __builtin_ctz((unsigned)c->cfg.page_size);
    g.n_pages = c->cfg.n_pages;
  } else {
    g.table = nullptr;
    g.pps = 0;
    g.page_shift = 0;
    g.n_pages = c->cfg.max_batch;
  }
  return g;
}

// Distinct, in-range slots (n_seq <= MAXSEQ; no allocation).
static bool slots_ok(const wushkv_cache* c, int32_t n_seq, const int32_t* slots) {
  for (int i = 0; i < n_seq; ++i) {
    const int s = slots[i];
    if (s < 0 || s >= c->cfg.max_batch) return false;
    for (int j = 0; j < i; ++j)
      if (slots[j] == s) return false;
  }
  return true;
}

extern "C" wushkv_status wushkv_append(wushkv_cache* c, int32_t layer, int32_t n_seq,
                                       const int32_t* slots, const int32_t* n_new, const void* k,
                                       const void* v, const float* tk, void* stream) {
  if (!c || !slots || !n_new || layer < 0 || layer >= c->cfg.n_layers || n_seq < 0)
    return WUSHKV_EINVAL;
  if (n_seq > MAXSEQ) return WUSHKV_EUNSUPPORTED;
  if (n_seq == 0) return WUSHKV_OK;
  if (!slots_ok(c, n_seq, slots)) return WUSHKV_EINVAL;
  if (c->cfg.page_size > 0 && !c->table) return WUSHKV_EINVAL;
  int64_t total = 0;
  int max_new = 0;
  for (int i = 0; i < n_seq; ++i) {
    if (n_new[i] < 0) return WUSHKV_EINVAL;
    int32_t L = c->len[(size_t)layer * c->cfg.max_batch + slots[i]];
    if ((int64_t)L + n_new[i] > c->cfg.ctx_cap) return WUSHKV_ECAPACITY;
    total += n_new[i];
    if (n_new[i] > max_new) max_new = n_new[i];
  }
  if (total > INT32_MAX) return WUSHKV_EINVAL;
  if (total > 0 && (!k || !v || !tk)) return WUSHKV_EINVAL;
  const size_t esz = c->cfg.io_dtype == WUSHKV_IO_FP32 ? 4 : 2;
  if (total > 0 && (((uintptr_t)k % esz) || ((uintptr_t)v % esz) || ((uintptr_t)tk % 16)))
    return WUSHKV_EINVAL;
  if (total == 0) return WUSHKV_OK;

  AppendArgs a;
  memset(&a, 0, sizeof(a));
  a.pl = planes_of(c);
  a.g = geometry_of(c);
  a.layer = layer;
  a.k = k;
  a.v = v;
  a.tk = tk;
  int32_t tok = 0;
  int max_chunks = 1;
  for (int i = 0; i < n_seq; ++i) {
    int32_t L = c->len[(size_t)layer * c->cfg.max_batch + slots[i]];
    a.s.slot[i] = slots[i];
    a.s.len0[i] = L;
    a.s.n_new[i] = n_new[i];
    a.s.tok0[i] = tok;
    tok += n_new[i];
    int base = L - L % CHUNK;
    int chunks = (L + n_new[i] - base + CHUNK - 1) / CHUNK;
    if (chunks > max_chunks) max_chunks = chunks;
  }
  hipStream_t st = (hipStream_t)stream;
  const int io_bf16 = c->cfg.io_dtype == WUSHKV_IO_BF16;
  hipError_t e;
  if (max_new <= 16) {
    // Few new positions: one workgroup per (sequence, KV head) quantizes the
    // entries leaving the ring, then places the new ones.
    a.mode = APPEND_FUSED;
    e = launch_append(a, io_bf16, 1, n_seq, st);
  } else {
    // Ring entries leaving the window are read before any new entry is
    // written (a new position may reuse the slot of an evicted one).
    a.mode = APPEND_EVICT;
    e = launch_append(a, io_bf16, 1, n_seq, st);
    if (e == hipSuccess) {
      if (io_bf16 && prefill_supported(c->cfg.codec, c->cfg.p_lo, c->cfg.p_hi)) {
        // key transform on the matrix cores, selection-based percentiles
        int spans = 1;
        for (int i = 0; i < n_seq; ++i) {
          const int base = a.s.len0[i] - a.s.len0[i] % PREFILL_TILE;
          const int x = (a.s.len0[i] + a.s.n_new[i] - base + PREFILL_SPAN - 1) / PREFILL_SPAN;
          if (x > spans) spans = x;
        }
        e = launch_prefill(a, spans, n_seq, st);
      } else {
        a.mode = APPEND_CHUNKED;
        e = launch_append(a, io_bf16, max_chunks, n_seq, st);
      }
    }
  }
  if (e != hipSuccess) return WUSHKV_EDEVICE;
  for (int i = 0; i < n_seq; ++i) c->len[(size_t)layer * c->cfg.max_batch + slots[i]] += n_new[i];
  return WUSHKV_OK;
}

// Bytes of the split partials at the start of the decode workspace; the
// query blocks follow.
static uint64_t split_ws_partials(const wushkv_cache* c, int32_t n_seq) {
  const uint64_t nq = (uint64_t)n_seq * c->cfg.n_q_heads;
  return align256(nq * (uint64_t)(max_chunks(n_seq, c->cfg.n_kv_heads) + 1) * PS * 4);
}

extern "C" uint64_t wushkv_decode_workspace_bytes(const wushkv_cache* c, int32_t n_seq) {
  if (!c || n_seq < 0) return 0;
  return split_ws_partials(c, n_seq) +
         align256((uint64_t)n_seq * c->cfg.n_kv_heads *
                  prep_words(c->cfg.n_q_heads / c->cfg.n_kv_heads) * 4);
}

// Shared by decode_attn and decode_step: validation of the attention
// arguments, then the per-sequence plan and the launch.  step = 1 adds the
// fused one-token append (k, v, tk non-null).
// scratch: the workspace is the library's per-device scratch array (ws and
// ws_bytes are ignored and looked up after the argument checks).
static wushkv_status decode_common(wushkv_cache* c, int32_t layer, int32_t n_seq,
                                   const int32_t* slots, const void* k, const void* v,
                                   const float* tk, const void* q, const float* tq, float* out,
                                   void* ws, uint64_t ws_bytes, void* stream, bool step,
                                   bool scratch = false) {
  if (!c || !slots || layer < 0 || layer >= c->cfg.n_layers || n_seq < 0) return WUSHKV_EINVAL;
  if (n_seq > MAXSEQ) return WUSHKV_EUNSUPPORTED;
  if (step && c->cfg.sink + c->cfg.recent + c->cfg.flush > WINDOW_MAX) return WUSHKV_EUNSUPPORTED;
  if (n_seq == 0) return WUSHKV_OK;
  if (scratch) {
    if (wushkv_decode_workspace_bytes(c, n_seq) > WUSHKV_NOALLOC_SCRATCH_BYTES)
      return WUSHKV_EWORKSPACE;
    ws = out;  // stands in until the checks pass (alignment of out is checked)
    ws_bytes = WUSHKV_NOALLOC_SCRATCH_BYTES;
  }
  if (!q || !tq || !out || !ws) return WUSHKV_EINVAL;
  if (step && (!k || !v || !tk)) return WUSHKV_EINVAL;
  const size_t esz = c->cfg.io_dtype == WUSHKV_IO_FP32 ? 4 : 2;
  if (((uintptr_t)q % esz) || ((uintptr_t)tq % 16) || ((uintptr_t)out % 16) ||
      ((uintptr_t)ws % 16))
    return WUSHKV_EINVAL;
  if (step && (((uintptr_t)k % esz) || ((uintptr_t)v % esz) || ((uintptr_t)tk % 16)))
    return WUSHKV_EINVAL;
  if (!slots_ok(c, n_seq, slots)) return WUSHKV_EINVAL;
  if (c->cfg.page_size > 0 && !c->table) return WUSHKV_EINVAL;
  if (ws_bytes < wushkv_decode_workspace_bytes(c, n_seq)) return WUSHKV_EWORKSPACE;
  if (step) {
    for (int i = 0; i < n_seq; ++i)
      if (c->len[(size_t)layer * c->cfg.max_batch + slots[i]] + 1 > c->cfg.ctx_cap)
        return WUSHKV_ECAPACITY;
  } else {
    for (int i = 0; i < n_seq; ++i)
      if (c->len[(size_t)layer * c->cfg.max_batch + slots[i]] < 1) return WUSHKV_EINVAL;
  }
  if (scratch) {
    uint64_t bytes = 0;
    if (noalloc_scratch(&ws, &bytes) != hipSuccess) return WUSHKV_EDEVICE;
    if (bytes < wushkv_decode_workspace_bytes(c, n_seq)) return WUSHKV_EWORKSPACE;
    ws_bytes = bytes;
  }
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.pl = planes_of(c);
  a.g = geometry_of(c);
  a.layer = layer;
  a.n_seq = n_seq;
  a.q = q;
  a.tq = tq;
  a.out = out;
  a.wsp = (float*)ws;
  a.prep = (uint32_t*)((char*)ws + split_ws_partials(c, n_seq));
  a.xcd_map = 1;  // used when the unit count is a multiple of 8
  a.contig = 0;
  if (step) {
    a.k_new = k;
    a.v_new = v;
    a.tk = tk;
  }
  const int sl = sub_len(c->cfg.bits);
  int max_sub = 0;
  int64_t total_sub = 0;
  for (int i = 0; i < n_seq; ++i) {
    const int32_t L = c->len[(size_t)layer * c->cfg.max_batch + slots[i]];
    if (step ? L + 1 > c->cfg.ctx_cap : L < 1) return step ? WUSHKV_ECAPACITY : WUSHKV_EINVAL;
    a.s.slot[i] = slots[i];
    // a step attends at length L + 1 with the boundary of length L (flush after)
    a.s.len[i] = step ? L + 1 : L;
    a.s.squant[i] = squant_of(L, c->cfg.sink, c->cfg.recent, c->cfg.flush);
    const int sq = a.s.squant[i];
    const int nsub = sq > c->cfg.sink ? (sq + sl - 1) / sl - c->cfg.sink / sl : 0;
    if (nsub > max_sub) max_sub = nsub;
    total_sub += nsub;
  }
  a.max_sub = max_sub;
  a.total_sub = total_sub * c->cfg.n_kv_heads;
  // workgroups per (sequence, KV head): at least one sub-chunk per wave, at
  // most what the launcher's grid policy allows, capped by the workspace
  // bound
  int cap = max_chunks(n_seq, c->cfg.n_kv_heads);
  // four waves per workgroup on different sub-chunks (G >= 4: of 64
  // positions, for the int8 matrix cores)
  const int G = c->cfg.n_q_heads / c->cfg.n_kv_heads;
  int need = G >= 4 ? (max_sub * (sl / 64) + 3) / 4 : (max_sub + 3) / 4;
  a.n_splits = need < cap ? need : cap;
  hipError_t e = launch_decode(a, c->cfg.io_dtype == WUSHKV_IO_BF16, (hipStream_t)stream,
                               c->ev_start, c->ev_stop, c->ev_cstart, c->ev_cstop);
  if (e != hipSuccess) return WUSHKV_EDEVICE;
  if (step)
    for (int i = 0; i < n_seq; ++i) c->len[(size_t)layer * c->cfg.max_batch + slots[i]] += 1;
  return WUSHKV_OK;
}

extern "C" wushkv_status wushkv_decode_attn(wushkv_cache* c, int32_t layer, int32_t n_seq,
                                            const int32_t* slots, const void* q, const float* tq,
                                            float* out, void* ws, uint64_t ws_bytes,
                                            void* stream) {
  return decode_common(c, layer, n_seq, slots, nullptr, nullptr, nullptr, q, tq, out, ws,
                       ws_bytes, stream, false);
}

extern "C" wushkv_status wushkv_decode_step(wushkv_cache* c, int32_t layer, int32_t n_seq,
                                            const int32_t* slots, const void* k, const void* v,
                                            const float* tk, const void* q, const float* tq,
                                            float* out, void* ws, uint64_t ws_bytes,
                                            void* stream) {
  return decode_common(c, layer, n_seq, slots, k, v, tk, q, tq, out, ws, ws_bytes, stream, true);
}

extern "C" wushkv_status wushkv_decode_step_noalloc(wushkv_cache* c, int32_t layer, int32_t n_seq,
                                                    const int32_t* slots, const void* k,
                                                    const void* v, const float* tk, const void* q,
                                                    const float* tq, float* out, void* stream) {
  return decode_common(c, layer, n_seq, slots, k, v, tk, q, tq, out, nullptr, 0, stream, true,
                       true);
}

extern "C" uint64_t wushkv_chunk_workspace_bytes(const wushkv_cache* c, int32_t n_seq,
                                                  int32_t max_new) {
  if (!c || n_seq < 0 || max_new < 1 || max_new > CHUNK_MAX) return 0;
  return chunk_ws_layout(n_seq, c->cfg.n_kv_heads, c->cfg.n_q_heads / c->cfg.n_kv_heads, max_new)
      .total;
}

extern "C" wushkv_status wushkv_chunk_step(wushkv_cache* c, int32_t layer, int32_t n_seq,
                                           const int32_t* slots, const int32_t* n_new,
                                           const void* k, const void* v, const float* tk,
                                           const void* q, const float* tq, float* out, void* ws,
                                           uint64_t ws_bytes, void* stream) {
  if (!c || !slots || !n_new || layer < 0 || layer >= c->cfg.n_layers || n_seq < 0)
    return WUSHKV_EINVAL;
  if (n_seq > MAXSEQ) return WUSHKV_EUNSUPPORTED;
  if (n_seq == 0) return WUSHKV_OK;
  if (!k || !v || !tk || !q || !tq || !out || !ws) return WUSHKV_EINVAL;
  const size_t esz = c->cfg.io_dtype == WUSHKV_IO_FP32 ? 4 : 2;
  if (((uintptr_t)k % esz) || ((uintptr_t)v % esz) || ((uintptr_t)q % esz) ||
      ((uintptr_t)tk % 16) || ((uintptr_t)tq % 16) || ((uintptr_t)out % 16) || ((uintptr_t)ws % 16))
    return WUSHKV_EINVAL;
  if (!slots_ok(c, n_seq, slots)) return WUSHKV_EINVAL;
  if (c->cfg.page_size > 0 && !c->table) return WUSHKV_EINVAL;
  int C = 0, T = 0;
  for (int i = 0; i < n_seq; ++i) {
    if (n_new[i] < 1 || n_new[i] > CHUNK_MAX) return WUSHKV_EINVAL;
    const int32_t L = c->len[(size_t)layer * c->cfg.max_batch + slots[i]];
    if ((int64_t)L + n_new[i] > c->cfg.ctx_cap) return WUSHKV_ECAPACITY;
    if (n_new[i] > C) C = n_new[i];
    T += n_new[i];
  }
  const int G = c->cfg.n_q_heads / c->cfg.n_kv_heads;
  const ChunkWs wl = chunk_ws_layout(n_seq, c->cfg.n_kv_heads, G, C);
  if (ws_bytes < wl.total) return WUSHKV_EWORKSPACE;
  ChunkArgs a;
  memset(&a, 0, sizeof(a));
  a.pl = planes_of(c);
  a.g = geometry_of(c);
  a.layer = layer;
  a.n_seq = n_seq;
  a.C = C;
  a.RT = (C * G + CROWS - 1) / CROWS;
  a.n_tok = T;
  a.k = k;
  a.v = v;
  a.q = q;
  a.tk = tk;
  a.tq = tq;
  a.out = out;
  uint8_t* w = (uint8_t*)ws;
  a.qf = (float*)(w + wl.qf);
  a.qa = (uint4*)(w + wl.qa);
  a.knew = (uint16_t*)(w + wl.knew);
  a.part = (float*)(w + wl.part);
  const int S = c->cfg.sink;
  int max_sub = 0, win = 1, tok = 0;
  for (int i = 0; i < n_seq; ++i) {
    const int32_t L = c->len[(size_t)layer * c->cfg.max_batch + slots[i]];
    const int sq = squant_of(L, S, c->cfg.recent, c->cfg.flush);
    a.s.slot[i] = slots[i];
    a.s.len[i] = L;
    a.s.squant[i] = sq;
    a.s.n_new[i] = n_new[i];
    a.s.tok0[i] = tok;
    tok += n_new[i];
    const int nsub = sq > S ? (sq + CSUB - 1) / CSUB - S / CSUB : 0;
    if (nsub > max_sub) max_sub = nsub;
    const int e = (L < S ? L : S) + (L > sq ? L - sq : 0) + n_new[i];
    if (e > win) win = e;
    // positions [sq, sq1) leave the window: ring entries below L, new ones above
    const int sq1 = squant_of(L + n_new[i], S, c->cfg.recent, c->cfg.flush);
    const int nr = (sq1 < L ? sq1 : L) - sq, nw = sq1 - (sq > L ? sq : L);
    if (nr > a.n_flush_ring) a.n_flush_ring = nr;
    if (nw > a.n_flush_new) a.n_flush_new = nw;
  }
  a.win_max = win;
  const int cap = chunk_split_cap(n_seq * c->cfg.n_kv_heads * a.RT);
  const int need = (max_sub + 3) / 4;
  a.n_splits = need < cap ? need : cap;
  hipError_t e = launch_chunk(a, c->cfg.io_dtype == WUSHKV_IO_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return WUSHKV_EDEVICE;
  for (int i = 0; i < n_seq; ++i) c->len[(size_t)layer * c->cfg.max_batch + slots[i]] += n_new[i];
  return WUSHKV_OK;
}

extern "C" wushkv_status wushkv_set_block_table(wushkv_cache* c, const int32_t* table) {
  if (!c || c->cfg.page_size == 0 || !table || ((uintptr_t)table % 4)) return WUSHKV_EINVAL;
  c->table = table;
  return WUSHKV_OK;
}

extern "C" wushkv_status wushkv_set_split_events(wushkv_cache* c, void* ev_start, void* ev_stop) {
  if (!c || (!ev_start) != (!ev_stop)) return WUSHKV_EINVAL;
  c->ev_start = (hipEvent_t)ev_start;
  c->ev_stop = (hipEvent_t)ev_stop;
  return WUSHKV_OK;
}

extern "C" wushkv_status wushkv_set_combine_events(wushkv_cache* c, void* ev_start, void* ev_stop) {
  if (!c || (!ev_start) != (!ev_stop)) return WUSHKV_EINVAL;
  c->ev_cstart = (hipEvent_t)ev_start;
  c->ev_cstop = (hipEvent_t)ev_stop;
  return WUSHKV_OK;
}

extern "C" wushkv_status wushkv_stream_read_probe(const void* buf, uint64_t bytes, int32_t blocks,
                                                  void* out, void* stream) {
  if (!buf || !out || blocks < 1 || bytes < 16 || (bytes % 16) || ((uintptr_t)buf % 16) ||
      ((uintptr_t)out % 4))
    return WUSHKV_EINVAL;
  return launch_stream_read(buf, bytes, blocks, out, (hipStream_t)stream) == hipSuccess
             ? WUSHKV_OK
             : WUSHKV_EDEVICE;
}

extern "C" const char* wushkv_status_str(wushkv_status s) {
  switch (s) {
    case WUSHKV_OK: return "ok";
    case WUSHKV_EINVAL: return "invalid argument";
    case WUSHKV_ECAPACITY: return "sequence capacity exceeded";
    case WUSHKV_EWORKSPACE: return "workspace too small";
    case WUSHKV_EUNSUPPORTED: return "unsupported configuration";
    case WUSHKV_EDEVICE: return "HIP launch error";
  }
  return "unknown status";
}
