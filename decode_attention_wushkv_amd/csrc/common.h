// Internal definitions shared by the libwushkv kernels and host code.
// gfx950 (CDNA4) only: wave64, HIP runtime.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wushkv.h"

namespace wkv {

constexpr int D = 128;          // head_dim (the only one built)
constexpr int MAXSEQ = 128;     // sequences per call (kernel-argument tables)
constexpr int WINDOW_MAX = 1024; // sink + ring entries scored by one workgroup
constexpr int CHUNK = 256;       // prefill append: positions per workgroup (multiple of vblock)

// Decode sub-chunk of one wave: 128 positions at 2 bits, 64 at 3 and 4 bits
// (whole 16-byte value rows; at 3 bits half of a block's high-plane row).
__host__ __device__ constexpr int sub_len(int bits) { return bits == 2 ? 128 : 64; }

// 3-bit codes are stored as two bit planes: the low two bits of every code in
// the 2-bit packing, and the high bit in a 1-bit plane where bit 4 n + k of
// 32-bit word j holds element 32 j + 16 (k >> 1) + 2 n + (k & 1) (element =
// dimension of a key row, position of a value row).  Then (word >> k) &
// 0x11111111 lines up nibble for nibble with the even (k even) or odd (k odd)
// elements of 2-bit word 2 j + (k >> 1), which the decode kernels unpack as
// (w & 0x33333333) and ((w >> 2) & 0x33333333).  hi_bit(e) is the bit of
// element e (0 <= e < 128) in its 128-bit high plane.
__host__ __device__ constexpr int hi_bit(int e) {
  return 32 * (e >> 5) + 4 * ((e & 15) >> 1) + ((((e & 31) >> 4) << 1) | (e & 1));
}
// Upper bound on workgroups per (sequence, KV head) in one decode call (the
// host picks the actual count from the GPU's occupancy); sizes the workspace.
__host__ __device__ inline int max_chunks(int n_seq, int n_kv) {
  int u = n_seq * n_kv;
  int c = (4096 + u - 1) / u;
  return c < 64 ? c : 64;
}

// Fixed-point precision of the decode dot products: the compensated query
// is held as QDIG signed base-16 digits (24 bits) and the softmax weights of
// a 128-position sub-chunk as WDIG unsigned ones (16 bits).  A score's error
// is the query's rounding error dotted with the key's codes times its scale,
// so it grows with the key's range; 16-bit queries exceeded the 2e-3 output
// bar on keys scaled x30 or holding constant rows of 1024, and 20-bit ones on
// 4-bit RMS-coded groups around 1024 (2.1 times the bar); 24 bits keep every
// tested case below a third of it.
constexpr int QDIG = 6;
constexpr int WDIG = 4;
constexpr int DIGP = 8;  // query digit words per group of 8 dimensions (padded for 16-byte loads)

// 32-bit words of one (sequence, KV head) query block: q' [G][D] floats,
// scales [G][4], digit words [G][16][DIGP] (in the split kernel's LDS order),
// then the decode step's new key and value as bfloat16 (D words).
__host__ __device__ constexpr int prep_words(int G) { return G * (D + 4 + 16 * DIGP) + D; }


constexpr int PS = 132;          // workspace stride of one split partial: o[128], m, l, pad

// Base addresses of the cache planes (arena + layout offsets).
struct Planes {
  uint8_t* kcode;
  uint8_t* vcode;
  uint32_t* ksz;   // {binary16 scale | binary16 zero << 16}
  uint32_t* vsz;
  uint16_t* ksink;  // bfloat16 bits
  uint16_t* vsink;
  uint16_t* kring;
  uint16_t* vring;
};

struct Geometry {
  int n_kv, n_q, G, bits;
  int S, R, F, W;  // sink, recent, flush, ring slots
  int code_bytes, vblock, ctx_blocks, cpos, max_batch;
  double p_lo, p_hi;
  int codec;     // WUSHKV_CODEC_PERCENTILE or WUSHKV_CODEC_RMS
  double alpha;  // RMS codec endpoint (resolved)
  // Quantized planes.  Contiguous: a unit's positions are rows unit * cpos +
  // p.  Paged: rows ((layer * n_pages + page) * n_kv + head) << page_shift +
  // (p & (page - 1)) with page = table[slot * pps + (p >> page_shift)].
  const int32_t* table;  // block table [max_batch][pps] (device); null when contiguous
  int pps, page_shift, n_pages;
};

// Where the quantized planes keep one (layer, sequence, KV head): position p
// is row r of kcode (bytes r * code_bytes), ksz and vsz, and its value codes
// lie in block r / vblock of vcode (one 16-byte row per dimension at 2 and 4
// bits; at 3 bits two low-plane rows and one high-plane row).  A page (at
// least 128 positions, a power of two) holds whole decode sub-chunks and
// value-code blocks.
struct QMap {
  const int32_t* pages;  // the sequence's block-table row; null when contiguous
  int64_t base;          // row of position 0 (contiguous) or of physical page 0 (paged)
  int64_t stride;        // rows from one physical page to the next (paged)
  int shift, n_pages;
};

__host__ __device__ inline QMap qmap_of(const Geometry& g, int layer, int slot, int head) {
  QMap m;
  m.shift = g.page_shift;
  m.n_pages = g.n_pages;
  if (g.table) {
    m.pages = g.table + (int64_t)slot * g.pps;
    m.stride = (int64_t)g.n_kv << g.page_shift;
    m.base = ((int64_t)layer * g.n_pages * g.n_kv + head) << g.page_shift;
  } else {
    m.pages = nullptr;
    m.stride = 0;
    m.base = (((int64_t)layer * g.max_batch + slot) * g.n_kv + head) * g.cpos;
  }
  return m;
}

// Row of position p; -1 when the block table maps no page of the pool there
// (writers then skip the position).
__device__ __forceinline__ int64_t qrow(const QMap& m, int p) {
  if (!m.pages) return m.base + p;
  const int pg = m.pages[p >> m.shift];
  if ((unsigned)pg >= (unsigned)m.n_pages) return -1;
  return m.base + pg * m.stride + (p & ((1 << m.shift) - 1));
}

// Row of position p for reads: an unmapped page reads the pool's first page
// (results for that sequence are then unspecified, but no access leaves the
// arena).
__device__ __forceinline__ int64_t qrow_read(const QMap& m, int p) {
  const int64_t r = qrow(m, p);
  return r >= 0 ? r : (int64_t)(p & ((1 << m.shift) - 1));
}

// squant(L): end of the quantized region [S, squant) at length L (section 4.4).
__host__ __device__ inline int squant_of(int L, int S, int R, int F) {
  int outside = L - R - S;
  if (outside < 0) outside = 0;
  return S + F * (outside / F);
}

struct AppendSeqs {
  int32_t slot[MAXSEQ];
  int32_t len0[MAXSEQ];   // length before this call
  int32_t n_new[MAXSEQ];
  int32_t tok0[MAXSEQ];   // first row of this sequence in k / v
};

enum AppendMode : int { APPEND_FUSED = 0, APPEND_EVICT = 1, APPEND_CHUNKED = 2 };

struct AppendArgs {
  Planes pl;
  Geometry g;
  int layer;
  int mode;
  const void* k;
  const void* v;
  const float* tk;
  AppendSeqs s;
};

struct DecodeSeqs {
  int32_t slot[MAXSEQ];
  int32_t len[MAXSEQ];
  int32_t squant[MAXSEQ];
  // Balanced grid (DecodeArgs::balanced): the quantized workgroups of
  // sequence i are grid blocks units + [wg0[i], wg0[i + 1]), KV head by KV
  // head, (wg0[i + 1] - wg0[i]) / n_kv per head
  int32_t wg0[MAXSEQ + 1];
};

struct DecodeArgs {
  Planes pl;
  Geometry g;
  int layer;
  int n_seq;
  int n_splits;  // workgroups over the quantized region per (sequence, KV head), plus one window workgroup
  // Block order of the 1-D grid (window workgroups first in both): 0 =
  // unit-major; 1 = XCD-affine (block b runs on XCD b % 8, so unit u takes the
  // blocks with b % 8 == u % 8 and all of a unit's workgroups share one L2).
  // Requires units % 8 == 0.
  int xcd_map;
  // Sub-chunk assignment: 0 = wave k of a unit takes sub-chunks k, k + nw,
  // k + 2 nw, ... (nw waves per unit); 1 = each wave takes one contiguous run;
  // 2 = each workgroup takes one contiguous run, which its four waves share
  // out in turn (k, k + 4, ...).  With the head split (G >= 4) 1 and 2 both
  // give each workgroup one run.
  int contig;
  // Groups of 4 and 8 (the matrix-core path): window workgroups first, then
  // each sequence's KV heads get quantized workgroups in proportion to their
  // sub-chunks (s.wg0); n_splits is the largest count per head, and also the
  // window partial's index
  int balanced;
  const void* q;
  const float* tq;
  float* out;
  float* wsp;     // [n_seq][n_q][n_splits + 1][PS]
  // Per (sequence, KV head) query block written by the prep kernel:
  // prep_words(G) words (q' floats, scales, digit words, new entry).
  uint32_t* prep;
  // Quantized sub-chunks of the launch: most in one unit, and the total over
  // units (the launcher's choice of query preparation and grid size).
  int max_sub;
  int64_t total_sub;
  // Decode step (fused one-token append): the new key and value rows
  // [n_seq][n_kv][D] in the io dtype and T_K [n_kv][D][D].  Null k_new means
  // attention only.  In a step, s.len is the length with the new position and
  // s.squant the quantized boundary before it (the window holds the new entry
  // in full precision; the flush follows the attention).
  const void* k_new;
  const void* v_new;
  const float* tk;
  DecodeSeqs s;
};

// Host-side launchers (defined in the .hip files); return hipSuccess or the
// launch error.
hipError_t launch_append(const AppendArgs& a, int io_bf16, int grid_x, int n_seq, hipStream_t st);
// Prefill kernel (bfloat16 inputs): workgroups of PREFILL_SPAN positions per
// (sequence, KV head), in tiles aligned to PREFILL_TILE; grid_x covers the
// longest run of new positions.  prefill_supported() tells whether the clip
// percentiles need only the three smallest and three largest values.
constexpr int PREFILL_TILE = 64;
constexpr int PREFILL_SPAN = 1024;
hipError_t launch_prefill(const AppendArgs& a, int grid_x, int n_seq, hipStream_t st);
bool prefill_supported(int codec, double p_lo, double p_hi);
hipError_t launch_stream_read(const void* buf, uint64_t bytes, int blocks, void* out, hipStream_t st);
hipError_t launch_decode(DecodeArgs& a, int io_bf16, hipStream_t st, hipEvent_t ev_start,
                         hipEvent_t ev_stop, hipEvent_t ev_cstart, hipEvent_t ev_cstop);
// Device address and size of the current device's file-scope scratch array
// (wushkv_decode_step_noalloc's workspace).
hipError_t noalloc_scratch(void** ptr, uint64_t* bytes);

}  // namespace wkv
