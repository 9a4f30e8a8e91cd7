// Chunked multi-query step (wushkv_chunk_step): shapes, workspace layout and
// launcher shared by api.cpp and chunk.hip.
#pragma once

#include "common.h"

namespace wkv {

constexpr int CHUNK_MAX = 16;   // new positions per sequence in one chunk step
constexpr int CSUB = 64;        // positions per quantized sub-chunk (one 2-bit value row)
constexpr int CROWS = 16;       // query rows per row tile (one 16x16x64 int8 MFMA tile)

struct ChunkSeqs {
  int32_t slot[MAXSEQ];
  int32_t len[MAXSEQ];     // length before the chunk
  int32_t squant[MAXSEQ];  // squant(len): the quantized boundary the chunk attends with
  int32_t n_new[MAXSEQ];   // chunk positions of the sequence (1 .. CHUNK_MAX)
  int32_t tok0[MAXSEQ];    // first row of the sequence in k, v, q and out
};

// Rows of one (sequence, KV head): row = c * G + g for chunk position c and
// query head g of the KV head's group; rows/CROWS tiles, the last one padded.
struct ChunkArgs {
  Planes pl;
  Geometry g;
  // positions leaving the window per (sequence, KV head), at most: ring entries
  // (quantized in the prep launch) and new entries (in a launch of their own)
  int layer, n_seq, C, RT, n_splits, xcd_map, n_tok, win_max, n_flush_ring, n_flush_new;
  const void* k;
  const void* v;
  const void* q;
  const float* tk;
  const float* tq;
  float* out;
  float* qf;       // [n_seq][n_kv][C G][D + 4]: q' (log2 domain), sigma, 1/S_q, 0
  uint4* qa;       // [n_seq][n_kv][RT][2 halves of d][3 digits][64 lanes]: int8 A operands
  uint16_t* knew;  // [n_seq][C][n_kv][2][D]: new entries as bfloat16 bits (T_K k, v)
  float* part;     // [n_seq][n_kv][RT][NP][CROWS][PS] partials, NP = 4 n_splits + 1
  ChunkSeqs s;
};

// Workgroups over the quantized region per (sequence, KV head, row tile):
// at most this many (sizes the workspace).
inline int chunk_split_cap(int tiles) {
  int c = (4096 + tiles - 1) / tiles;
  return c < 64 ? c : 64;
}

struct ChunkWs {
  uint64_t qf, qa, knew, part, total;  // byte offsets and size
};

inline ChunkWs chunk_ws_layout(int n_seq, int n_kv, int G, int C) {
  auto al = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
  const uint64_t units = (uint64_t)n_seq * n_kv;
  const int rt = (C * G + CROWS - 1) / CROWS;
  const uint64_t np = 4 * (uint64_t)chunk_split_cap((int)(units * rt)) + 1;
  ChunkWs w;
  w.qf = 0;
  w.qa = al(w.qf + units * C * G * (D + 4) * 4);
  w.knew = al(w.qa + units * rt * 6 * 64 * 16);
  w.part = al(w.knew + units * C * 2 * D * 2);
  w.total = al(w.part + units * rt * np * CROWS * PS * 4);
  return w;
}

// Launches the four kernels of a chunk step (query preparation, attention,
// flush, merge + stores); a.n_splits is the requested count, capped by
// occupancy.
hipError_t launch_chunk(ChunkArgs& a, int io_bf16, hipStream_t st);

}  // namespace wkv
