// Host-only driver of libwushkv's C ABI for AddressSanitizer and
// UndefinedBehaviorSanitizer builds (g++, no GPU): api.cpp is compiled as is
// and linked against the stub launchers below, which record each launch and
// check its arguments against the buffers the caller handed over (no kernel
// runs).  Prints "host driver OK" and exits 0 when every check holds.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../decode_attention_wushkv_amd/csrc/chunk.h"
#include "../../decode_attention_wushkv_amd/csrc/common.h"

using namespace wkv;

static int g_fail = 0;
#define CHECK(c)                                                 \
  do {                                                           \
    if (!(c)) {                                                  \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      g_fail = 1;                                                \
    }                                                            \
  } while (0)

// The fake device buffers: host memory whose addresses the stubs compare with.
static uint8_t* g_arena;
static uint64_t g_arena_bytes;
static uint8_t* g_ws;
static uint64_t g_ws_bytes;
static int g_launches;

static bool in_arena(const void* p) {
  return (const uint8_t*)p >= g_arena && (const uint8_t*)p <= g_arena + g_arena_bytes;
}
static bool in_ws(const void* p, uint64_t n) {
  return (const uint8_t*)p >= g_ws && (const uint8_t*)p + n <= g_ws + g_ws_bytes;
}

namespace wkv {
hipError_t launch_append(const AppendArgs& a, int, int grid_x, int n_seq, hipStream_t) {
  ++g_launches;
  CHECK(grid_x >= 1 && n_seq >= 1 && n_seq <= MAXSEQ);
  CHECK(in_arena(a.pl.kcode) && in_arena(a.pl.vring));
  for (int i = 0; i < n_seq; ++i) CHECK(a.s.n_new[i] >= 0 && a.s.len0[i] >= 0);
  return hipSuccess;
}
hipError_t launch_prefill(const AppendArgs& a, int grid_x, int n_seq, hipStream_t) {
  ++g_launches;
  CHECK(grid_x >= 1 && n_seq >= 1 && a.g.bits >= 2 && a.g.bits <= 4);
  return hipSuccess;
}
bool prefill_supported(int codec, double p_lo, double p_hi) {
  return codec == WUSHKV_CODEC_RMS || (p_lo <= 0.0157 && p_hi >= 0.985);
}
hipError_t launch_stream_read(const void*, uint64_t, int, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode(DecodeArgs& a, int, hipStream_t, hipEvent_t, hipEvent_t, hipEvent_t, hipEvent_t) {
  ++g_launches;
  CHECK(a.n_seq >= 1 && a.n_seq <= MAXSEQ);
  CHECK(a.n_splits >= 0 && a.n_splits <= max_chunks(a.n_seq, a.g.n_kv));
  // partials [n_seq][n_q][n_splits + 1][PS] and one query block per unit
  const uint64_t part = (uint64_t)a.n_seq * a.g.n_q * (a.n_splits + 1) * PS * 4;
  CHECK(in_ws(a.wsp, part));
  CHECK(in_ws(a.prep, (uint64_t)a.n_seq * a.g.n_kv * prep_words(a.g.G) * 4));
  for (int i = 0; i < a.n_seq; ++i) {
    // S_quant starts at the sink and never passes the length beyond it
    CHECK(a.s.squant[i] >= a.g.S);
    CHECK(a.s.len[i] >= 1 && a.s.squant[i] <= (a.s.len[i] > a.g.S ? a.s.len[i] : a.g.S));
  }
  return hipSuccess;
}
hipError_t launch_chunk(ChunkArgs& a, int, hipStream_t) {
  ++g_launches;
  CHECK(a.n_seq >= 1 && a.C >= 1 && a.C <= CHUNK_MAX);
  const ChunkWs w = chunk_ws_layout(a.n_seq, a.g.n_kv, a.g.G, a.C);
  CHECK(in_ws(a.part, w.total - w.part));
  CHECK(a.n_splits >= 0 && a.n_splits <= chunk_split_cap(a.n_seq * a.g.n_kv * a.RT));
  return hipSuccess;
}
// The no-allocation entry point's scratch: a host buffer stands in.
static uint8_t* g_scratch;
hipError_t noalloc_scratch(void** ptr, uint64_t* bytes) {
  *ptr = g_scratch;
  *bytes = WUSHKV_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}
}  // namespace wkv

static wushkv_config cfg_of(int bits, int G, int page) {
  wushkv_config c;
  memset(&c, 0, sizeof(c));
  c.n_layers = 3;
  c.n_kv_heads = 2;
  c.n_q_heads = 2 * G;
  c.head_dim = 128;
  c.bits = bits;
  c.sink = 4;
  c.recent = 32;
  c.flush = 3;
  c.p_lo = 0.01;
  c.p_hi = 0.99;
  c.max_batch = 5;
  c.ctx_cap = 700;
  c.io_dtype = WUSHKV_IO_BF16;
  c.page_size = page;
  c.n_pages = page ? 40 : 0;
  return c;
}

static void run(int bits, int G, int page) {
  wushkv_config c = cfg_of(bits, G, page);
  wushkv_layout_t lay;
  CHECK(wushkv_layout(&c, &lay) == WUSHKV_OK);
  // an arena in host memory stands in for the device one (never dereferenced
  // by the library's host code)
  std::vector<uint8_t> arena(lay.total_bytes + 256);
  g_arena = (uint8_t*)(((uintptr_t)arena.data() + 255) & ~(uintptr_t)255);
  g_arena_bytes = lay.total_bytes;
  wushkv_cache* h = nullptr;
  CHECK(wushkv_cache_create(&c, g_arena, g_arena_bytes, &h) == WUSHKV_OK);
  std::vector<int32_t> table(5 * (size_t)(lay.pages_per_seq + 1), 0);
  if (page) {
    CHECK(wushkv_append(h, 0, 0, nullptr, nullptr, 0, 0, 0, 0) == WUSHKV_EINVAL);
    CHECK(wushkv_set_block_table(h, table.data()) == WUSHKV_OK);
  }
  const float* tk = (const float*)(g_arena + 16);  // any aligned address
  int32_t slots[3] = {0, 2, 4}, n_new[3] = {300, 0, 17};
  CHECK(wushkv_append(h, 1, 3, slots, n_new, g_arena, g_arena, tk, 0) == WUSHKV_OK);
  int32_t L = -1, sq = -1;
  CHECK(wushkv_get_len(h, 1, 0, &L, &sq) == WUSHKV_OK && L == 300 && sq == 4 + 3 * 88);
  int32_t b = 0, e = 0;
  CHECK(wushkv_quantized_range(h, 300, &b, &e) == WUSHKV_OK && b == 4 && e == sq);
  // decode needs L >= 1 in every named slot
  const uint64_t ws = wushkv_decode_workspace_bytes(h, 3);
  std::vector<uint8_t> wsbuf(ws + 16);
  g_ws = (uint8_t*)(((uintptr_t)wsbuf.data() + 15) & ~(uintptr_t)15);
  g_ws_bytes = ws;
  float* out = (float*)g_arena;
  CHECK(wushkv_decode_attn(h, 1, 3, slots, g_arena, tk, out, g_ws, ws, 0) == WUSHKV_EINVAL);
  int32_t two[2] = {0, 4};
  CHECK(wushkv_decode_attn(h, 1, 2, two, g_arena, tk, out, g_ws, ws, 0) == WUSHKV_OK);
  CHECK(wushkv_decode_attn(h, 1, 2, two, g_arena, tk, out, g_ws, ws - 1, 0) ==
        (ws - 1 < wushkv_decode_workspace_bytes(h, 2) ? WUSHKV_EWORKSPACE : WUSHKV_OK));
  for (int st = 0; st < 40; ++st)
    CHECK(wushkv_decode_step(h, 1, 3, slots, g_arena, g_arena, tk, g_arena, tk, out, g_ws, ws,
                             0) == WUSHKV_OK);
  CHECK(wushkv_get_len(h, 1, 2, &L, &sq) == WUSHKV_OK && L == 40);
  // the same steps with the library's scratch as workspace
  std::vector<uint8_t> scratch(WUSHKV_NOALLOC_SCRATCH_BYTES + 256);
  g_scratch = (uint8_t*)(((uintptr_t)scratch.data() + 255) & ~(uintptr_t)255);
  g_ws = g_scratch;
  g_ws_bytes = WUSHKV_NOALLOC_SCRATCH_BYTES;
  CHECK(wushkv_decode_step_noalloc(h, 1, 3, slots, g_arena, g_arena, tk, g_arena, tk, out, 0) ==
        WUSHKV_OK);
  CHECK(wushkv_get_len(h, 1, 2, &L, &sq) == WUSHKV_OK && L == 41);
  int32_t dup[2] = {2, 2};
  CHECK(wushkv_decode_step_noalloc(h, 1, 2, dup, g_arena, g_arena, tk, g_arena, tk, out, 0) ==
        WUSHKV_EINVAL);
  CHECK(wushkv_decode_step_noalloc(h, 1, 3, slots, g_arena, g_arena, tk, nullptr, tk, out, 0) ==
        WUSHKV_EINVAL);
  // chunk steps
  const uint64_t cws = wushkv_chunk_workspace_bytes(h, 3, 16);
  std::vector<uint8_t> cbuf(cws + 16);
  g_ws = (uint8_t*)(((uintptr_t)cbuf.data() + 15) & ~(uintptr_t)15);
  g_ws_bytes = cws;
  int32_t cn[3] = {16, 1, 9};
  CHECK(wushkv_chunk_step(h, 1, 3, slots, cn, g_arena, g_arena, tk, g_arena, tk, out, g_ws, cws,
                          0) == WUSHKV_OK);
  int32_t big[3] = {17, 1, 1};
  CHECK(wushkv_chunk_step(h, 1, 3, slots, big, g_arena, g_arena, tk, g_arena, tk, out, g_ws, cws,
                          0) == WUSHKV_EINVAL);
  // capacity: 700 positions per slot
  int32_t one[1] = {0}, many[1] = {1000};
  CHECK(wushkv_append(h, 1, 1, one, many, g_arena, g_arena, tk, 0) == WUSHKV_ECAPACITY);
  CHECK(wushkv_reset_seq(h, 0) == WUSHKV_OK);
  CHECK(wushkv_get_len(h, 1, 0, &L, &sq) == WUSHKV_OK && L == 0 && sq == 4);
  CHECK(wushkv_get_len(h, 3, 0, &L, &sq) == WUSHKV_EINVAL);
  CHECK(wushkv_stream_read_probe(g_arena, 4096, 4, g_arena, 0) == WUSHKV_OK);
  wushkv_cache_destroy(h);
}

int main() {
  for (int bits = 2; bits <= 4; ++bits)
    for (int G : {1, 2, 4, 8})
      for (int page : {0, 128}) run(bits, G, page);
  for (int s = 0; s <= 6; ++s) CHECK(wushkv_status_str((wushkv_status)s) != nullptr);
  CHECK(wushkv_gaussian_alpha(2) > 1.49 && wushkv_gaussian_alpha(2) < 1.50);
  CHECK(wushkv_gaussian_alpha(0) == 0.0);
  wushkv_config bad = cfg_of(5, 1, 0);
  CHECK(wushkv_config_check(&bad) == WUSHKV_EUNSUPPORTED);
  CHECK(g_launches > 0);
  if (g_fail) return 1;
  printf("host driver OK (%d launches recorded)\n", g_launches);
  return 0;
}
