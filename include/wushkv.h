/*
 * wushkv.h -- C ABI of libwushkv: the WUSH-KV transformed low-bit KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * The method ("WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms",
 * paper page) stores, per KV head, one cache column per position (section
 * 4.1).  Keys arrive after RoPE and are multiplied by a fixed d x d key
 * transform T_K before caching; queries are compensated by T_K^{-T} (section
 * 4.2, appendix B.1).  Values arrive already in the value transform's basis,
 * which is folded into the projection weights (section 4.5), so the
 * attention output also leaves in that basis.  Cached entries outside a fixed
 * sink window and a rolling recent window (section 4.4) are quantized per
 * token with percentile clipping and asymmetric affine scaling (section 5.3;
 * 2^b equally spaced levels, appendix B.3).
 *
 * Two operations carry the method: wushkv_append (transform + window
 * placement + quantize/pack) and wushkv_decode_attn (query compensation +
 * split-K decode attention over the mixed cache + merge).  Everything else
 * here is layout, bookkeeping and error reporting.
 *
 * Conventions for every call:
 *   - Device pointers are HIP device addresses on the current device; host
 *     pointers are ordinary process memory.  Nothing is retained after a call
 *     returns except by wushkv_cache_create (the arena address).
 *   - The library never allocates device memory.  The caller owns the arena,
 *     every input/output buffer and the decode workspace.
 *   - All argument checks happen before any kernel launch; a call that returns
 *     an error has changed no state (host lengths, device memory).
 *   - Kernels are enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and run asynchronously; the library does no host
 *     synchronisation.  One cache must not be used from two streams at once.
 *   - No C++ exception crosses this interface.
 */
#ifndef WUSHKV_H
#define WUSHKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WUSHKV_OK = 0,
  WUSHKV_EINVAL = 1,       /* null/misaligned pointer, index out of range, duplicate slot, bad config value */
  WUSHKV_ECAPACITY = 2,    /* an append would make a sequence longer than ctx_cap */
  WUSHKV_EWORKSPACE = 3,   /* decode workspace smaller than wushkv_decode_workspace_bytes() */
  WUSHKV_EUNSUPPORTED = 4, /* valid but not built: head_dim != 128, bits not in {2, 3, 4}, too many sequences per call */
  WUSHKV_EDEVICE = 5       /* the HIP runtime reported an error when launching */
} wushkv_status;

enum { WUSHKV_IO_FP32 = 0, WUSHKV_IO_BF16 = 1 };

/* Clip ends of a quantization group (one position's 128 key or value
 * entries):
 *   PERCENTILE  lo, hi = the p_lo and p_hi linear-interpolation percentiles of
 *               the group (asymmetric, adaptive zero point; paper section 5.3).
 *   RMS         lo, hi = -alpha * rms, +alpha * rms with rms the group's root
 *               mean square: the QuEST-style symmetric grid of 2^b levels from
 *               -alpha to alpha on the RMS-normalized group (paper appendix
 *               B.3); alpha defaults to the endpoint minimizing the
 *               mean-squared error for a standard Gaussian.
 * Both store s = (hi - lo)/(2^b - 1) and z = lo in binary16 and the level
 * nearest to (x - z16)/s16, so decoding is the same for both. */
enum { WUSHKV_CODEC_PERCENTILE = 0, WUSHKV_CODEC_RMS = 1 };

/* Largest number of sequences one append or decode call may name. */
#define WUSHKV_MAX_SEQ_PER_CALL 128

/* Fixed at cache creation. */
typedef struct {
  int32_t n_layers;     /* attention modules sharing this cache object            */
  int32_t n_q_heads;    /* query heads; query head j reads KV head j / (n_q/n_kv) */
  int32_t n_kv_heads;   /* KV heads (n_q_heads % n_kv_heads == 0)                 */
  int32_t head_dim;     /* d; must be 128                                         */
  int32_t bits;         /* code width b: 2, 3 or 4                                */
  int32_t sink;         /* S_sink >= 0: first positions kept in bfloat16          */
  int32_t recent;       /* S_keep >= 0: newest positions kept in bfloat16         */
  int32_t flush;        /* S_flush >= 1: quantize in multiples of this            */
  double p_lo, p_hi;    /* clip percentiles, 0 <= p_lo < p_hi <= 1 (e.g. .01/.99) */
  int32_t max_batch;    /* sequence slots                                         */
  int32_t ctx_cap;      /* positions per slot (>= 1)                              */
  int32_t io_dtype;     /* WUSHKV_IO_FP32 or WUSHKV_IO_BF16 for k, v, q inputs   */
  int32_t codec;        /* WUSHKV_CODEC_PERCENTILE (0) or WUSHKV_CODEC_RMS       */
  double clip_alpha;    /* RMS codec endpoint; 0 = wushkv_gaussian_alpha(bits)   */
  int32_t page_size;    /* 0: contiguous quantized planes per slot; else paged:  */
                        /* positions per page, a power of two in [128, 2^20]    */
  int32_t n_pages;      /* paged: physical pages per layer in the pool (>= 1);  */
                        /* contiguous: must be 0                                */
} wushkv_config;

/*
 * Device layout of one cache.  All planes live in one caller-allocated
 * arena; offsets are bytes from the arena start, each a multiple of 256.
 * A "unit" is one (layer, slot, KV head): u = (layer * max_batch + slot) *
 * n_kv_heads + head.  Positions p are absolute (0-based) in the sequence.
 *
 *   kcode  uint8  [unit][cpos][code_bytes]         token-major key codes;
 *                 bits 2, 4: element i of position p sits in byte (i*bits)/8
 *                 at bit (i*bits)%8 of that position's code_bytes = d*bits/8
 *                 bytes.
 *   vcode  uint8  [unit][ctx_blocks][d][16]        value codes, dim-major per
 *                 block of vblock = 128/bits positions (bits 2, 4): element i
 *                 of position p sits in row i of block p/vblock, byte
 *                 ((p%vblock)*bits)/8, bit ((p%vblock)*bits)%8.
 *
 * 3-bit codes (the paper evaluates 2, 3 and 4 bits, section 5.2; appendix
 * B.3 for the 2^b levels) are stored as two bit planes.  The low plane holds
 * the low two bits of every code in the 2-bit packing, the high plane the
 * third bit in the order hi(e) = 32 (e / 32) + 4 ((e % 16) / 2) +
 * 2 ((e % 32) / 16) + e % 2: element e's bit is bit hi(e) % 32 of 32-bit word
 * hi(e) / 32 of a 16-byte high-plane row.
 *   kcode  [unit][cpos][48]: bytes 0..31 the low plane of the 128 elements,
 *          bytes 32..47 their high plane (code_bytes = 48).
 *   vcode  [unit][ctx_blocks][3][d][16] with vblock = 128 positions: per
 *          dimension, low-plane rows of positions 0..63 and 64..127 of the
 *          block (2-bit packing), then the high-plane row of the block's 128
 *          positions (element = position in the block).
 *   ksz,vsz uint16[unit][cpos][2]                  binary16 {scale, zero} of
 *                 the key / value group of each quantized position.
 *   ksink,vsink bfloat16 [unit][sink][d]           positions [0, sink).
 *   kring,vring bfloat16 [unit][ring_slots][d]     recent window; position p
 *                 (p >= sink) lives in slot (p - sink) % ring_slots.
 *
 * Paged caches (page_size P > 0) keep the quantized planes (kcode, vcode,
 * ksz, vsz) in a pool of n_pages physical pages per layer, each holding P
 * positions of every KV head, the form of the paged KV caches of the serving
 * system the paper integrates the method into (paper page, section 2 on
 * SGLang's paged caches; section 5.3 for the integration):
 *
 *   kcode  uint8  [layer][page][head][P][code_bytes]
 *   vcode  uint8  [layer][page][head][P/vblock][d][16]
 *   ksz,vsz uint16[layer][page][head][P][2]
 *
 * Position p of slot s lives at offset p % P of physical page
 * table[s][p / P] of the block table bound with wushkv_set_block_table (the
 * same page in every layer).  Windows (sink, ring) stay per slot as above.
 *
 * Keys in the cache are in the transformed basis (T_K k, rounded to bfloat16
 * before quantization); values are as given (rounded to bfloat16).  After a
 * sequence reaches length L, positions [sink, squant(L)) are quantized and
 * [squant(L), L) are in the ring, with squant(L) = sink + flush *
 * floor(max(0, L - recent - sink) / flush) (section 4.4; S_quant starts at
 * sink for an empty cache).  Entries of a code plane at positions that are not
 * quantized hold unspecified bits.
 */
typedef struct {
  uint64_t total_bytes;
  uint64_t off_kcode, off_vcode, off_ksz, off_vsz, off_ksink, off_vsink, off_kring, off_vring;
  uint64_t bytes_kcode, bytes_vcode, bytes_ksz, bytes_vsz, bytes_ksink, bytes_vsink,
      bytes_kring, bytes_vring;
  int32_t code_bytes;   /* d * bits / 8 per position per K (or V)   */
  int32_t vblock;       /* positions per value-code block = 128/bits */
  int32_t ctx_blocks;   /* cpos / vblock                             */
  int32_t cpos;         /* positions per unit: ctx_cap rounded up to 128 */
  int32_t ring_slots;   /* recent + flush - 1                        */
  int32_t units;        /* n_layers * max_batch * n_kv_heads         */
  int32_t page_size;    /* paged: P; contiguous: 0                   */
  int32_t n_pages;      /* paged: physical pages per layer; else 0   */
  int32_t pages_per_seq; /* paged: block-table row length ceil(ctx_cap / P); else 0 */
} wushkv_layout_t;

typedef struct wushkv_cache wushkv_cache;

/* The endpoint alpha minimizing E[(x - Q_alpha(x))^2] for x ~ N(0, 1), with
 * Q_alpha rounding to the nearest of 2^bits equally spaced levels from -alpha
 * to alpha (paper appendix B.3's optimal endpoint); computed on the host to
 * about 1e-12.  0 for bits outside 1..8. */
double wushkv_gaussian_alpha(int32_t bits);

/* Check a config.  Host only.  EINVAL / EUNSUPPORTED as described above. */
wushkv_status wushkv_config_check(const wushkv_config* cfg);

/* Fill *out with the arena layout for cfg (host only, no device calls). */
wushkv_status wushkv_layout(const wushkv_config* cfg, wushkv_layout_t* out);

/* Bind a cache descriptor to a device arena of at least layout.total_bytes,
 * 256-byte aligned (EINVAL otherwise).  The arena needs no initialisation.
 * All sequence lengths start at 0.  *out is owned by the caller and released
 * with wushkv_cache_destroy; the arena stays the caller's. */
wushkv_status wushkv_cache_create(const wushkv_config* cfg, void* arena, uint64_t arena_bytes,
                                  wushkv_cache** out);
void wushkv_cache_destroy(wushkv_cache* cache);

/*
 * Paged caches only (EINVAL otherwise, or for a null or unaligned table):
 * bind the block table, device int32 [max_batch][pages_per_seq].  Entry
 * [s][i] names the physical page (0 <= id < n_pages) that holds positions
 * [i P, (i + 1) P) of slot s in every layer.  Kernels read the table when
 * they run, in stream order, so the caller may change entries between calls
 * with stream-ordered copies; the table must stay allocated while calls that
 * use it are in flight.  Before a call, every page holding a position that
 * the call quantizes (positions of [sink, squant(L')) it writes) or that
 * attention reads (positions of [sink, squant(L))) must be mapped, and two
 * slots must not map the same page.  Entries of pages without such positions
 * are not read.  An out-of-range entry makes the library skip the writes to
 * that page and read the pool's first page instead: the results for that
 * sequence are then unspecified, but no access leaves the arena.  Host only;
 * append and decode calls on a paged cache with no table return EINVAL.
 */
wushkv_status wushkv_set_block_table(wushkv_cache* cache, const int32_t* table);

/* Forget slot's contents in every layer (length 0; S_quant back to sink). */
wushkv_status wushkv_reset_seq(wushkv_cache* cache, int32_t slot);

/* Host-side length L of (layer, slot) and its quantized-region end squant(L). */
wushkv_status wushkv_get_len(const wushkv_cache* cache, int32_t layer, int32_t slot,
                             int32_t* len, int32_t* squant);

/* Host only.  The positions [*begin, *end) that are quantized once a sequence
 * of this cache reaches length len >= 0 (paper page, section 4.4: the sink
 * and the newest positions stay in full precision; the region grows in
 * multiples of S_flush): *begin = sink and *end = squant(len) (*end ==
 * *begin when nothing is quantized).  A paged cache's caller maps the pages
 * that hold [*begin, *end) of the length a call leaves before making it (see
 * wushkv_set_block_table).  EINVAL for a null argument or len < 0. */
wushkv_status wushkv_quantized_range(const wushkv_cache* cache, int32_t len, int32_t* begin,
                                     int32_t* end);

/*
 * Append n_new[i] >= 0 positions to sequence slots[i] (distinct, i < n_seq <=
 * WUSHKV_MAX_SEQ_PER_CALL) of one layer.  Section 4.4: new entries are first
 * rounded to bfloat16; positions that leave the recent window (old ring
 * entries or new ones) are quantized, in the order they become eligible.
 *
 *   k   device, io_dtype [sum(n_new)][n_kv_heads][head_dim]: post-RoPE keys,
 *       the sequences' tokens concatenated in the order of slots[].
 *   v   device, same shape: values, already in the value transform's basis.
 *   tk  device, float32 [n_kv_heads][d][d] row-major: k'_i = sum_j tk[i][j] k_j
 *       (the key transform T_K of this layer).
 * The transform is evaluated to fp64 accuracy before rounding to bfloat16.
 * ECAPACITY if any L + n_new > ctx_cap.  Updates the host lengths on success.
 */
wushkv_status wushkv_append(wushkv_cache* cache, int32_t layer, int32_t n_seq, const int32_t* slots,
                            const int32_t* n_new, const void* k, const void* v, const float* tk,
                            void* stream);

/* Bytes of device workspace wushkv_decode_attn needs for n_seq sequences. */
uint64_t wushkv_decode_workspace_bytes(const wushkv_cache* cache, int32_t n_seq);

/*
 * One decode query per query head for each of n_seq sequences (distinct
 * slots, each with length >= 1) of one layer, attending to all L cached
 * positions of its sequence (section 4.1, GQA: query head j reads KV head
 * j / (n_q/n_kv); the newest position is in the cache, so no mask applies).
 *
 *   q    device, io_dtype [n_seq][n_q_heads][d]: post-RoPE, uncompensated.
 *   tq   device, float32 [n_kv_heads][d][d] row-major, = T_K^{-T}:
 *        q'_i = sum_j tq[i][j] q_j.
 *   out  device, float32 [n_seq][n_q_heads][d]: softmax(q'.k / sqrt(d)) v over
 *        the cache, in the value-transform basis (window entries read as
 *        stored bfloat16, quantized entries as z16 + s16 * code).
 *   ws   device workspace of ws_bytes >= wushkv_decode_workspace_bytes(),
 *        16-byte aligned; contents on entry are ignored.
 */
wushkv_status wushkv_decode_attn(wushkv_cache* cache, int32_t layer, int32_t n_seq,
                                 const int32_t* slots, const void* q, const float* tq, float* out,
                                 void* ws, uint64_t ws_bytes, void* stream);

/*
 * One decode step of one layer for n_seq sequences (distinct slots, each with
 * length L >= 0 and L + 1 <= ctx_cap): append one new position per sequence
 * and attend the queries to all L + 1 positions, in the order of section 4.4
 * -- the new entry is attended in full precision together with the recent
 * window, and the window is flushed afterwards.  The attention therefore sees
 * squant(L) as its quantized boundary (L + 1 - squant(L) <= recent + flush
 * bfloat16 window entries plus the sink), and the cache left behind is the
 * one wushkv_append with n_new = 1 would leave (boundary squant(L + 1)).
 * Equivalent to wushkv_append with recent + 1 followed by wushkv_decode_attn,
 * in two kernel launches.
 *
 *   k, v  device, io_dtype [n_seq][n_kv_heads][d]: the new position's
 *         post-RoPE key and its value (as in wushkv_append).
 *   tk    device, float32 [n_kv_heads][d][d] = T_K (as in wushkv_append).
 *   q, tq, out, ws  as in wushkv_decode_attn.
 * EUNSUPPORTED if sink + recent + flush > 1024 (the window one workgroup
 * holds); ECAPACITY if any L + 1 > ctx_cap.  Updates the host lengths on
 * success; a failing call changes nothing.  Groups of 4 and 8 query heads
 * per KV head score and accumulate on the int8 matrix cores inside the same
 * launch.
 */
wushkv_status wushkv_decode_step(wushkv_cache* cache, int32_t layer, int32_t n_seq,
                                 const int32_t* slots, const void* k, const void* v,
                                 const float* tk, const void* q, const float* tq, float* out,
                                 void* ws, uint64_t ws_bytes, void* stream);

/*
 * wushkv_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as wushkv_decode_step,
 * without the workspace: the library keeps it in a file-scope device array
 * of WUSHKV_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  A
 * call whose workspace (wushkv_decode_workspace_bytes) exceeds that returns
 * WUSHKV_EWORKSPACE before any launch (e.g. a step of 8 sequences with 64
 * query heads, whose split partials take about 17.6 MB).  No call allocates or
 * frees memory.  Every call on one GPU shares its array: calls that overlap
 * on one GPU (two streams, two threads) race and must be serialized by the
 * caller.  Nothing in the array needs to start at zero.
 */
#define WUSHKV_NOALLOC_SCRATCH_BYTES (16ull << 20)
wushkv_status wushkv_decode_step_noalloc(wushkv_cache* cache, int32_t layer, int32_t n_seq,
                                         const int32_t* slots, const void* k, const void* v,
                                         const float* tk, const void* q, const float* tq,
                                         float* out, void* stream);

/* Largest number of new positions per sequence in one wushkv_chunk_step. */
#define WUSHKV_MAX_CHUNK 16

/* Bytes of device workspace wushkv_chunk_step needs for n_seq sequences whose
 * largest chunk has max_new positions (0 if max_new is outside 1..16). */
uint64_t wushkv_chunk_workspace_bytes(const wushkv_cache* cache, int32_t n_seq, int32_t max_new);

/*
 * One chunked step of one layer (paper page, section 4.4: each new chunk is
 * first appended in full precision and used for its own attention output,
 * then the entries that left the windows are quantized; section 5.2 evaluates
 * in 16-token chunks).  For each of n_seq sequences (distinct slots, length
 * L >= 0, L + n_new[i] <= ctx_cap), append n_new[i] (1..WUSHKV_MAX_CHUNK)
 * positions and, for every new position L + c, attend its queries to the
 * positions [0, L + c] of the cache (causal inside the chunk; quantized
 * boundary squant(L), the chunk's own entries in bfloat16).  The cache left
 * behind is the one wushkv_append of the same positions leaves.  Sequences
 * of length L >= 1 with n_new = 1 give the result of wushkv_decode_step.
 *
 *   n_new   host int32 [n_seq].
 *   k, v    device, io_dtype [sum(n_new)][n_kv_heads][d]: the sequences'
 *           new positions concatenated in the order of slots[] (post-RoPE
 *           keys; values in the value-transform basis).
 *   tk, tq  device, float32 [n_kv_heads][d][d]: T_K and T_K^{-T}.
 *   q       device, io_dtype [sum(n_new)][n_q_heads][d]: one query per new
 *           position and query head (post-RoPE, uncompensated).
 *   out     device, float32 [sum(n_new)][n_q_heads][d]: attention outputs in
 *           the value-transform basis.
 *   ws      device workspace of ws_bytes >= wushkv_chunk_workspace_bytes(
 *           n_seq, max n_new), 16-byte aligned; contents on entry ignored.
 * The quantized part runs on the int8 matrix cores at every bit width
 * (2, 3, 4): the compensated queries and the softmax weights in 24- and
 * 15-bit fixed point against exact code products.  Updates the host lengths
 * on success; a failing call changes nothing.
 */
wushkv_status wushkv_chunk_step(wushkv_cache* cache, int32_t layer, int32_t n_seq,
                                const int32_t* slots, const int32_t* n_new, const void* k,
                                const void* v, const float* tk, const void* q, const float* tq,
                                float* out, void* ws, uint64_t ws_bytes, void* stream);

/* Instrumentation, not part of the method.  When ev_start and ev_stop are
 * hipEvent_t handles (created by the caller), every later wushkv_decode_attn
 * or wushkv_decode_step call on this cache records ev_start on its stream immediately before the
 * split-K scan kernel and ev_stop immediately after it, so that a caller can
 * time that kernel alone.  Pass NULL, NULL to stop.  Host only. */
wushkv_status wushkv_set_split_events(wushkv_cache* cache, void* ev_start, void* ev_stop);

/* Instrumentation, not part of the method: as wushkv_set_split_events, for
 * the log-sum-exp combine kernel that follows the split-K scan in
 * wushkv_decode_attn and wushkv_decode_step (ev_start immediately before its
 * launch, ev_stop immediately after).  Pass NULL, NULL to stop.  Host only;
 * EINVAL when exactly one of the two is NULL. */
wushkv_status wushkv_set_combine_events(wushkv_cache* cache, void* ev_start, void* ev_stop);

/* Instrumentation, not part of the method: read bytes (a multiple of 16) of
 * the 16-byte-aligned device buffer buf once with a grid-stride kernel of
 * `blocks` workgroups of 256 threads, writing one word per thread to out
 * (device, blocks * 256 uint32).  Its bandwidth is the practical HBM read
 * ceiling the decode kernels are compared with.  Asynchronous on stream. */
wushkv_status wushkv_stream_read_probe(const void* buf, uint64_t bytes, int32_t blocks, void* out,
                                       void* stream);

/* Static string for a status code. */
const char* wushkv_status_str(wushkv_status status);

#ifdef __cplusplus
}
#endif
#endif /* WUSHKV_H */
