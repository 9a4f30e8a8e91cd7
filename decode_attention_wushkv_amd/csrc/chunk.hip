// wushkv_chunk_step kernels: a chunk of up to 16 new positions per sequence
// is appended in full precision, each new position's queries attend to the
// cache up to and including that position, and the window is flushed
// afterwards (WUSH-KV paper page, section 4.4 for the order; section 5.2 for
// evaluation in 16-token chunks; section 4.1 for GQA head sharing; appendix
// D.1 for the 1/sqrt(d) scale).
//
// Four launches per call:
//   prep     one workgroup per (chunk position, KV head, sequence): the G
//            compensated queries q' = T_K^{-T} q (prescaled by log2(e)/sqrt(d),
//            with sigma = sum_i q'_i) as floats and as 24-bit fixed point in
//            three balanced base-256 int8 digits laid out as MFMA operands; the
//            new key transformed with the fp64 arithmetic of every append
//            path and rounded to bfloat16, the new value rounded to bfloat16.
//   attend   per (sequence, KV head, tile of 16 query rows): workgroups over
//            the quantized region [sink, squant(L)) -- every chunk position
//            sees all of it -- and one window workgroup over the sink, the
//            ring and the chunk's own entries (causal inside the chunk).
//            The quantized scan is a dense (16 rows) x (64 positions) x (128
//            dims) contraction per sub-chunk on the int8 matrix cores
//            (v_mfma_i32_16x16x64_i8): scores from the query digits and the
//            2-, 3- or 4-bit codes unpacked to bytes, then o += w c from 15-bit
//            fixed-point softmax weights (two int8 digits) and the value codes;
//            the zero point factors out of both sums (q'.(z + s c) = z sigma +
//            s q'.c).  The window workgroup works in fp32 on bfloat16 rows.
//            Every wave writes its own partial (o, m, l) per row.
//   flush    one workgroup per (position leaving the recent window, KV head,
//            sequence): quantizes it (from the ring, or from the chunk's
//            entries); value-code bits go into their shared 16-byte rows with
//            word atomics, since neighbouring positions are flushed by other
//            workgroups at the same time.
//   merge    one workgroup per (chunk position, query head): log-sum-exp
//            merge into the fp32 output; one more per (sequence, KV head)
//            stores the chunk's entries that stay in bfloat16 (after every
//            read of the ring has finished).
#include "chunk.h"
#include "i8ops.h"
#include "quant.h"

namespace wkv {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kL2eSqrtD = 1.4426950408889634f / 11.313708498984761f;
// Largest |q| (three balanced base-256 digits, each in [-128, 127]) and
// largest softmax-weight code (two such digits).  16-bit queries left score
// errors near 1e-3 relative on keys with large scales; 24 bits remove them.
constexpr int Q8MAX = 8355711;
constexpr int W8MAX = 32639;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float h2f(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

template <int IO_BF16>
__device__ __forceinline__ float ld_io(const void* p, int64_t i) {
  if (IO_BF16) return bf2f(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

template <int IO_BF16>
__device__ __forceinline__ uint16_t io_bf16_bits(const void* p, int64_t i) {
  if (IO_BF16) return ((const uint16_t*)p)[i];
  return f32_to_bf16(((const float*)p)[i]);
}

template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Maxima and sums over the 16 lanes of a DPP row (every lane gets the result).

// Max over the 16 lanes of a DPP row of a non-negative float: its bits as an
// unsigned integer are ordered the same, and an unsigned max (identity 0)
// takes the DPP move into the max itself (a float max needs two more
// operations per step to canonicalize its operand).
__device__ __forceinline__ float row16_max_nonneg(float x) {
  uint32_t v = __float_as_uint(x);
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  return __uint_as_float(v);
}

// Max over the 16 lanes of a DPP row of non-NaN floats (-inf included),
// through an order-preserving signed-integer key: a negative float's bits
// other than the sign flipped (the same map takes the key back).
__device__ __forceinline__ float row16_max_key(float x) {
  int v = __float_as_int(x);
  v ^= (v >> 31) & 0x7FFFFFFF;
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
  v ^= (v >> 31) & 0x7FFFFFFF;
  return __int_as_float(v);
}

__device__ __forceinline__ float row16_sum(float x) {
  x += dppf<0xB1>(x);
  x += dppf<0x4E>(x);
  x += dppf<0x124>(x);
  x += dppf<0x128>(x);
  return x;
}

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Two balanced base-256 digits of |x| <= 32639: x = 256 hi + lo.
__device__ __forceinline__ void digits8(int x, int& lo, int& hi) {
  lo = ((x + 128) & 255) - 128;
  hi = (x - lo) >> 8;
}

// Three balanced base-256 digits of |x| <= 8355711: x = 65536 d2 + 256 d1 + d0.
__device__ __forceinline__ void digits8x3(int x, int& d0, int& d1, int& d2) {
  d0 = ((x + 128) & 255) - 128;
  x = (x - d0) >> 8;
  d1 = ((x + 128) & 255) - 128;
  d2 = (x - d1) >> 8;
}

// Lanes l and l ^ 32 combined (v_permlane32_swap gives every lane both
// values, in the same order on both sides).
__device__ __forceinline__ float cross_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float cross_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// ---------------------------------------------------------------- prep

template <bool B3>
__device__ void flush_entry(const ChunkArgs& a, int si, int h, int p);

// Blocks x < C: the queries and the new entry of chunk position x.  Blocks
// x >= C: ring entry squant(L) + x - C leaves the window in this step and is
// quantized now; the attention reads the window entries from the ring and
// masks their positions in the code planes, so this can precede it.
template <int IO_BF16>
__global__ __launch_bounds__(256) void chunk_prep_kernel(ChunkArgs a) {
  if ((int)blockIdx.x >= a.C) {
    const int si = blockIdx.z, L = a.s.len[si];
    const int sq1 = squant_of(L + a.s.n_new[si], a.g.S, a.g.R, a.g.F);
    const int p = a.s.squant[si] + (int)blockIdx.x - a.C;
    if (p < (sq1 < L ? sq1 : L)) {
      if (a.g.bits == 3)
        flush_entry<true>(a, si, blockIdx.y, p);
      else
        flush_entry<false>(a, si, blockIdx.y, p);
    }
    return;
  }
  __shared__ float qv[8][D];
  __shared__ float hs[2][8][D];
  __shared__ float qs[8][D];
  __shared__ float stat[8][2];
  __shared__ float kin[D];
  __shared__ double khs[2][D];  // half-row sums of the new key's transform
  const int c = blockIdx.x, h = blockIdx.y, si = blockIdx.z, tid = threadIdx.x;
  const Geometry& g = a.g;
  const int G = g.G, M = a.C * G, i = tid & (D - 1), hf = tid >> 7;
  const bool valid = c < a.s.n_new[si];
  const int64_t tok = (int64_t)a.s.tok0[si] + c;  // row in k, v, q, out
  const int64_t unit = (int64_t)si * g.n_kv + h;  // (sequence, KV head) of this call
  for (int x = tid; x < G * D; x += 256)
    qv[x / D][x % D] = valid ? ld_io<IO_BF16>(a.q, (tok * g.n_q + h * G) * D + x) : 0.f;
  float t[64];
  const float4* tp = (const float4*)(a.tq + ((int64_t)h * D + i) * D + 64 * hf);
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const float4 t4 = tp[x];
    t[4 * x] = t4.x;
    t[4 * x + 1] = t4.y;
    t[4 * x + 2] = t4.z;
    t[4 * x + 3] = t4.w;
  }
  // this thread's half row of T_K for the new key (all loads issued before
  // the first wait)
  float tkr[64];
  {
    const float4* kp = (const float4*)(a.tk + ((int64_t)h * D + i) * D + 64 * hf);
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const float4 t4 = kp[x];
      tkr[4 * x] = t4.x;
      tkr[4 * x + 1] = t4.y;
      tkr[4 * x + 2] = t4.z;
      tkr[4 * x + 3] = t4.w;
    }
  }
  if (tid < D) kin[tid] = valid ? ld_io<IO_BF16>(a.k, (tok * g.n_kv + h) * D + tid) : 0.f;
  __syncthreads();
  // k' = T_K k in the shared fp64 order: thread (i, hf) sums chains 2 hf and
  // 2 hf + 1 of row i (dimensions [64 hf, 64 hf + 64)); row i's entry is
  // (s0 + s1) + (s2 + s3)
  {
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int j = 0; j < D / 4; ++j) {
      s0 = fma((double)tkr[j], (double)kin[64 * hf + j], s0);
      s1 = fma((double)tkr[32 + j], (double)kin[64 * hf + 32 + j], s1);
    }
    khs[hf][i] = s0 + s1;
  }
  for (int gg = 0; gg < G; ++gg) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 64; ++j) acc = fmaf(t[j], qv[gg][64 * hf + j], acc);
    hs[hf][gg][i] = acc;
  }
  __syncthreads();
  if (tid < D)
    for (int gg = 0; gg < G; ++gg) qs[gg][i] = (hs[0][gg][i] + hs[1][gg][i]) * kL2eSqrtD;
  __syncthreads();
  // sigma and max |q'| per head: 32 lanes per head, four dimensions each
  {
    const int gg = tid >> 5, part = tid & 31;
    float s = 0.f, mx = 0.f;
    if (gg < G)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = qs[gg][4 * part + e];
        s += x;
        mx = fmaxf(mx, fabsf(x));
      }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      s += __shfl_xor(s, o);
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    if (gg < G && part == 0) {
      stat[gg][0] = s;
      stat[gg][1] = mx;
    }
  }
  __syncthreads();
  // float rows, sigma and 1/S_q; int8 operand digits (zero for positions
  // past the sequence's chunk and for the padding rows of the last tile)
  const int nrows = a.RT * CROWS;
  for (int x = tid; x < G * D; x += 256) {
    const int gg = x / D, d = x % D;
    const int row = c * G + gg;
    const float maxabs = stat[gg][1];
    const float sq = maxabs > 0.f ? (float)Q8MAX / maxabs : 1.f;
    int qi = 0;
    if (valid) {
      qi = (int)rintf(qs[gg][d] * sq);
      qi = qi > Q8MAX ? Q8MAX : (qi < -Q8MAX ? -Q8MAX : qi);
    }
    float* qrow = a.qf + (unit * M + row) * (D + 4);
    qrow[d] = valid ? qs[gg][d] : 0.f;
    if (d == 0) {
      qrow[D] = valid ? stat[gg][0] : 0.f;
      qrow[D + 1] = valid ? 1.f / sq : 0.f;
      qrow[D + 2] = 0.f;
      qrow[D + 3] = 0.f;
    }
    int d0, d1, d2;
    digits8x3(qi, d0, d1, d2);
    const int rt = row >> 4, r16 = row & 15;
    const int ks = d >> 6, grp = (d >> 4) & 3;
    const int lane = r16 + 16 * grp, e = g.bits == 4 ? opnd_byte4(d & 15) : opnd_byte(d & 15);
    int8_t* base = (int8_t*)(a.qa + ((unit * a.RT + rt) * 2 + ks) * 3 * 64);
    base[(0 * 64 + lane) * 16 + e] = (int8_t)d0;
    base[(1 * 64 + lane) * 16 + e] = (int8_t)d1;
    base[(2 * 64 + lane) * 16 + e] = (int8_t)d2;
  }
  if (c == 0)  // padding rows [C G, RT 16) of the last tile: zero digits
    for (int x = tid; x < (nrows - M) * D; x += 256) {
      const int row = M + x / D, d = x % D;
      const int rt = row >> 4, r16 = row & 15;
      const int ks = d >> 6, grp = (d >> 4) & 3;
      const int lane = r16 + 16 * grp, e = g.bits == 4 ? opnd_byte4(d & 15) : opnd_byte(d & 15);
      int8_t* base = (int8_t*)(a.qa + ((unit * a.RT + rt) * 2 + ks) * 3 * 64);
      base[(0 * 64 + lane) * 16 + e] = 0;
      base[(1 * 64 + lane) * 16 + e] = 0;
      base[(2 * 64 + lane) * 16 + e] = 0;
    }
  // the chunk position's new entry: k' rounded once to bfloat16; v
  // (khs was written before the barriers above)
  if (valid) {
    uint16_t* dst = a.knew + (((int64_t)si * a.C + c) * g.n_kv + h) * 2 * D;
    if (tid < D)
      dst[tid] = f64_to_bf16(khs[0][tid] + khs[1][tid]);
    else
      dst[D + i] = io_bf16_bits<IO_BF16>(a.v, (tok * g.n_kv + h) * D + i);
  }
}

// ---------------------------------------------------------------- attend

// One sub-chunk of 64 positions for one wave: key-code words (position 16 cb
// + lane % 16, dimensions 64 ks + 16 (lane / 16) ..), scale/zero words of
// those positions, value-code words (dimension 16 db + lane % 16, positions
// 16 (lane / 16) ..).  Four bits: two words per group of 16; three bits: the
// low-plane word and the high-plane word holding the group's high bits.
template <int BITS>
struct CBuf {
  static constexpr int NW = BITS == 4 ? 2 : 1;
  uint32_t kc[4][2][NW];
  uint32_t kh[BITS == 3 ? 4 : 1][2];
  uint32_t ksz[4], vsz[4];
  uint32_t vc[8][NW];
  uint32_t vh[BITS == 3 ? 8 : 1];
};

// Non-temporal load of one code-plane word: the codes are read once per
// step, so they stream past the caches (as in the split kernel).
__device__ __forceinline__ uint32_t ntl(const uint32_t* p) { return __builtin_nontemporal_load(p); }

template <int BITS>
__device__ __forceinline__ void cload(CBuf<BITS>& b, const ChunkArgs& a, const QMap& qm, int pbase) {
  const int lane = threadIdx.x & 63, m16 = lane & 15, grp = lane >> 4;
  const int64_t row = qrow_read(qm, pbase);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int64_t r = row + 16 * cb + m16;
    const uint32_t* kw = (const uint32_t*)(a.pl.kcode + r * (16 * BITS));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (BITS == 4) {
        b.kc[cb][ks][0] = ntl(kw + (8 * ks + 2 * grp));
        b.kc[cb][ks][1] = ntl(kw + (8 * ks + 2 * grp + 1));
      } else {
        b.kc[cb][ks][0] = ntl(kw + (4 * ks + grp));
      }
      // three bits: the high plane (bytes [32, 48)) word of this group
      if constexpr (BITS == 3) b.kh[cb][ks] = ntl(kw + (8 + 2 * ks + (grp >> 1)));
    }
    b.ksz[cb] = ntl(a.pl.ksz + r);
    b.vsz[cb] = ntl(a.pl.vsz + r);
  }
  if constexpr (BITS == 2) {
    const uint32_t* vw = (const uint32_t*)(a.pl.vcode + ((row >> 6) * D + m16) * 16) + grp;
#pragma unroll
    for (int db = 0; db < 8; ++db) b.vc[db][0] = ntl(vw + (db * 16 * 4));
  } else if constexpr (BITS == 4) {
    // 32 positions per row: this group's 16 in block (row / 32) + grp / 2
    const uint32_t* vw =
        (const uint32_t*)(a.pl.vcode + (((row >> 5) + (grp >> 1)) * D + m16) * 16) + 2 * (grp & 1);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      b.vc[db][0] = ntl(vw + (db * 16 * 4));
      b.vc[db][1] = ntl(vw + (db * 16 * 4 + 1));
    }
  } else {
    // 128-position block: low-plane rows sel = 0, 1 and the high-plane row,
    // whose 8-byte half sel belongs to this sub-chunk
    const int64_t blk = row >> 7;
    const int sel = (int)((row >> 6) & 1);
    const uint32_t* vw = (const uint32_t*)(a.pl.vcode + ((blk * 3 + sel) * D + m16) * 16) + grp;
    const uint32_t* hw = (const uint32_t*)(a.pl.vcode + ((blk * 3 + 2) * D + m16) * 16 + 8 * sel) + (grp >> 1);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      b.vc[db][0] = ntl(vw + (db * 16 * 4));
      b.vh[db] = ntl(hw + (db * 16 * 4));
    }
  }
}

template <int BITS>
__device__ __forceinline__ v4i key_bytes(const CBuf<BITS>& b, int cb, int ks, int grp) {
  if constexpr (BITS == 2) return unpack2(b.kc[cb][ks][0]);
  else if constexpr (BITS == 4) return unpack4(b.kc[cb][ks][0], b.kc[cb][ks][1]);
  else return unpack3(b.kc[cb][ks][0], b.kh[cb][ks], 2 * (grp & 1));
}

template <int BITS>
__device__ __forceinline__ v4i value_bytes(const CBuf<BITS>& b, int db, int grp) {
  if constexpr (BITS == 2) return unpack2(b.vc[db][0]);
  else if constexpr (BITS == 4) return unpack4(b.vc[db][0], b.vc[db][1]);
  else return unpack3(b.vc[db][0], b.vh[db], 2 * (grp & 1));
}

// PAIR (2 bits, one row tile holding at most 8 query rows, e.g. a decode
// step with groups of 8): rows 8..15 of the tile carry the same queries as rows 0..7
// and score the odd 16-position column blocks while rows 0..7 score the even
// ones, so every lane's softmax and weight work is useful.  The two halves
// share each row's maximum; their sums and outputs add up at the end.
template <int BITS, bool PAIR>
__global__ __launch_bounds__(256) void chunk_kernel(ChunkArgs a) {
  extern __shared__ uint4 smem4[];
  const Geometry& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, m16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform for the compiler
  const int nsp = a.n_splits + 1, per = a.RT * nsp, NP = 4 * a.n_splits + 1;
  int u, rem;
  if (a.xcd_map) {
    const int r = blockIdx.x >> 3;
    u = (blockIdx.x & 7) + 8 * (r / per);
    rem = r % per;
  } else {
    u = blockIdx.x / per;
    rem = blockIdx.x % per;
  }
  const int rt = rem / nsp, j = rem % nsp;
  const int h = u % g.n_kv, si = u / g.n_kv;
  const int slot = a.s.slot[si], L = a.s.len[si], sq = a.s.squant[si], nn = a.s.n_new[si];
  const int G = g.G, M = a.C * G;
  float* part = a.part + ((int64_t)u * a.RT + rt) * NP * CROWS * PS;

  if (j < a.n_splits) {
    // ---------------- quantized region, one wave per run of sub-chunks
    const QMap qm = qmap_of(g, a.layer, slot, h);
    const int lo = g.S, hi = sq;
    const int c_first = lo / CSUB;
    const int c_end = hi > lo ? (hi + CSUB - 1) / CSUB : c_first;
    const int nw = 4 * a.n_splits;
    const int c0 = c_first + 4 * j + w;
    const v4i* qa = (const v4i*)(a.qa + ((int64_t)u * a.RT + rt) * 6 * 64);
    v4i A[2][3];  // [d half][digit]
#pragma unroll
    for (int x = 0; x < 6; ++x) A[x / 3][x % 3] = qa[x * 64 + lane];
    // PAIR: the operand with rows 0..7 moved to rows 8..15 (row_shr:8 inside
    // each 16-lane row; rows 0..7 become 0)
    v4i Ah[PAIR ? 2 : 1][3];
    if constexpr (PAIR) {
#pragma unroll
      for (int x = 0; x < 6; ++x)
#pragma unroll
        for (int q = 0; q < 4; ++q) Ah[x / 3][x % 3][q] = __builtin_amdgcn_update_dpp(0, A[x / 3][x % 3][q], 0x118, 0xF, 0xF, false);
    }
    constexpr int NC = PAIR ? 2 : 4;  // 16-position column blocks scored per lane
    const int half = grp >> 1;        // PAIR: lanes 32..63 hold rows 8..15
    float sig[4], inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = PAIR ? (4 * grp + r) & 7 : 16 * rt + 4 * grp + r;
      const float* qr = a.qf + ((int64_t)u * M + (row < M ? row : 0)) * (D + 4);
      sig[r] = row < M ? qr[D] : 0.f;
      inv[r] = row < M ? qr[D + 1] : 0.f;
    }
    uint16_t* wl = (uint16_t*)smem4 + w * 64 * 16;  // this wave's weight operands
    float O[8][4], Mx[4], Lp[4], Zp[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Mx[r] = -INFINITY;
      Lp[r] = Zp[r] = 0.f;
#pragma unroll
      for (int db = 0; db < 8; ++db) O[db][r] = 0.f;
    }
    const int eb = opnd_byte_b<BITS>(m16);
    auto process = [&](const CBuf<BITS>& B0, int c) {
      const int pbase = c * CSUB;
      // ---- scores: D layout lane, r -> row 4 grp + r, position 16 cbl + m16
      // (cbl = cc, or in PAIR 2 cc + half)
      float sc[NC][4], vs[NC], vz[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        v4i a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0}, a2 = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if constexpr (PAIR) {
            const v4i Be = key_bytes<BITS>(B0, 2 * cc, ks, grp);
            const v4i Bo = key_bytes<BITS>(B0, 2 * cc + 1, ks, grp);
            a0 = mfma8(Ah[ks][0], Bo, mfma8(A[ks][0], Be, a0));
            a1 = mfma8(Ah[ks][1], Bo, mfma8(A[ks][1], Be, a1));
            a2 = mfma8(Ah[ks][2], Bo, mfma8(A[ks][2], Be, a2));
          } else {
            const v4i Bk = key_bytes<BITS>(B0, cc, ks, grp);
            a0 = mfma8(A[ks][0], Bk, a0);
            a1 = mfma8(A[ks][1], Bk, a1);
            a2 = mfma8(A[ks][2], Bk, a2);
          }
        }
        const int cbl = PAIR ? 2 * cc + half : cc;
        const int p = pbase + 16 * cbl + m16;
        const bool ok = p >= lo && p < hi;
        const uint32_t kw = PAIR ? (half ? B0.ksz[2 * cc + 1] : B0.ksz[2 * cc]) : B0.ksz[cc];
        const uint32_t vr = PAIR ? (half ? B0.vsz[2 * cc + 1] : B0.vsz[2 * cc]) : B0.vsz[cc];
        const float ksv = h2f(kw & 0xFFFFu), kzv = h2f(kw >> 16);
        const uint32_t vw = ok ? vr : 0u;  // masked positions: scale and zero 0
        vs[cc] = h2f(vw & 0xFFFFu);
        vz[cc] = h2f(vw >> 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // 256 d2 + d1 fits in 32 bits (below 2^24, exact as a float, at 2
          // bits; one more rounding of relative size 2^-24 at 3 and 4 bits)
          const float dot = fmaf((float)(a2[r] * 256 + a1[r]), 256.f, (float)a0[r]);
          sc[cc][r] = ok ? fmaf(ksv, dot * inv[r], kzv * sig[r]) : -INFINITY;
        }
      }
      // ---- per row: sub-chunk max, weights p = exp2(s - m), w = p s_v
      float m[4], wmax[4], lsum[4], zsum[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = sc[0][r];
#pragma unroll
        for (int cc = 1; cc < NC; ++cc) x = fmaxf(x, sc[cc][r]);
        m[r] = row16_max_key(x);  // scores are never NaN (masked: -inf)
        if constexpr (PAIR) m[r] = cross_max(m[r]);
        float wm = 0.f;
        lsum[r] = zsum[r] = 0.f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          const float pp = __builtin_amdgcn_exp2f(sc[cc][r] - m[r]);
          sc[cc][r] = pp * vs[cc];
          lsum[r] += pp;
          zsum[r] = fmaf(pp, vz[cc], zsum[r]);
          wm = fmaxf(wm, sc[cc][r]);
        }
        wmax[r] = row16_max_nonneg(wm);  // weights are >= 0
        if constexpr (PAIR) wmax[r] = cross_max(wmax[r]);
      }
      // ---- weight codes into this wave's A operand (row, position) layout:
      // lane 4 grp + r + 16 cbl, operand byte of m16; lo digit in the low
      // byte.  PAIR: each row's other column blocks get zero weights.
      wave_fence();  // the previous sub-chunk's operand reads are done
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float wsc = wmax[r] > 0.f ? (float)W8MAX * __builtin_amdgcn_rcpf(wmax[r]) : 0.f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          // wq = the weight times wsc rounded to the nearest integer (ties to
          // even), at most W8MAX: added to 1.5 * 2^23 in one rounding, it sits
          // in the low bits of the float (whose bits are 0x4B400000 + wq)
          const uint32_t rb = __float_as_uint(fminf(fmaf(sc[cc][r], wsc, 12582912.f), 12582912.f + (float)W8MAX));
          // balanced digits lo = ((wq + 128) & 255) - 128, hi = (wq + 128) >> 8
          // as two's-complement bytes: lo byte = wq & 255 (the 16-bit store
          // drops the bits above)
          const int cbl = PAIR ? 2 * cc + half : cc;
          wl[((4 * grp + r) + 16 * cbl) * 16 + eb] = (uint16_t)((((rb + 128u) ^ rb) & 0xFF00u) ^ rb);
          if constexpr (PAIR) wl[((4 * grp + r) + 16 * (2 * cc + 1 - half)) * 16 + eb] = 0;
        }
      }
      wave_fence();
      v4i Wl, Wh;
      {
        const uint4* src = (const uint4*)(wl + lane * 16);
        const uint4 x0 = src[0], x1 = src[1];
        const uint32_t dw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        // low (high) bytes of the four 16-bit codes in d0, d1, in order
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t d0 = dw[2 * q], d1 = dw[2 * q + 1];
          Wl[q] = (int)__builtin_amdgcn_perm(d1, d0, 0x06040200u);
          Wh[q] = (int)__builtin_amdgcn_perm(d1, d0, 0x07050301u);
        }
      }
      // ---- online softmax fold and o += w c (lane, r -> row 4 grp + r, dim 16 db + m16)
      float fo[4], fn[4], back[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float Mn = fmaxf(Mx[r], m[r]);
        fo[r] = __builtin_amdgcn_exp2f(Mx[r] - Mn);
        fn[r] = __builtin_amdgcn_exp2f(m[r] - Mn);
        back[r] = wmax[r] * (1.f / (float)W8MAX) * fn[r];
        Lp[r] = fmaf(Lp[r], fo[r], lsum[r] * fn[r]);
        Zp[r] = fmaf(Zp[r], fo[r], zsum[r] * fn[r]);
        Mx[r] = Mn;
      }
      // once the running maxima settle (the common case) no rescale is needed
      const bool keep = __all(fo[0] == 1.f && fo[1] == 1.f && fo[2] == 1.f && fo[3] == 1.f);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const v4i Bv = value_bytes<BITS>(B0, db, grp);
        const v4i pL = mfma8(Wl, Bv, v4i{0, 0, 0, 0});
        const v4i pH = mfma8(Wh, Bv, v4i{0, 0, 0, 0});
        if (keep) {
#pragma unroll
          for (int r = 0; r < 4; ++r) O[db][r] = fmaf((float)(pH[r] * 256 + pL[r]), back[r], O[db][r]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) O[db][r] = fmaf(O[db][r], fo[r], (float)(pH[r] * 256 + pL[r]) * back[r]);
        }
      }
    };
    // two buffers, alternating: the next sub-chunk's codes load during the
    // current one's arithmetic
    CBuf<BITS> B0, B1;
    const int n_my = c0 < c_end ? (c_end - c0 + nw - 1) / nw : 0;  // this wave's sub-chunks
    if (n_my > 0) cload(B0, a, qm, c0 * CSUB);
    // next-buffer loads unconditional (past the end they re-read the current
    // sub-chunk from L2), so that the compiler's wait counts keep them in
    // flight while the current one is processed
    for (int it = 0; it < n_my; it += 2) {
      cload(B1, a, qm, (c0 + (it + 1 < n_my ? it + 1 : it) * nw) * CSUB);
      process(B0, c0 + it * nw);
      if (it + 1 >= n_my) break;
      cload(B0, a, qm, (c0 + (it + 2 < n_my ? it + 2 : it + 1) * nw) * CSUB);
      process(B1, c0 + (it + 1) * nw);
    }
    // ---- this wave's partial: o (unnormalized, zero-point term added), m, l
    // (PAIR: the two halves of each row added; rows 0..7 written)
    float* dst = part + (int64_t)(4 * j + w) * CROWS * PS;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float Lw = row16_sum(Lp[r]);
      float Zw = row16_sum(Zp[r]);
      if constexpr (PAIR) {
        Lw = cross_sum(Lw);
        Zw = cross_sum(Zw);
      }
      float* pr = dst + (4 * grp + r) * PS;
      const bool wr = !PAIR || half == 0;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const float o = PAIR ? cross_sum(O[db][r]) : O[db][r];
        if (wr) pr[16 * db + m16] = o + Zw;
      }
      if (wr && m16 == 0) {
        pr[D] = Mx[r];
        pr[D + 1] = Lw;
      }
    }
    return;
  }

  // ---------------- window: sink, ring and the chunk's own entries (fp32)
  float* qs = (float*)smem4;            // [CROWS][D] q' rows of this tile
  float* sc = qs + CROWS * D;           // [CROWS][win_max] scores, then weights
  const int64_t wunit = ((int64_t)a.layer * g.max_batch + slot) * g.n_kv + h;
  const int ns = L < g.S ? L : g.S;                 // sink entries already cached
  const int nr = L > sq ? L - sq : 0;               // ring entries already cached
  const int E = ns + nr + nn;
  for (int x = tid; x < CROWS * D; x += 256) {
    const int row = 16 * rt + x / D;
    const bool rv = row < M && row / G < nn;
    qs[x] = rv ? a.qf[((int64_t)u * M + row) * (D + 4) + x % D] : 0.f;
  }
  __syncthreads();
  auto pos_of = [&](int e) { return e < ns ? e : (e < ns + nr ? sq + (e - ns) : L + (e - ns - nr)); };
  auto row_ptr = [&](int e, int which) -> const uint16_t* {
    if (e < ns) return (which ? a.pl.vsink : a.pl.ksink) + (wunit * g.S + e) * D;
    if (e < ns + nr) {
      const int p = sq + (e - ns);
      return (which ? a.pl.vring : a.pl.kring) + (wunit * g.W + (p - g.S) % g.W) * D;
    }
    return a.knew + (((int64_t)si * a.C + (e - ns - nr)) * g.n_kv + h) * 2 * D + which * D;
  };
  // scores on the matrix cores (v_mfma_f32_16x16x32_bf16): q' = hi + lo
  // as two bfloat16 operands (16 significant bits), keys exact in bfloat16,
  // fp32 accumulation.  Wave w takes blocks of 16 entries w, w + 4, ...
  {
    bf16x8 Ah[4], Al[4];  // [32-dimension step]: row lane % 16, dims 32 ks + 8 (lane / 16) ..
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        uint32_t hb[2], lb[2];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const float x = qs[m16 * D + 32 * ks + 8 * grp + 2 * q2 + t2];
          const uint16_t h16 = f32_to_bf16(x);
          hb[t2] = h16;
          lb[t2] = f32_to_bf16(x - bf2f(h16));
        }
        hw[q2] = hb[0] | (hb[1] << 16);
        lw[q2] = lb[0] | (lb[1] << 16);
      }
      Ah[ks] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      Al[ks] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
    for (int eb = w; eb * 16 < E; eb += 4) {
      const int e = eb * 16 + m16;
      const uint4* kr = (const uint4*)row_ptr(e < E ? e : E - 1, 0);
      uint4 kb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[ks] = kr[4 * ks + grp];
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 B = __builtin_bit_cast(bf16x8, kb[ks]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[ks], B, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al[ks], B, acc, 0, 0, 0);
      }
      // D: lane, r -> row 4 grp + r, entry e
      if (e < E) {
        const int p = pos_of(e);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + 4 * grp + r;
          const bool vis = row < M && row / G < nn && p <= L + row / G;
          sc[(4 * grp + r) * a.win_max + e] = vis ? acc[r] : -INFINITY;
        }
      }
    }
  }
  __syncthreads();
  // per row: max, weights, sum (16 threads per row)
  float* rstat = sc + CROWS * a.win_max;  // [CROWS][2]: m, l
  {
    const int r = tid >> 4, part16 = tid & 15;
    float mx = -INFINITY;
    for (int e = part16; e < E; e += 16) mx = fmaxf(mx, sc[r * a.win_max + e]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float ls = 0.f;
    for (int e = part16; e < E; e += 16) {
      const float s = sc[r * a.win_max + e];
      const float p = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s - mx);
      sc[r * a.win_max + e] = p;
      ls += p;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ls += __shfl_xor(ls, o);
    if (part16 == 0) {
      rstat[2 * r] = mx;
      rstat[2 * r + 1] = ls;
    }
  }
  __syncthreads();
  // o[row][dim] = sum_e p v: thread = dimension, rows 8 hf .. 8 hf + 8
  {
    const int dim = tid & (D - 1), hf = tid >> 7;
    float acc[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = 0.f;
    // value rows in batches of 16 entries, all loads of a batch in flight
    for (int e0 = 0; e0 < E; e0 += 16) {
      float vv[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) vv[k] = e0 + k < E ? bf2f(row_ptr(e0 + k, 1)[dim]) : 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int e = e0 + k < E ? e0 + k : E - 1;  // vv is 0 past the end
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] = fmaf(sc[(8 * hf + r) * a.win_max + e], vv[k], acc[r]);
      }
    }
    float* dst = part + (int64_t)(NP - 1) * CROWS * PS;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float* pr = dst + (8 * hf + r) * PS;
      pr[dim] = acc[r];
      if (dim == 0) {
        pr[D] = rstat[2 * (8 * hf + r)];
        pr[D + 1] = rstat[2 * (8 * hf + r) + 1];
      }
    }
  }
}

// ---------------------------------------------------------------- merge, flush

__global__ __launch_bounds__(256) void chunk_merge_kernel(ChunkArgs a) {
  __shared__ float red[4][D];
  __shared__ float mred[256];
  const Geometry& g = a.g;
  const int tid = threadIdx.x;
  const int nmerge = a.n_tok * g.n_q;
  const int NP = 4 * a.n_splits + 1;
  if ((int)blockIdx.x < nmerge) {
    const int tr = blockIdx.x / g.n_q, jq = blockIdx.x % g.n_q;
    int si = 0;
    while (si + 1 < a.n_seq && a.s.tok0[si + 1] <= tr) ++si;
    const int c = tr - a.s.tok0[si];
    const int h = jq / g.G, gg = jq % g.G;
    const int row = c * g.G + gg, rt = row >> 4, r16 = row & 15;
    const float* src = a.part + (((int64_t)si * g.n_kv + h) * a.RT + rt) * NP * CROWS * PS + r16 * PS;
    // thread = (dimension, partial residue mod 2).  Every load of the first
    // 2 KM partials is issued before the maximum is known (one round trip);
    // the first wave reduces the maximum over all NP <= 4 * 64 + 1 partials.
    constexpr int KM = 16;
    const int dim = tid & (D - 1), hf = tid >> 7;
    float ov[KM], mv[KM], lv[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      const int x = hf + 2 * k;
      ov[k] = mv[k] = lv[k] = 0.f;
      if (x < NP) {
        const float* px = src + (int64_t)x * CROWS * PS;
        ov[k] = px[dim];
        mv[k] = px[D];
        lv[k] = px[D + 1];
      }
    }
    if (tid < 64) {
      float mx = -INFINITY;
      for (int x = tid; x < NP; x += 64) {
        const float* px = src + (int64_t)x * CROWS * PS;
        if (px[D + 1] > 0.f) mx = fmaxf(mx, px[D]);
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      if (tid == 0) mred[0] = mx;
    }
    __syncthreads();
    const float mx = mred[0];
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (lv[k] > 0.f) {
        const float f = __builtin_amdgcn_exp2f(mv[k] - mx);
        o = fmaf(ov[k], f, o);
        l = fmaf(lv[k], f, l);
      }
    }
    for (int x = hf + 2 * KM; x < NP; x += 2) {
      const float* px = src + (int64_t)x * CROWS * PS;
      const float lx = px[D + 1];
      if (lx > 0.f) {
        const float f = __builtin_amdgcn_exp2f(px[D] - mx);
        o = fmaf(px[dim], f, o);
        l = fmaf(lx, f, l);
      }
    }
    red[hf][dim] = o;
    red[2 + hf][dim] = l;
    __syncthreads();
    if (tid < D) a.out[((int64_t)tr * g.n_q + jq) * D + tid] = (red[0][tid] + red[1][tid]) / (red[2][tid] + red[3][tid]);
    return;
  }
  // stores of one (sequence, KV head): the chunk's entries that stay in
  // bfloat16 go to the sink or the ring (the flush kernel has read every
  // ring entry it quantizes)
  const int fb = blockIdx.x - nmerge;
  const int si = fb / g.n_kv, h = fb % g.n_kv;
  const int slot = a.s.slot[si], L = a.s.len[si], nn = a.s.n_new[si];
  const int sq1 = squant_of(L + nn, g.S, g.R, g.F);
  const int64_t wunit = ((int64_t)a.layer * g.max_batch + slot) * g.n_kv + h;
  const uint16_t* knew = a.knew + ((int64_t)si * a.C * g.n_kv + h) * 2 * D;
  for (int x = tid; x < nn * 2 * D; x += 256) {
    const int c = x / (2 * D), which = (x / D) & 1, i = x % D;
    const int p = L + c;
    const uint16_t b = knew[(int64_t)c * g.n_kv * 2 * D + which * D + i];
    if (p < g.S)
      (which ? a.pl.vsink : a.pl.ksink)[(wunit * g.S + p) * D + i] = b;
    else if (p >= sq1)
      (which ? a.pl.vring : a.pl.kring)[(wunit * g.W + (p - g.S) % g.W) * D + i] = b;
  }
}

// Quantizes position p of sequence si, KV head h, as it leaves the window:
// threads 0..127 its key entry, 128..255 its value entry.  Ring entries
// (p < L) are read from the ring, new entries from the prep kernel's output.
template <bool B3>
__device__ void flush_entry(const ChunkArgs& a, int si, int h, int p) {
  __shared__ QLds ql;
  const Geometry& g = a.g;
  const int tid = threadIdx.x;
  const int slot = a.s.slot[si], L = a.s.len[si];
  const int i = tid & (D - 1);
  const bool is_v = tid >= D;
  const int64_t wunit = ((int64_t)a.layer * g.max_batch + slot) * g.n_kv + h;
  uint16_t b;
  if (p < L) {
    const int64_t o = (wunit * g.W + (p - g.S) % g.W) * D + i;
    b = is_v ? a.pl.vring[o] : a.pl.kring[o];
  } else {
    b = a.knew[(((int64_t)si * a.C + (p - L)) * g.n_kv + h) * 2 * D + (is_v ? D : 0) + i];
  }
  const float x = bf2f(b);
  const QMap qm = qmap_of(g, a.layer, slot, h);
  VRows vr;
  vrows_init(vr);
  store_quantized<B3>(p, x, x, ql, vr, a.pl, qm, g);
  // the value code of this position, left in vr (the low plane, and at 3
  // bits the high plane): only its own bits of the dimension's row words change
  if (is_v) {
    const VRow* rows[2] = {&vr.lo, &vr.hi};
#pragma unroll
    for (int k = 0; k < (B3 ? 2 : 1); ++k) {
      const VRow& v = *rows[k];
      if (v.row < 0) continue;
      uint32_t* wd = (uint32_t*)(a.pl.vcode + (v.row * D + i) * 16);
      const uint32_t bb[4] = {v.b0, v.b1, v.b2, v.b3};
      const uint32_t mm[4] = {v.m0, v.m1, v.m2, v.m3};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (mm[q]) {
          atomicAnd(wd + q, ~mm[q]);
          atomicOr(wd + q, bb[q]);
        }
    }
  }
}

// One new position p = max(squant(L), L) + blockIdx.x of those that leave the
// window in this step, after the prep kernel has made its entry.
template <bool B3>
__global__ __launch_bounds__(256) void chunk_flush_kernel(ChunkArgs a) {
  const int si = blockIdx.z, h = blockIdx.y;
  const int L = a.s.len[si], sq0 = a.s.squant[si];
  const int sq1 = squant_of(L + a.s.n_new[si], a.g.S, a.g.R, a.g.F);
  const int p = (sq0 > L ? sq0 : L) + blockIdx.x;
  if (p < sq1) flush_entry<B3>(a, si, h, p);
}

}  // namespace

hipError_t launch_chunk(ChunkArgs& a, int io_bf16, hipStream_t st) {
  dim3 pgrid(a.C + a.n_flush_ring, a.g.n_kv, a.n_seq);
  if (io_bf16)
    hipLaunchKernelGGL(chunk_prep_kernel<1>, pgrid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(chunk_prep_kernel<0>, pgrid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds_q = 4 * 64 * 16 * 2;
  const size_t lds_w = ((size_t)CROWS * D + (size_t)CROWS * a.win_max + 2 * CROWS) * 4;
  const size_t lds = lds_q > lds_w ? lds_q : lds_w;
  const int tiles = a.n_seq * a.g.n_kv * a.RT;
  if (a.n_splits > 0) {
    int dev = 0, cus = 0, per = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per, a.g.bits == 2 ? chunk_kernel<2, false> : a.g.bits == 3 ? chunk_kernel<3, false> : chunk_kernel<4, false>,
          256, lds);
    if (e != hipSuccess) return e;
    int fill = (cus * (per > 0 ? per : 1) - tiles) / tiles;
    if (fill < 1) fill = 1;
    if (a.n_splits > fill) a.n_splits = fill;
  }
  a.xcd_map = (a.n_seq * a.g.n_kv) % 8 == 0;
  const dim3 grid(tiles * (a.n_splits + 1));
  // paired rows at 2 bits (0.178 -> 0.163 ms per layer for a decode step
  // with groups of 8 on the 64K-prefill cache); at 3 and 4 bits the extra
  // operand registers cost more than the halved row work saves
  const bool pair = a.g.bits == 2 && a.RT == 1 && a.C * a.g.G <= 8;
  if (a.g.bits == 2) {
    if (pair)
      hipLaunchKernelGGL((chunk_kernel<2, true>), grid, dim3(256), lds, st, a);
    else
      hipLaunchKernelGGL((chunk_kernel<2, false>), grid, dim3(256), lds, st, a);
  } else if (a.g.bits == 3) {
    hipLaunchKernelGGL((chunk_kernel<3, false>), grid, dim3(256), lds, st, a);
  } else {
    hipLaunchKernelGGL((chunk_kernel<4, false>), grid, dim3(256), lds, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.n_flush_new > 0) {
    const dim3 fgrid(a.n_flush_new, a.g.n_kv, a.n_seq);
    if (a.g.bits == 3)
      hipLaunchKernelGGL(chunk_flush_kernel<true>, fgrid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(chunk_flush_kernel<false>, fgrid, dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(chunk_merge_kernel, dim3(a.n_tok * a.g.n_q + a.n_seq * a.g.n_kv), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace wkv
