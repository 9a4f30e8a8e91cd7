// wushkv_decode_attn kernels: GQA decode attention over the mixed cache
// (WUSH-KV paper page: section 4.1 for the cache and GQA head sharing,
// section 4.2 / appendix B.1 for the T_K^{-T} query compensation, section
// 4.4 for the full-precision windows, appendix D.1 for the 1/sqrt(d) scale).
//
// Two launches per call:
//   split   workgroups (4 waves) per (sequence, KV head): n_splits over the
//           quantized region plus one over the bfloat16 sink + recent entries.
//           Every workgroup first compensates the G query heads of its KV
//           head: q' = T_K^{-T} q, prescaled by log2(e)/sqrt(d); sigma =
//           sum_i q'_i (the zero point factors out of a score:
//           q'.(z + s c) = z sigma + s (q'.c)); q' also as a 24-bit
//           fixed-point vector in signed base-16 digits for v_dot8.
//             quantized workgroups: each wave walks 128-position sub-chunks
//             (64 at 4 bits) with the next sub-chunk's codes in flight.
//             Scores q'.c come from v_dot8 (4-bit x 4-bit) on unpacked codes
//             and the query digits; the sub-chunk max gives exp2 weights
//             w_t = p_t s_t, quantized to 16 bits against the sub-chunk's
//             largest one and split into base-16 digit words; o_i =
//             sum_t w_t c_{t,i} is again v_dot8 over the dim-major value rows
//             (two dimensions per lane); o += sum_t p_t z_t; an online
//             softmax in float folds the sub-chunks together.
//             window workgroup: fp32 dot products over bfloat16 rows.
//           Each workgroup writes (o, m, l) per query head.
//   combine one workgroup per (sequence, query head): log-sum-exp merge of the
//           partials into the fp32 output.
//
// Decode step (attention fused with the one-token append, in the order of
// section 4.4: the new entry is attended in full precision, then the window
// is flushed): the window workgroup also transforms the new key, includes the
// new position in its window, and after writing its partial quantizes the
// ring entries that leave the recent window and stores the new entry.  The
// quantized workgroups read positions below the old boundary only, so the
// codes it writes (at or above that boundary) never race with them.
#include "i8ops.h"
#include "quant.h"

namespace wkv {
namespace {

constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;
constexpr int pow16m1(int n) { return n == 0 ? 0 : 16 * pow16m1(n - 1) + 15; }
// Largest |q_i| representable by QDIG balanced base-16 digits in [-8, 7].
constexpr int QMAX = 7 * (pow16m1(QDIG) / 15);
// Largest softmax-weight code: WDIG unsigned base-16 digits.
constexpr uint32_t WMAX = (uint32_t)pow16m1(WDIG);

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

template <int IO_BF16>
__device__ __forceinline__ float load_io(const void* base, int64_t idx) {
  if (IO_BF16) return bf16_to_f32(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

// Wave-wide sum / max: DPP within rows of 16 lanes, then the four row
// results read into scalars.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x124>(x);  // row_ror:4
  x += dpp_f<0x128>(x);  // row_ror:8
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  x = fmaxf(x, dpp_f<0x128>(x));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// 2^x for x <= 0 straight from v_exp_f32 (results below 2^-126 may flush to 0,
// which only drops weights too small to matter).
__device__ __forceinline__ float exp2_nonpos(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of the neighbouring lane (lane ^ 1) via DPP quad_perm [1, 0, 3, 2].
__device__ __forceinline__ int swap_adjacent(int x) {
  return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
}

// Block-wide (256 threads) reductions of NV values per thread (all threads get
// the results).
template <int NV, bool MAX>
__device__ __forceinline__ void block_reduce(float (&v)[NV], float* red) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = MAX ? wave_max(v[k]) : wave_sum(v[k]);
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < NV; ++k) red[w * 16 + k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float a0 = red[k], a1 = red[16 + k], a2 = red[32 + k], a3 = red[48 + k];
    v[k] = MAX ? fmaxf(fmaxf(a0, a1), fmaxf(a2, a3)) : (a0 + a1) + (a2 + a3);
  }
}

// Block-wide sums of v[0, NV) and maxima of v[NV, 2 NV) in one pass.
template <int NV>
__device__ __forceinline__ void block_reduce_sum_max(float (&v)[2 * NV], float* red) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    v[k] = wave_sum(v[k]);
    v[NV + k] = wave_max(v[NV + k]);
  }
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < 2 * NV; ++k) red[w * 16 + k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    v[k] = (red[k] + red[16 + k]) + (red[32 + k] + red[48 + k]);
    v[NV + k] = fmaxf(fmaxf(red[NV + k], red[16 + NV + k]), fmaxf(red[32 + NV + k], red[48 + NV + k]));
  }
}

// Orders this wave's LDS accesses before the following ones (lanes of one
// wave exchange data through LDS without a workgroup barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- layout

template <int BITS, int G>
struct SplitCfg {
  static constexpr int TW = sub_len(BITS);     // positions per wave sub-chunk
  // positions per 16-byte value row of a dimension (at 3 bits: per low-plane
  // row; a sub-chunk reads half of its block's high-plane row)
  static constexpr int VB = BITS == 3 ? 64 : 128 / BITS;
  static constexpr int NBW = TW / VB;          // value rows per sub-chunk (2; 1 at 3 bits)
  static constexpr int CB = 16 * BITS;         // key-code bytes per position
  static constexpr int ROWS = TW / 32;         // positions per lane pair
  static constexpr int KQ = BITS == 4 ? 2 : 1; // uint4 per lane (half a position; low plane at 3 bits)
  static constexpr bool SPLIT2 = BITS != 4;    // 2-bit nibble unpacking (low plane at 3 bits)
  static constexpr int GS = SPLIT2 ? 16 : 8;   // positions per 32-bit value-row word
  static constexpr int NG = TW / GS;           // value-row words per sub-chunk (8)
  static constexpr int WGW = SPLIT2 ? 2 * WDIG : WDIG;  // digit words per row word
  static constexpr int WGP = (WGW + 3) / 4 * 4;            // ... padded to 16 bytes
  // G >= 4: the quantized waves run on the int8 matrix cores, each wave on
  // its own MT-position sub-chunks for all G heads, in NTL tiles of four
  static constexpr bool HS = G >= 4;
  static constexpr int MT = 64;
  static constexpr int NTL = HS ? G / 4 : 1;
  // LDS (32-bit words).  Persistent part:
  static constexpr int O_OBUF = 0;                          // [G][D] partial o
  static constexpr int O_RED = O_OBUF + G * D;              // [64] reductions
  static constexpr int O_QF = O_RED + 64;                   // [G][D] q' (float)
  static constexpr int O_QSC = O_QF + G * D;                // [G][4] sigma, 1/S_q, qsum0, qsum1
  static constexpr int O_QD = O_QSC + G * 4;                // [G][16][DIGP] digit words
  static constexpr int O_UNION = O_QD + G * 16 * DIGP;
  // Union: query setup | quantized waves | window.
  static constexpr int SETUP = G * D + 2 * G * D + QDIG * G * D / 4;   // qv, halves, digits (bytes/4)
  // per wave: weight staging (16-bit codes; [tile][head][group][16] on the
  // matrix-core path)
  static constexpr int WAVE = HS ? NTL * 128 : G * TW + G * NG * WGP;
  static constexpr int QUANT = 4 * WAVE + 4 * G * (D + 2);
  // window workgroup, in the union: scores [G][WINDOW_MAX], the decode-step
  // new key and value (bfloat16, D words), per-wave PV partials [4][G][D]
  static constexpr int O_NEW = G * WINDOW_MAX;
  static constexpr int O_WPART = O_NEW + D;
  static constexpr int WIN = O_WPART + 4 * G * D;
  static constexpr int U1 = SETUP > QUANT ? SETUP : QUANT;
  static constexpr int UNION = U1 > WIN ? U1 : WIN;
  static constexpr int TOTAL = O_UNION + UNION;
};

// ---------------------------------------------------------------- query

// A thread's inputs to the query compensation: its elements of the G raw
// queries (element tid + 256 n) and its half row of T_K^{-T}.
template <int G>
struct QueryIn {
  float q[(G * D + 255) / 256];
  float t[64];
};

// Issues the global loads of the compensation inputs.  Callers issue their
// first code loads after this, so that waiting for these inputs does not wait
// for the codes as well.
// The raw-query part of the compensation inputs.
template <int IO_BF16, int G>
__device__ __forceinline__ void compensate_load_q(const DecodeArgs& a, int h, int si, QueryIn<G>& in) {
  const int tid = threadIdx.x;
  const int64_t q0 = ((int64_t)si * a.g.n_q + h * G) * D;
  // (every thread loads, past the end a repeat of the last element that the
  // caller ignores: a load under a branch would be waited for at the branch
  // join, before the loads that follow are issued)
#pragma unroll
  for (int n = 0; n < (G * D + 255) / 256; ++n) {
    const int x = tid + 256 * n;
    in.q[n] = load_io<IO_BF16>(a.q, q0 + (x < G * D ? x : G * D - 1));
  }
}

template <int IO_BF16, int G>
__device__ __forceinline__ void compensate_load(const DecodeArgs& a, int h, int si, QueryIn<G>& in) {
  const int tid = threadIdx.x, i = tid & (D - 1), hf = tid >> 7;
  compensate_load_q<IO_BF16, G>(a, h, si, in);
  const float4* tp = (const float4*)(a.tq + ((int64_t)h * D + i) * D + 64 * hf);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const float4 t4 = tp[c];
    in.t[4 * c] = t4.x;
    in.t[4 * c + 1] = t4.y;
    in.t[4 * c + 2] = t4.z;
    in.t[4 * c + 3] = t4.w;
  }
}

// q' = T_K^{-T} q for the G query heads of KV head h (all 256 threads):
// float copy, sigma, and the digit words for the integer dot products.
template <int IO_BF16, int BITS, int G>
__device__ __forceinline__ void compensate_query(const DecodeArgs& a, int h, int si, uint32_t* sm,
                                                 const QueryIn<G>& in) {
  using C = SplitCfg<BITS, G>;
  float* qf = (float*)(sm + C::O_QF);
  float* qsc = (float*)(sm + C::O_QSC);
  uint32_t* qdw = sm + C::O_QD;
  float* red = (float*)(sm + C::O_RED);
  float* qv = (float*)(sm + C::O_UNION);     // [G][D] raw queries
  float* hsum = qv + G * D;                  // [2][G][D] half-row sums
  int8_t* dig = (int8_t*)(hsum + 2 * G * D); // [QDIG][G][D]
  const int tid = threadIdx.x, i = tid & (D - 1), hf = tid >> 7;
#pragma unroll
  for (int n = 0; n < (G * D + 255) / 256; ++n)
    if (tid + 256 * n < G * D) qv[tid + 256 * n] = in.q[n];
  const float* t = in.t;
  __syncthreads();
  // half-row sums in four interleaved chains (independent FMAs in flight)
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    float c4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 64; j += 4) {
      const float4 q4 = *(const float4*)(qv + gg * D + 64 * hf + j);
      c4[0] = fmaf(t[j], q4.x, c4[0]);
      c4[1] = fmaf(t[j + 1], q4.y, c4[1]);
      c4[2] = fmaf(t[j + 2], q4.z, c4[2]);
      c4[3] = fmaf(t[j + 3], q4.w, c4[3]);
    }
    hsum[(hf * G + gg) * D + i] = (c4[0] + c4[1]) + (c4[2] + c4[3]);
  }
  __syncthreads();
  float v[2 * G];
  float q[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    q[gg] = (hsum[gg * D + i] + hsum[(G + gg) * D + i]) * kLog2eOverSqrtD;
    v[gg] = hf ? 0.f : q[gg];
    v[G + gg] = fabsf(q[gg]);
  }
  block_reduce_sum_max<G>(v, red);
  // fixed point: qi = rint(q' S_q), |qi| <= QMAX; balanced base-16 digits
  int qsum_h[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float maxabs = v[G + gg];
    const float sq = maxabs > 0.f ? (float)QMAX / maxabs : 1.f;
    int qi = (int)rint((double)q[gg] * (double)sq);
    qi = qi > QMAX ? QMAX : (qi < -QMAX ? -QMAX : qi);
    if (hf == 0) {
      qf[gg * D + i] = q[gg];
      int r = qi;
      if constexpr (C::HS) {
        // three balanced base-256 digits (|qi| <= QMAX < 2^23, so the top one
        // stays within [-128, 127]) for the int8 matrix cores
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int d = ((r + 128) & 255) - 128;
          dig[(k * G + gg) * D + i] = (int8_t)d;
          r = (r - d) >> 8;
        }
        dig[(2 * G + gg) * D + i] = (int8_t)r;
      } else {
#pragma unroll
        for (int k = 0; k < QDIG - 1; ++k) {
          const int d = ((r + 8) & 15) - 8;
          dig[(k * G + gg) * D + i] = (int8_t)d;
          r = (r - d) >> 4;
        }
        dig[((QDIG - 1) * G + gg) * D + i] = (int8_t)r;
      }
    }
    if (tid == 0) {
      qsc[gg * 4] = v[gg];
      qsc[gg * 4 + 1] = 1.f / sq;
    }
    if constexpr (!C::HS) {
      // sums of qi over dimensions [0, 64) and [64, 128) (waves 0 and 1),
      // exact in int32 (|qi| < 2^23), stored as floats for the 4-bit code
      // offset of the integer-dot path
      qsum_h[gg] = hf ? 0 : qi;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) qsum_h[gg] += __shfl_xor(qsum_h[gg], o);
      if (tid == 0) qsc[gg * 4 + 2] = (float)qsum_h[gg];
      if (tid == 64) qsc[gg * 4 + 3] = (float)qsum_h[gg];
    }
  }
  __syncthreads();
  if constexpr (C::HS) {
    // A operands of the int8 matrix cores, [tile][ks][lane] 16 bytes each:
    // lane = (row = lane % 16, group = lane / 16), row 4 h + k holds digit k of
    // head 4 tile + h (k = 3: zero); operand byte e of the lane holds dimension
    // 32 group + 16 ks + m with e the operand byte of m in the order the key
    // codes unpack to (the same dimensions the lane's key words hold).
    for (int x = tid; x < C::NTL * 2 * 64 * 4; x += 256) {
      const int qw = x & 3, ln = (x >> 2) & 63, ks = (x >> 8) & 1, t = x >> 9;
      const int row = ln & 15, grp = ln >> 4, hh = 4 * t + (row >> 2), dg = row & 3;
      uint32_t word = 0;
      if (dg < 3)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          // element m with operand byte 4 qw + jb
          const int m = BITS == 4 ? 8 * (qw >> 1) + 2 * jb + (qw & 1) : 4 * jb + qw;
          word |= (uint32_t)(uint8_t)dig[(dg * G + hh) * D + 32 * grp + 16 * ks + m] << (8 * jb);
        }
      qdw[x] = word;
    }
    __syncthreads();
    return;
  }
  // digit words: group x / DIGP of 8 dimensions, digit k = x % DIGP; nibble n
  // holds that digit of one dimension of the group.
  //   2, 3 bits: group = half * 8 + w * 2 + parity, dims 64 half + 16 w + 2 n + parity
  //   4 bits:    group = half * 8 + w,              dims 64 half + 8 w + n
  for (int x = tid; x < G * 16 * DIGP; x += 256) {
    const int gg = x / (16 * DIGP), rem = x % (16 * DIGP);
    const int grp16 = rem / DIGP, k = rem % DIGP, half = grp16 >> 3;
    int e0, step;
    if (BITS != 4) {
      e0 = 64 * half + 16 * ((grp16 >> 1) & 3) + (grp16 & 1);
      step = 2;
    } else {
      e0 = 64 * half + 8 * (grp16 & 7);
      step = 1;
    }
    uint32_t word = 0;
    if (k < QDIG)
#pragma unroll
      for (int n = 0; n < 8; ++n) word |= ((uint32_t)dig[(k * G + gg) * D + e0 + step * n] & 15u) << (4 * n);
    qdw[x] = word;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- quantized

// Registers holding one sub-chunk's codes: key codes (lane pair per
// position), scale/zero words, value rows of dimensions lane and lane + 64.
// Loads are unconditional: a sub-chunk never leaves its unit (cpos and the
// page size are multiples of 128); positions outside [lo, hi) are masked
// arithmetically.
template <int BITS, int G>
struct SubBuf {
  using C = SplitCfg<BITS, G>;
  uint4 kc[C::ROWS][C::KQ];
  uint32_t ksz[C::ROWS], vsz[C::ROWS];
  uint4 vc[C::NBW][2];
  // 3 bits: high-plane bits of the keys (half a position) and of the value
  // rows (the sub-chunk's 64 positions)
  uint2 kh[BITS == 3 ? C::ROWS : 1];
  uint2 vh[2];
};

// Buffer resource over `bytes` bytes from a wave-uniform address (raw
// buffer, byte offsets, bounds-checked).  The code loads carry the
// non-temporal hint (cache policy bit nt) where one wave reads each sub-chunk:
// the codes are read once per step, and streaming them past the caches
// measured 108 -> 94 us per 128K MHA launch at 4 bits and 65 -> 63 us at
// 2 bits.  With the head split the four waves of a workgroup read the same
// sub-chunks, and there the default policy keeps them in L2 for each other.
constexpr int CPOL_NT = 2;  // cache-policy operand of the buffer-load builtins: nt
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

template <int CP>
__device__ __forceinline__ uint4 buf_b128(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CP);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int CP>
__device__ __forceinline__ uint2 buf_b64(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, CP);
  return make_uint2(v[0], v[1]);
}

// Issues the loads of the sub-chunk at position pbase.  Buffer loads: the
// sub-chunk's base addresses are wave-uniform (resources in scalar
// registers) and every lane offset is loop-invariant, so a load needs no
// per-sub-chunk vector address registers.  pbase < 0 issues the same loads
// from `spare` instead (any 16-byte aligned 8 KB the workgroup has just read,
// so served by L2): the prefetch past a wave's last sub-chunk stays
// unconditional without re-reading codes from HBM.
template <int BITS, int G, int CP>
__device__ __forceinline__ void load_sub(SubBuf<BITS, G>& b, const DecodeArgs& a, const QMap& qm,
                                         int pbase, const uint8_t* spare) {
  using C = SplitCfg<BITS, G>;
  const int lane = threadIdx.x & 63, half = lane & 1, tq = lane >> 1;
  const bool past = pbase < 0;
  const int64_t row = qrow_read(qm, past ? 0 : pbase);
  // key codes: C::TW positions of C::CB bytes (3 bits: low plane in bytes
  // [0, 32) of a position, high plane in [32, 48))
  const auto rk = wave_rsrc(past ? spare : a.pl.kcode + row * C::CB, C::TW * C::CB);
  const auto rks = wave_rsrc(past ? (const void*)spare : (const void*)(a.pl.ksz + row), C::TW * 4);
  const auto rvs = wave_rsrc(past ? (const void*)spare : (const void*)(a.pl.vsz + row), C::TW * 4);
  const int ko = tq * C::CB + half * (BITS == 3 ? 16 : C::CB / 2);
#pragma unroll
  for (int r = 0; r < C::ROWS; ++r) {
#pragma unroll
    for (int q = 0; q < C::KQ; ++q) b.kc[r][q] = buf_b128<CP>(rk, ko + 32 * r * C::CB + 16 * q, 0);
    if constexpr (BITS == 3) b.kh[r] = buf_b64<CP>(rk, tq * C::CB + 32 + 8 * half + 32 * r * C::CB, 0);
    b.ksz[r] = __builtin_amdgcn_raw_buffer_load_b32(rks, 4 * (tq + 32 * r), 0, CP);
    b.vsz[r] = __builtin_amdgcn_raw_buffer_load_b32(rvs, 4 * (tq + 32 * r), 0, CP);
  }
  // value rows of dimensions lane and lane + 64; at 3 bits the 128-position
  // block holds two low-plane rows (the sub-chunk's is row sel) and the
  // high-plane row (the sub-chunk's half at byte 8 sel)
  if constexpr (BITS == 3) {
    const int sel = (int)((row >> 6) & 1);
    const auto rv = wave_rsrc(past ? spare : a.pl.vcode + (row >> 7) * 3 * D * 16, 3 * D * 16);
    b.vc[0][0] = buf_b128<CP>(rv, lane * 16, sel * D * 16);
    b.vc[0][1] = buf_b128<CP>(rv, lane * 16 + 64 * 16, sel * D * 16);
    b.vh[0] = buf_b64<CP>(rv, lane * 16 + 2 * D * 16, 8 * sel);
    b.vh[1] = buf_b64<CP>(rv, lane * 16 + 2 * D * 16 + 64 * 16, 8 * sel);
  } else {
    const auto rv = wave_rsrc(past ? spare : a.pl.vcode + (row / C::VB) * D * 16, C::NBW * D * 16);
#pragma unroll
    for (int k = 0; k < C::NBW; ++k) {
      b.vc[k][0] = buf_b128<CP>(rv, lane * 16 + k * D * 16, 0);
      b.vc[k][1] = buf_b128<CP>(rv, lane * 16 + k * D * 16 + 64 * 16, 0);
    }
  }
}

struct QueryRegs {
  float sig, inv, qsum;
};

// Scores, weights and value accumulation of one sub-chunk; folds the result
// into the wave's running (M, Lrun, O) (online softmax across sub-chunks).
// Nibble word x (0..7) of a lane's half position: the codes of the 8
// dimensions that digit group x of the query covers, as signed or unsigned
// 4-bit lanes for v_dot8.
template <int BITS, int G>
__device__ __forceinline__ int code_nibbles(const SubBuf<BITS, G>& b, int r, int x) {
  using C = SplitCfg<BITS, G>;
  const uint4 k0 = b.kc[r][0];
  const uint32_t d0[4] = {k0.x, k0.y, k0.z, k0.w};
  if constexpr (BITS == 2) {
    // x = 2 w + parity: parity 0 takes the even dimensions of code word w
    const uint32_t dw = d0[x >> 1];
    return (int)((x & 1) ? ((dw >> 2) & 0x33333333u) : (dw & 0x33333333u));
  } else if constexpr (BITS == 3) {
    // low two bits as at 2 bits, high bit from high-plane word w / 2 at
    // shift k = 2 (w & 1) + parity (the plane's element order)
    const uint32_t dw = d0[x >> 1];
    const uint32_t hw = (x >> 2) ? b.kh[r].y : b.kh[r].x;
    const int k = (((x >> 1) & 1) << 1) | (x & 1);
    const uint32_t lo2 = (x & 1) ? ((dw >> 2) & 0x33333333u) : (dw & 0x33333333u);
    return (int)(lo2 | (((hw >> k) & 0x11111111u) << 2));
  } else {
    static_assert(C::KQ == 2, "4-bit positions take two 16-byte words per lane");
    const uint4 k1 = b.kc[r][1];
    const uint32_t d1[4] = {k1.x, k1.y, k1.z, k1.w};
    return (int)((x < 4 ? d0[x & 3] : d1[x & 3]) ^ 0x88888888u);  // code - 8 as a signed nibble
  }
}

// QREG (one query head): the query's digit words are held in registers qd
// (16 words per lane, loaded once per wave); otherwise read from LDS per
// digit group.  At one wave per SIMD the LDS reads' latency is not hidden.
template <int BITS, int G, bool QREG>
__device__ __forceinline__ void process_sub(const SubBuf<BITS, G>& b, int pbase, int lo, int hi,
                                            const uint4 (*qd)[2], const uint32_t* qdw,
                                            const QueryRegs* qr, uint32_t* wsm, float* M,
                                            float* Lrun, float* Zrun, float (*O)[2]) {
  using C = SplitCfg<BITS, G>;
  const int lane = threadIdx.x & 63, half = lane & 1, tq = lane >> 1;

  // ---- scores (log2 domain); -inf outside [lo, hi).  Per digit group x of 8
  // dimensions the query's QDIG digit words come from LDS once and meet the
  // codes of every row; one accumulator per (row, head, digit).
  int acc[C::ROWS][G][QDIG];
#pragma unroll
  for (int r = 0; r < C::ROWS; ++r)
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
#pragma unroll
      for (int k = 0; k < QDIG; ++k) acc[r][gg][k] = 0;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    int X[C::ROWS];
#pragma unroll
    for (int r = 0; r < C::ROWS; ++r) X[r] = code_nibbles<BITS, G>(b, r, x);
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      uint4 L0, L1;
      if constexpr (QREG) {
        L0 = qd[x][0];
        L1 = qd[x][1];
      } else {
        const uint4* qx = (const uint4*)(qdw + (gg * 16 + half * 8 + x) * DIGP);
        L0 = qx[0];
        L1 = qx[1];
      }
      const uint32_t Lk[8] = {L0.x, L0.y, L0.z, L0.w, L1.x, L1.y, L1.z, L1.w};
#pragma unroll
      for (int r = 0; r < C::ROWS; ++r)
#pragma unroll
        for (int k = 0; k < QDIG; ++k)
          acc[r][gg][k] = __builtin_amdgcn_sdot8(X[r], (int)Lk[k], acc[r][gg][k], false);
    }
  }
  float sc[C::ROWS][G];
  float vs[C::ROWS], vz[C::ROWS];
#pragma unroll
  for (int r = 0; r < C::ROWS; ++r) {
    const int p = pbase + 32 * r + tq;
    const bool ok = p >= lo && p < hi;
    const float ks = f16_to_f32(b.ksz[r] & 0xFFFFu), kz = f16_to_f32(b.ksz[r] >> 16);
    const uint32_t vszr = ok ? b.vsz[r] : 0u;  // masked positions: scale and zero 0
    vs[r] = f16_to_f32(vszr & 0xFFFFu);
    vz[r] = f16_to_f32(vszr >> 16);
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      // sum_k acc_k 16^k in two exact halves of three digits (each below
      // 2^23), joined in float
      static_assert(QDIG == 6, "the digit join assumes six digits");
      const int dlo = acc[r][gg][0] + 16 * acc[r][gg][1] + 256 * acc[r][gg][2];
      const int dhi = acc[r][gg][3] + 16 * acc[r][gg][4] + 256 * acc[r][gg][5];
      float dot = fmaf((float)dhi, 4096.f, (float)dlo);
      if constexpr (BITS == 4) dot += 8.f * qr[gg].qsum;
      dot += __int_as_float(swap_adjacent(__float_as_int(dot)));
      sc[r][gg] = ok ? ks * (dot * qr[gg].inv) + kz * qr[gg].sig : -INFINITY;
    }
  }

  // ---- sub-chunk max, weights p = exp2(s - m) (even lanes), w = p s
  float m[G], pw[C::ROWS][G], wmax[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    m[gg] = -INFINITY;
#pragma unroll
    for (int r = 0; r < C::ROWS; ++r) m[gg] = fmaxf(m[gg], sc[r][gg]);
    m[gg] = wave_max(m[gg]);
    wmax[gg] = 0.f;
#pragma unroll
    for (int r = 0; r < C::ROWS; ++r) {
      pw[r][gg] = half ? 0.f : exp2_nonpos(sc[r][gg] - m[gg]);
      wmax[gg] = fmaxf(wmax[gg], pw[r][gg] * vs[r]);
    }
    wmax[gg] = wave_max(wmax[gg]);
  }
  uint32_t* wq = wsm;                 // [G][TW], positions of a row word grouped by parity
  uint32_t* wl = wsm + G * C::TW;     // [G][NG][WGP] digit words
  float lsum[G], zsum[G];
  wave_sync();  // the previous sub-chunk's reads of wq / wl are done
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float wscale = wmax[gg] > 0.f ? (float)WMAX * __builtin_amdgcn_rcpf(wmax[gg]) : 0.f;
    lsum[gg] = zsum[gg] = 0.f;
#pragma unroll
    for (int r = 0; r < C::ROWS; ++r) {
      const int t = 32 * r + tq;
      const int slot = C::SPLIT2 ? ((t & ~15) | ((t & 1) << 3) | ((t & 15) >> 1)) : t;
      lsum[gg] += pw[r][gg];
      zsum[gg] = fmaf(pw[r][gg], vz[r], zsum[gg]);
      if (!half) wq[gg * C::TW + slot] = (uint32_t)fminf(rintf(pw[r][gg] * vs[r] * wscale), (float)WMAX);
    }
    // lsum, zsum stay per-lane partials; the wave sums them once at its end
  }
  wave_sync();

  // ---- weight digit words: group gi of GS positions, digit k; nibble n holds
  // digit k of position n of the group's (parity) set
  for (int x = lane; x < G * C::NG * C::WGW; x += 64) {
    const int gg = x / (C::NG * C::WGW), rem = x % (C::NG * C::WGW);
    const int gi = rem / C::WGW, r2 = rem % C::WGW;
    const int par = C::SPLIT2 ? r2 / WDIG : 0, k = r2 % WDIG;
    const uint4* src = (const uint4*)(wq + gg * C::TW + gi * C::GS + par * 8);
    const uint4 s0 = src[0], s1 = src[1];
    const uint32_t wv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    uint32_t word = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) word |= ((wv[n] >> (4 * k)) & 15u) << (4 * n);
    wl[(gg * C::NG + gi) * C::WGP + par * WDIG + k] = word;
  }
  wave_sync();

  // ---- o_i = sum_t w_t c_{t,i}: lane = dimensions lane, lane + 64.  Value
  // codes of positions outside [lo, hi) meet zero weights.
  uint32_t pa[G][2][WDIG];
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int k = 0; k < WDIG; ++k) pa[gg][e][k] = 0u;
#pragma unroll
  for (int kb = 0; kb < C::NBW; ++kb) {
    const uint32_t rw[2][4] = {{b.vc[kb][0].x, b.vc[kb][0].y, b.vc[kb][0].z, b.vc[kb][0].w},
                               {b.vc[kb][1].x, b.vc[kb][1].y, b.vc[kb][1].z, b.vc[kb][1].w}};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int gi = kb * 4 + w;
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const uint4* W4 = (const uint4*)(wl + (gg * C::NG + gi) * C::WGP);
        uint32_t W[C::WGP];
#pragma unroll
        for (int q = 0; q < C::WGP / 4; ++q) {
          const uint4 t4 = W4[q];
          W[4 * q] = t4.x;
          W[4 * q + 1] = t4.y;
          W[4 * q + 2] = t4.z;
          W[4 * q + 3] = t4.w;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          if constexpr (C::SPLIT2) {
            uint32_t E = rw[e][w] & 0x33333333u, Od = (rw[e][w] >> 2) & 0x33333333u;
            if constexpr (BITS == 3) {
              // high bits of positions 16 w + 2 n (+ 1) of the sub-chunk:
              // word w / 2 of its half row, shifts 2 (w & 1) and 2 (w & 1) + 1
              const uint32_t hw = (w >> 1) ? b.vh[e].y : b.vh[e].x;
              const int k0 = (w & 1) << 1;
              E |= ((hw >> k0) & 0x11111111u) << 2;
              Od |= ((hw >> (k0 + 1)) & 0x11111111u) << 2;
            }
#pragma unroll
            for (int k = 0; k < WDIG; ++k) {
              pa[gg][e][k] = __builtin_amdgcn_udot8(E, W[k], pa[gg][e][k], false);
              pa[gg][e][k] = __builtin_amdgcn_udot8(Od, W[WDIG + k], pa[gg][e][k], false);
            }
          } else {
#pragma unroll
            for (int k = 0; k < WDIG; ++k)
              pa[gg][e][k] = __builtin_amdgcn_udot8(rw[e][w], W[k], pa[gg][e][k], false);
          }
        }
      }
    }
  }

  // ---- fold into the running (M, Lrun, O)
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float Mn = fmaxf(M[gg], m[gg]);
    const float fo = exp2_nonpos(M[gg] - Mn), fn = exp2_nonpos(m[gg] - Mn);
    const float back = wmax[gg] * (1.f / (float)WMAX);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float of = (float)pa[gg][e][WDIG - 1];
#pragma unroll
      for (int k = WDIG - 2; k >= 0; --k) of = fmaf(of, 16.f, (float)pa[gg][e][k]);
      O[gg][e] = fmaf(O[gg][e], fo, of * back * fn);
    }
    Lrun[gg] = fmaf(Lrun[gg], fo, lsum[gg] * fn);  // per-lane partial
    Zrun[gg] = fmaf(Zrun[gg], fo, zsum[gg] * fn);  // per-lane partial of sum p z
    M[gg] = Mn;
  }
}

// Issues the loads of a wave's first sub-chunk c0 into A.  The load is
// unconditional (a wave without sub-chunks loads sub-chunk 0, inside every
// unit): a load under a branch would leave the compiler's wait counts
// conservative where the branch joins, and waiting for the query inputs,
// issued before, would then wait for these codes too.
template <int BITS, int G, int CP = CPOL_NT>
__device__ __forceinline__ void load_first(SubBuf<BITS, G>& A, const DecodeArgs& a, const QMap& qm,
                                           int c0, int c_end, const uint8_t* spare) {
  using C = SplitCfg<BITS, G>;
  load_sub<BITS, G, CP>(A, a, qm, c0 < c_end ? c0 * C::TW : -1, spare);
}

// One wave, G query heads (scales qsc, digit words qdw): sub-chunks c0,
// c0 + stride, ... (< c_end) of the quantized region [lo, hi), two sub-chunks
// of codes in flight; leaves the partial (o[D], m, l) of head gg at
// out + gg * hstride.  On entry A and B hold (in flight) sub-chunks c0 and
// c0 + stride, both issued by the caller before the query preparation, so
// the loop starts with two sub-chunks on their way.  A third buffer measured
// slower at one wave per SIMD (86 against 79 us per 128K layer): more
// requests in flight do not pay on this access pattern.
template <int BITS, int G, int CP = CPOL_NT, bool QREG = false>
__device__ void quant_wave(const DecodeArgs& a, const QMap& qm, int c0, int stride, int c_end, int lo,
                           int hi, const float* qsc, const uint32_t* qdw, uint32_t* wsm, float* out,
                           int64_t hstride, SubBuf<BITS, G>& A, SubBuf<BITS, G>& B,
                           const uint8_t* spare) {
  using C = SplitCfg<BITS, G>;
  static_assert(!QREG || G == 1, "register digits for one head");
  const int lane = threadIdx.x & 63, half = lane & 1;
  uint4 qd[QREG ? 8 : 1][2];
  QueryRegs qr[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    qr[gg].sig = qsc[gg * 4];
    qr[gg].inv = qsc[gg * 4 + 1];
    qr[gg].qsum = qsc[gg * 4 + 2 + half];
  }
  if constexpr (QREG)
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      qd[x][0] = *(const uint4*)(qdw + (half * 8 + x) * DIGP);
      qd[x][1] = *(const uint4*)(qdw + (half * 8 + x) * DIGP + 4);
    }
  // running softmax state: M wave-uniform; Lrun and Zrun (sum of p z) per-lane
  // partials, O per dimension
  float M[G], Lrun[G], Zrun[G], O[G][2];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    M[gg] = -INFINITY;
    Lrun[gg] = Zrun[gg] = 0.f;
    O[gg][0] = O[gg][1] = 0.f;
  }
  int c = c0;
  // A buffer is refilled with the sub-chunk two steps ahead as soon as it has
  // been processed.  The loads are issued unconditionally (past the end they
  // read the spare block, from L2): a conditional load leaves the compiler's
  // wait counts conservative at the join, and it would then wait for the
  // prefetch before processing the next sub-chunk.
  while (c < c_end) {
    process_sub<BITS, G, QREG>(A, c * C::TW, lo, hi, qd, qdw, qr, wsm, M, Lrun, Zrun, O);
    __builtin_amdgcn_sched_barrier(0);
    load_sub<BITS, G, CP>(A, a, qm, c + 2 * stride < c_end ? (c + 2 * stride) * C::TW : -1, spare);
    c += stride;
    if (c >= c_end) break;
    process_sub<BITS, G, QREG>(B, c * C::TW, lo, hi, qd, qdw, qr, wsm, M, Lrun, Zrun, O);
    __builtin_amdgcn_sched_barrier(0);
    load_sub<BITS, G, CP>(B, a, qm, c + 2 * stride < c_end ? (c + 2 * stride) * C::TW : -1, spare);
    c += stride;
  }
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float Lw = wave_sum(Lrun[gg]);
    const float Zw = wave_sum(Zrun[gg]);  // zero-point term, the same for every dimension
    float* po = out + gg * hstride;       // o[D], m, l of head gg
    po[lane] = O[gg][0] + Zw;
    po[lane + 64] = O[gg][1] + Zw;
    if (lane == 0) {
      po[D] = M[gg];
      po[D + 1] = Lw;
    }
  }
}

// ---------------------------------------------------------------- quantized, int8 matrix cores

// Groups of 4 and 8 query heads.  A wave takes 64-position sub-chunks for
// all G heads of its KV head and contracts them on v_mfma_i32_16x16x64_i8:
//   scores  A = query digits, row 4 h + k holding digit k of head h's 24-bit
//           fixed-point query (three balanced base-256 digits, the same
//           integer query as the integer-dot path); B = key codes, column =
//           position.  Lane (m16, group) of the result then holds the three
//           digit sums of head `group` at position 16 cb + m16, joined in the
//           lane, and the 16 lanes of a row group share a head.
//   values  A = softmax-weight digits, row 4 h + k holding digit k of head h's
//           15-bit weight codes (with eight heads, rows 4 h + 2 and 4 h + 3
//           hold those of head h of the second tile); B = value codes,
//           column = dimension.  Lane (m16, group) of the result holds both
//           digit sums of head `group` (of each tile) at dimension 16 db + m16.
// Per 64 positions and four heads that is 8 + 8 matrix-core instructions (8 +
// 8 more score and no more value instructions for the second four heads);
// the vector work left is the code unpacking (shared by the heads), one
// softmax per (head, position) in the lanes that hold it, and the weights'
// transposition into the A layout through 512 bytes of LDS.

// Max / sum over the 16 lanes of a DPP row (every lane gets the result).
__device__ __forceinline__ float group16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  x = fmaxf(x, dpp_f<0x128>(x));
  return x;
}

// Max over the 16 lanes of a DPP row of a non-negative float: its bits as an
// unsigned integer are ordered the same, and an unsigned max (identity 0)
// folds each DPP move into the max (a float max needs two more operations per
// step to canonicalize its operand).
__device__ __forceinline__ float group16_max_nonneg(float x) {
  uint32_t v = __float_as_uint(x);
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  return __uint_as_float(v);
}

__device__ __forceinline__ float group16_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x128>(x);
  return x;
}

// Largest softmax-weight code: two balanced base-256 digits.
constexpr int W8MAX = 32639;

// Registers of one 64-position sub-chunk, lane = (m16 = lane % 16, group =
// lane / 16):
//   kc[cb]   key codes of position 16 cb + m16, dimensions 32 group .. + 31:
//            2 bits words 2 group, 2 group + 1 of the position's code row;
//            3 bits those low-plane words, and kh[cb] = high-plane word group;
//            4 bits words 4 group .. 4 group + 3
//   ksz, vsz scale/zero words of those four positions
//   vc[db]   value codes of dimension 16 db + m16, positions 16 group .. + 15
//            (3 bits: vh[db] = the high-plane word holding their high bits)
template <int BITS>
struct MBuf {
  static constexpr int KW = BITS == 4 ? 4 : 2;
  static constexpr int VW = BITS == 4 ? 2 : 1;
  uint32_t kc[4][KW];
  uint32_t kh[BITS == 3 ? 4 : 1];
  uint32_t ksz[4], vsz[4];
  uint32_t vc[8][VW];
  uint32_t vh[BITS == 3 ? 8 : 1];
};

// Issues the loads of the sub-chunk at position pbase (a multiple of 64, so
// its rows are consecutive and its value codes whole 16-byte row words);
// pbase < 0 loads from `spare` instead, as load_sub does.  One wave reads
// each sub-chunk, so the loads carry the non-temporal hint.
template <int BITS>
__device__ __forceinline__ void mload(MBuf<BITS>& b, const DecodeArgs& a, const QMap& qm, int pbase,
                                      const uint8_t* spare) {
  constexpr int CB = 16 * BITS;
  const int lane = threadIdx.x & 63, m16 = lane & 15, grp = lane >> 4;
  const bool past = pbase < 0;
  const int64_t row = qrow_read(qm, past ? 0 : pbase);
  const auto rk = wave_rsrc(past ? spare : a.pl.kcode + row * CB, 64 * CB);
  const auto rks = wave_rsrc(past ? (const void*)spare : (const void*)(a.pl.ksz + row), 64 * 4);
  const auto rvs = wave_rsrc(past ? (const void*)spare : (const void*)(a.pl.vsz + row), 64 * 4);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int ko = (16 * cb + m16) * CB;
    if constexpr (BITS == 4) {
      const uint4 v = buf_b128<CPOL_NT>(rk, ko + 16 * grp, 0);
      b.kc[cb][0] = v.x;
      b.kc[cb][1] = v.y;
      b.kc[cb][2] = v.z;
      b.kc[cb][3] = v.w;
    } else {
      const uint2 v = buf_b64<CPOL_NT>(rk, ko + 8 * grp, 0);
      b.kc[cb][0] = v.x;
      b.kc[cb][1] = v.y;
      if constexpr (BITS == 3) b.kh[cb] = __builtin_amdgcn_raw_buffer_load_b32(rk, ko + 32 + 4 * grp, 0, CPOL_NT);
    }
    b.ksz[cb] = __builtin_amdgcn_raw_buffer_load_b32(rks, 4 * (16 * cb + m16), 0, CPOL_NT);
    b.vsz[cb] = __builtin_amdgcn_raw_buffer_load_b32(rvs, 4 * (16 * cb + m16), 0, CPOL_NT);
  }
  if constexpr (BITS == 2) {
    // one 64-position row per dimension
    const auto rv = wave_rsrc(past ? spare : a.pl.vcode + (row >> 6) * D * 16, D * 16);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      b.vc[db][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, (16 * db + m16) * 16 + 4 * grp, 0, CPOL_NT);
  } else if constexpr (BITS == 4) {
    // two 32-position rows per dimension: this group's 16 positions are words
    // 2 (group % 2), + 1 of row group / 2
    const auto rv = wave_rsrc(past ? spare : a.pl.vcode + (row >> 5) * D * 16, 2 * D * 16);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint2 v = buf_b64<CPOL_NT>(rv, (grp >> 1) * D * 16 + (16 * db + m16) * 16 + 8 * (grp & 1), 0);
      b.vc[db][0] = v.x;
      b.vc[db][1] = v.y;
    }
  } else {
    // 128-position block: low-plane row sel (the sub-chunk's half) and the
    // high-plane row, whose bytes [8 sel, 8 sel + 8) belong to this half
    const int sel = (int)((row >> 6) & 1);
    const auto rv = wave_rsrc(past ? spare : a.pl.vcode + (row >> 7) * 3 * D * 16, 3 * D * 16);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      b.vc[db][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, (16 * db + m16) * 16 + 4 * grp, sel * D * 16, CPOL_NT);
      b.vh[db] = __builtin_amdgcn_raw_buffer_load_b32(rv, 2 * D * 16 + (16 * db + m16) * 16 + 4 * (grp >> 1),
                                                      8 * sel, CPOL_NT);
    }
  }
}

// One sub-chunk for NTL tiles of four heads: scores, weights and value sums,
// folded into the running state (M wave-uniform per row group, Lp and Zp
// per-lane partials, O per lane's dimensions 16 db + m16).  wl is the wave's
// weight staging ([tile][head][group][16] 16-bit codes), wsel the byte
// selector that takes this lane's digit (row % 4) of four codes.
template <int BITS, int NTL>
__device__ __forceinline__ void mprocess(const MBuf<BITS>& b, int pbase, int lo, int hi,
                                         const v4i (&Aq)[NTL][2], const float (&sig)[NTL],
                                         const float (&inv)[NTL], uint16_t* wl, uint32_t wsel,
                                         float (&M)[NTL], float (&Lp)[NTL], float (&Zp)[NTL],
                                         float (&O)[NTL][8]) {
  const int lane = threadIdx.x & 63, m16 = lane & 15, grp = lane >> 4;
  // ---- scores (log2 domain), -inf outside [lo, hi).  Every matrix-core
  // product is issued before the first result is read, and the mask is
  // arithmetic (a branch per position would make the scheduler wait out
  // each product's latency in turn).
  v4i acc[NTL][4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    v4i k0, k1;  // dimensions 32 group + [0, 16) and + [16, 32)
    if constexpr (BITS == 2) {
      k0 = unpack2(b.kc[cb][0]);
      k1 = unpack2(b.kc[cb][1]);
    } else if constexpr (BITS == 3) {
      k0 = unpack3(b.kc[cb][0], b.kh[cb], 0);
      k1 = unpack3(b.kc[cb][1], b.kh[cb], 2);
    } else {
      k0 = unpack4(b.kc[cb][0], b.kc[cb][1]);
      k1 = unpack4(b.kc[cb][2], b.kc[cb][3]);
    }
#pragma unroll
    for (int t = 0; t < NTL; ++t) acc[t][cb] = mfma8(Aq[t][1], k1, mfma8(Aq[t][0], k0, v4i{0, 0, 0, 0}));
  }
  float ksv[4], kzv[4], vsv[4], vzv[4], lim[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int p = pbase + 16 * cb + m16;
    const bool ok = p >= lo && p < hi;
    lim[cb] = ok ? INFINITY : -INFINITY;
    ksv[cb] = f16_to_f32(b.ksz[cb] & 0xFFFFu);
    kzv[cb] = f16_to_f32(b.ksz[cb] >> 16);
    const uint32_t vw = ok ? b.vsz[cb] : 0u;  // masked positions: scale and zero 0
    vsv[cb] = f16_to_f32(vw & 0xFFFFu);
    vzv[cb] = f16_to_f32(vw >> 16);
  }
  float s[NTL][4];
#pragma unroll
  for (int t = 0; t < NTL; ++t)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      // 256 d2 + d1 fits in 32 bits (below 2^24, exact as a float, at 2
      // bits; one more rounding of relative size 2^-24 at 3 and 4 bits)
      const v4i& d = acc[t][cb];
      const float dot = fmaf((float)(d[2] * 256 + d[1]), 256.f, (float)d[0]);
      // fminf with -inf masks (also a NaN score from a masked position's
      // stale scale/zero), with +inf keeps the score
      s[t][cb] = fminf(fmaf(ksv[cb], dot * inv[t], kzv[cb] * sig[t]), lim[cb]);
    }
  // ---- per head: the new running maximum M' = max(M, sub-chunk max) is the
  // reference, p = exp2(s - M'), w = p s_v.  Once the running maxima settle
  // no score exceeds them, M' = M, and the reduction over the head's lanes
  // is skipped.
  float fo[NTL], wm[NTL], ls[NTL], zs[NTL], w[NTL][4];
  {
    float lm[NTL];
    bool above = false;
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      lm[t] = fmaxf(fmaxf(s[t][0], s[t][1]), fmaxf(s[t][2], s[t][3]));
      above = above || lm[t] > M[t];
    }
    if (__any(above)) {
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const float Mn = fmaxf(M[t], group16_max(lm[t]));
        fo[t] = exp2_nonpos(M[t] - Mn);
        M[t] = Mn;
      }
    } else {
#pragma unroll
      for (int t = 0; t < NTL; ++t) fo[t] = 1.f;
    }
  }
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
    wm[t] = ls[t] = zs[t] = 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const float p = exp2_nonpos(s[t][cb] - M[t]);
      w[t][cb] = p * vsv[cb];
      ls[t] += p;
      zs[t] = fmaf(p, vzv[cb], zs[t]);
      wm[t] = fmaxf(wm[t], w[t][cb]);
    }
    wm[t] = group16_max_nonneg(wm[t]);
  }
  // ---- weight codes into the A layout: this lane's code of (head group,
  // position 16 cb + m16) goes to slot (operand byte of m16) of block
  // [tile][group][cb]; lane (row, group) then reads block [tile][row / 4]
  // [group] and keeps digit row % 4 (low byte: low digit)
  const int eb = opnd_byte_b<BITS>(m16);
  wave_sync();  // the previous sub-chunk's reads of wl are done
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
    const float wsc = wm[t] > 0.f ? (float)W8MAX * __builtin_amdgcn_rcpf(wm[t]) : 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      // wq = w wsc rounded to the nearest integer (ties to even), at most
      // W8MAX: added to 1.5 * 2^23 in one rounding, it sits in the low bits
      // of the float (whose bits are 0x4B400000 + wq)
      const uint32_t rb = __float_as_uint(fminf(fmaf(w[t][cb], wsc, 12582912.f), 12582912.f + (float)W8MAX));
      // balanced digits lo = ((wq + 128) & 255) - 128, hi = (wq + 128) >> 8
      // as two's-complement bytes: the low byte is wq & 255 (the 16-bit store
      // drops the bits above)
      wl[((t * 4 + grp) * 4 + cb) * 16 + eb] = (uint16_t)((((rb + 128u) ^ rb) & 0xFF00u) ^ rb);
    }
  }
  wave_sync();
  static_assert(NTL == 1 || NTL == 2, "one or two tiles of four heads");
  // One operand for both tiles at NTL = 2: row 4 h + k holds digit k % 2 of
  // head h of tile k / 2 (one value product per dimension block for all
  // eight heads); at NTL = 1 rows 4 h + 2, 4 h + 3 are zero.
  v4i W;
  {
    const int tsel = NTL == 2 ? (m16 >> 1) & 1 : 0;
    const uint4* src = (const uint4*)(wl + ((tsel * 4 + (m16 >> 2)) * 4 + grp) * 16);
    const uint4 x0 = src[0], x1 = src[1];
    W[0] = (int)__builtin_amdgcn_perm(x0.y, x0.x, wsel);
    W[1] = (int)__builtin_amdgcn_perm(x0.w, x0.z, wsel);
    W[2] = (int)__builtin_amdgcn_perm(x1.y, x1.x, wsel);
    W[3] = (int)__builtin_amdgcn_perm(x1.w, x1.z, wsel);
  }
  // ---- online softmax fold and o += w c
  float back[NTL];
  bool settled = true;
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
    back[t] = wm[t] * (1.f / (float)W8MAX);
    Lp[t] = fmaf(Lp[t], fo[t], ls[t]);
    Zp[t] = fmaf(Zp[t], fo[t], zs[t]);
    settled = settled && fo[t] == 1.f;
  }
  // once the running maxima settle (the common case) no rescale is needed
  if (!__all(settled)) {
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
      for (int db = 0; db < 8; ++db) O[t][db] *= fo[t];
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    v4i vb;
    if constexpr (BITS == 2) vb = unpack2(b.vc[db][0]);
    else if constexpr (BITS == 3) vb = unpack3(b.vc[db][0], b.vh[db], 2 * (grp & 1));
    else vb = unpack4(b.vc[db][0], b.vc[db][1]);
    const v4i pv = mfma8(W, vb, v4i{0, 0, 0, 0});
#pragma unroll
    for (int t = 0; t < NTL; ++t)
      O[t][db] = fmaf((float)(pv[2 * t + 1] * 256 + pv[2 * t]), back[t], O[t][db]);
  }
}

// One wave, all G = 4 NTL heads: sub-chunks c0, c0 + 4, ... (< c_end) of the
// quantized region [lo, hi), two in flight (A and B hold c0 and c0 + 4 on
// entry, issued by the caller before the query preparation); leaves the
// partial (o[D], m, l) of head gg at out + gg (D + 2).
// A lane's query operands (NTL tiles x 2 halves of the dimensions) and its
// head's sigma and 1/S_q, from a query block's scales qsc and operand words
// qop (in LDS, or in global memory as the prep kernel wrote them).
template <int NTL>
struct MQuery {
  v4i A[NTL][2];
  float sig[NTL], inv[NTL];
};

template <int NTL>
__device__ __forceinline__ void mquery_load(MQuery<NTL>& q, const float* qsc, const uint32_t* qop) {
  const int lane = threadIdx.x & 63, grp = lane >> 4;
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) q.A[t][ks] = ((const v4i*)qop)[(2 * t + ks) * 64 + lane];
    q.sig[t] = qsc[(4 * t + grp) * 4];
    q.inv[t] = qsc[(4 * t + grp) * 4 + 1];
  }
}

template <int BITS, int NTL>
__device__ void mquant_wave(const DecodeArgs& a, const QMap& qm, int c0, int c_end, int lo, int hi,
                            const MQuery<NTL>& qy, uint16_t* wl, float* out, MBuf<BITS>& A,
                            MBuf<BITS>& B, const uint8_t* spare) {
  constexpr int MT = 64;
  const int lane = threadIdx.x & 63, m16 = lane & 15, grp = lane >> 4;
  // the byte selector of this lane's weight digit: low or high byte of four
  // 16-bit codes (NTL = 1: rows 4 h + 2, 4 h + 3 take zeros)
  const int wd = NTL == 2 ? m16 & 1 : m16 & 3;
  const uint32_t wsel = wd == 0 ? 0x06040200u : (wd == 1 ? 0x07050301u : 0x0C0C0C0Cu);
  float M[NTL], Lp[NTL], Zp[NTL], O[NTL][8];
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
    M[t] = -INFINITY;
    Lp[t] = Zp[t] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) O[t][db] = 0.f;
  }
  // as in quant_wave: a buffer is refilled with the sub-chunk two steps
  // ahead as soon as it has been processed, unconditionally
  int c = c0;
  while (c < c_end) {
    mprocess<BITS, NTL>(A, c * MT, lo, hi, qy.A, qy.sig, qy.inv, wl, wsel, M, Lp, Zp, O);
    __builtin_amdgcn_sched_barrier(0);
    mload<BITS>(A, a, qm, c + 8 < c_end ? (c + 8) * MT : -1, spare);
    c += 4;
    if (c >= c_end) break;
    mprocess<BITS, NTL>(B, c * MT, lo, hi, qy.A, qy.sig, qy.inv, wl, wsel, M, Lp, Zp, O);
    __builtin_amdgcn_sched_barrier(0);
    mload<BITS>(B, a, qm, c + 8 < c_end ? (c + 8) * MT : -1, spare);
    c += 4;
  }
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
    const float Lw = group16_sum(Lp[t]);
    const float Zw = group16_sum(Zp[t]);  // zero-point term, the same for every dimension
    float* po = out + (4 * t + grp) * (D + 2);
#pragma unroll
    for (int db = 0; db < 8; ++db) po[16 * db + m16] = O[t][db] + Zw;
    if (m16 == 0) {
      po[D] = M[t];
      po[D + 1] = Lw;
    }
  }
}

// Log-sum-exp merge of the four waves' partials part[wave][G][D + 2] (a wave
// without sub-chunks has l = 0): o into obuf, m and l per head.
template <int G>
__device__ __forceinline__ void merge_waves(const float* part, float* obuf, float (&m)[G], float (&l)[G]) {
  const int tid = threadIdx.x, i = tid & (D - 1), hf = tid >> 7;
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    float Mx = -INFINITY;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float* px = part + (x * G + gg) * (D + 2);
      if (px[D + 1] > 0.f) Mx = fmaxf(Mx, px[D]);
    }
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float* px = part + (x * G + gg) * (D + 2);
      const float f = px[D + 1] > 0.f ? exp2f(px[D] - Mx) : 0.f;
      lsum = fmaf(px[D + 1], f, lsum);
      o = fmaf(px[i], f, o);
    }
    if (hf == 0) obuf[gg * D + i] = o;
    m[gg] = Mx;
    l[gg] = lsum;
  }
}

// ---------------------------------------------------------------- decode step

template <int IO_BF16>
__device__ __forceinline__ uint16_t io_to_bf16(const void* base, int64_t idx) {
  if (IO_BF16) return ((const uint16_t*)base)[idx];
  return f32_to_bf16(((const float*)base)[idx]);
}

// The new position's entries as bfloat16 bits in LDS: k' = T_K k in fp64
// (the arithmetic of transform_entry, shared by every append path, so all
// store identical bits) with one rounding, and v rounded to bfloat16.  Thread
// (i, hf) computes the two chains of row i over dimensions [64 hf, 64 hf + 64)
// (chains 2 hf and 2 hf + 1) and their sum; row i's entry is then
// (s0 + s1) + (s2 + s3), the same operations in the same order.  All loads
// are issued before the first wait.
template <int IO_BF16, int BITS, int G>
__device__ void new_entry(const DecodeArgs& a, int h, int si, uint32_t* sm) {
  using C = SplitCfg<BITS, G>;
  float* kin = (float*)(sm + C::O_UNION);
  double* hs = (double*)(kin + D);  // [2][D] half sums
  uint16_t* knew = (uint16_t*)(sm + C::O_UNION + C::O_NEW);
  uint16_t* vnew = knew + D;
  const int tid = threadIdx.x, i = tid & (D - 1), hf = tid >> 7;
  const int64_t row = ((int64_t)si * a.g.n_kv + h) * D;
  // every thread loads both (no load under a branch, whose join would wait
  // for it and, in order, for every load issued before)
  const float x = load_io<IO_BF16>(a.k_new, row + i);
  const uint16_t vb = io_to_bf16<IO_BF16>(a.v_new, row + i);
  float t[64];
  const float4* tp = (const float4*)(a.tk + ((int64_t)h * D + i) * D + 64 * hf);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const float4 t4 = tp[c];
    t[4 * c] = t4.x;
    t[4 * c + 1] = t4.y;
    t[4 * c + 2] = t4.z;
    t[4 * c + 3] = t4.w;
  }
  if (hf == 0)
    kin[i] = x;
  else
    vnew[i] = vb;
  __syncthreads();
  double s0 = 0.0, s1 = 0.0;
#pragma unroll
  for (int j = 0; j < D / 4; ++j) {
    s0 = fma((double)t[j], (double)kin[64 * hf + j], s0);
    s1 = fma((double)t[32 + j], (double)kin[64 * hf + 32 + j], s1);
  }
  hs[hf * D + i] = s0 + s1;
  __syncthreads();
  if (tid < D) knew[tid] = f64_to_bf16(hs[tid] + hs[D + tid]);
  __syncthreads();
}

// After the window partial is written: quantize the ring entries leaving the
// recent window at length Lq ([sq, squant(Lq)) minus the new position), then
// store the new entry in the sink, the ring or, when the window has no room
// for it, as codes.  Threads 0..127 handle key dimensions, 128..255 value
// dimensions.
template <int BITS, int G>
__device__ void step_append(const DecodeArgs& a, int64_t unit, const QMap& qm, int Lq, int sq,
                            uint32_t* sm, uint16_t first) {
  using C = SplitCfg<BITS, G>;
  const Geometry& g = a.g;
  const int tid = threadIdx.x, i = tid & (D - 1);
  const bool is_v = tid >= D;
  const int L0 = Lq - 1;
  const int sq1 = squant_of(Lq, g.S, g.R, g.F);
  QLds& ql = *(QLds*)(sm + C::O_UNION);
  const uint16_t* knew = (const uint16_t*)(sm + C::O_UNION + C::O_NEW);
  const uint16_t* vnew = knew + D;
  VRows vr;
  vrows_init(vr);
  __syncthreads();  // window scores in the union are dead
  const int e1 = sq1 < L0 ? sq1 : L0;
  for (int p = sq; p < e1; ++p) {
    const int64_t row = (unit * g.W + (p - g.S) % g.W) * D + i;
    // the first leaving entry was read at the window workgroup's start
    const float x = bf16_bits_to_f32(p == sq ? first : (is_v ? a.pl.vring[row] : a.pl.kring[row]));
    store_quantized<BITS == 3>(p, x, x, ql, vr, a.pl, qm, g);
  }
  __syncthreads();  // ring reads above complete before the ring write below
  const uint16_t nb = is_v ? vnew[i] : knew[i];
  if (L0 < g.S) {
    const int64_t o = (unit * g.S + L0) * D + i;
    (is_v ? a.pl.vsink : a.pl.ksink)[o] = nb;
  } else if (L0 >= sq1) {
    const int64_t o = (unit * g.W + (L0 - g.S) % g.W) * D + i;
    (is_v ? a.pl.vring : a.pl.kring)[o] = nb;
  } else {
    const float x = bf16_bits_to_f32(nb);
    store_quantized<BITS == 3>(L0, x, x, ql, vr, a.pl, qm, g);
  }
  vrows_flush<BITS == 3>(vr, a.pl);
}

// ---------------------------------------------------------------- window

template <int BITS, int G>
__device__ void window_chunk(const DecodeArgs& a, int64_t unit, int Lq, int sq, uint32_t* sm,
                             float (&m_out)[G], float (&l_out)[G]) {
  using C = SplitCfg<BITS, G>;
  const Geometry& g = a.g;
  const int tid = threadIdx.x, half = tid & 1, lane = tid & 63, wv = tid >> 6;
  const float* qs = (const float*)(sm + C::O_QF);
  float* obuf = (float*)(sm + C::O_OBUF);
  float* red = (float*)(sm + C::O_RED);
  float* scw = (float*)(sm + C::O_UNION);  // [G][WINDOW_MAX]
  const uint16_t* knew = (const uint16_t*)(sm + C::O_UNION + C::O_NEW);
  const uint16_t* vnew = knew + D;
  float* part = (float*)(sm + C::O_UNION + C::O_WPART);  // [4 waves][G][D]
  const int ns = Lq < g.S ? Lq : g.S;
  const int ntok = ns + (Lq > sq ? Lq - sq : 0);
  // decode step: the newest position is read from LDS
  const int pnew = a.k_new ? Lq - 1 : -1;
  auto row_of = [&](int tok, const uint16_t* sink, const uint16_t* ring,
                    const uint16_t* nw) -> const uint16_t* {
    const int p = tok < ns ? tok : sq + (tok - ns);
    return p == pnew ? nw
           : tok < ns ? sink + (unit * g.S + p) * D
                      : ring + (unit * g.W + (p - g.S) % g.W) * D;
  };

  // G <= 2: the value rows of the first PV round (tokens 0..127) in flight
  // with the key rows, so the PV starts without another round trip (with
  // more heads the registers are needed by the scores)
  const int dg = tid & 15, tl = tid >> 4;
  uint4 vb0[G <= 2 ? 8 : 1];
  if constexpr (G <= 2) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int tok = 16 * r + tl;
      vb0[r] = tok < ntok ? ((const uint4*)row_of(tok, a.pl.vsink, a.pl.vring, vnew))[dg]
                          : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // ---- scores: a lane pair per token (64 dimensions each)
  if constexpr (G <= 2) {
    // two tokens per pair with all their loads in flight together
    for (int base = 0; base < ntok; base += 256) {
      uint4 kb[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tok = base + 128 * u + (tid >> 1);
        if (tok < ntok) {
          const uint4* s4 = (const uint4*)(row_of(tok, a.pl.ksink, a.pl.kring, knew) + half * 64);
#pragma unroll
          for (int c = 0; c < 8; ++c) kb[u][c] = s4[c];
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tok = base + 128 * u + (tid >> 1);
        if (tok < ntok) {  // uniform within a lane pair
          float dot[G];
#pragma unroll
          for (int gg = 0; gg < G; ++gg) dot[gg] = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint32_t ww[4] = {kb[u][c].x, kb[u][c].y, kb[u][c].z, kb[u][c].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = bf16_to_f32((uint16_t)(ww[e >> 1] >> ((e & 1) * 16)));
#pragma unroll
              for (int gg = 0; gg < G; ++gg)
                dot[gg] = fmaf(qs[gg * D + half * 64 + c * 8 + e], x, dot[gg]);
            }
          }
#pragma unroll
          for (int gg = 0; gg < G; ++gg) {
            const float d2 = dot[gg] + __int_as_float(swap_adjacent(__float_as_int(dot[gg])));
            if (!half) scw[gg * WINDOW_MAX + tok] = d2;
          }
        }
      }
    }
  } else {
    // many heads: the pair's 64 key values in registers, one head at a time
    for (int tok = tid >> 1; tok < ntok; tok += 128) {  // uniform within a lane pair
      const uint4* s4 = (const uint4*)(row_of(tok, a.pl.ksink, a.pl.kring, knew) + half * 64);
      float xk[64];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 k4 = s4[c];
        const uint32_t ww[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) xk[8 * c + e] = bf16_to_f32((uint16_t)(ww[e >> 1] >> ((e & 1) * 16)));
      }
#pragma unroll 1
      for (int gg = 0; gg < G; ++gg) {
        const float* qg = qs + gg * D + half * 64;
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < 64; ++j) dot = fmaf(qg[j], xk[j], dot);
        const float d2 = dot + __int_as_float(swap_adjacent(__float_as_int(dot)));
        if (!half) scw[gg * WINDOW_MAX + tok] = d2;
      }
    }
  }
  __syncthreads();
  float mx[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    mx[gg] = -INFINITY;
    for (int t = tid; t < ntok; t += 256) mx[gg] = fmaxf(mx[gg], scw[gg * WINDOW_MAX + t]);
  }
  block_reduce<G, true>(mx, red);
  float ls[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    ls[gg] = 0.f;
    for (int t = tid; t < ntok; t += 256) {
      const float p = exp2f(scw[gg * WINDOW_MAX + t] - mx[gg]);
      ls[gg] += p;
      scw[gg * WINDOW_MAX + t] = p;
    }
  }
  block_reduce<G, false>(ls, red);  // its barriers also publish the weights

  // ---- o = sum_t p_t v_t: thread = (8 dimensions, token lane of 16); eight
  // rows per thread in flight per round of 128 tokens
  float acc[G][8];
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[gg][e] = 0.f;
  for (int base = 0; base < ntok; base += 128) {
    uint4 vb[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int tok = base + 16 * r + tl;
      if (G <= 2 && base == 0)
        vb[r] = vb0[G <= 2 ? r : 0];
      else
        vb[r] = tok < ntok ? ((const uint4*)row_of(tok, a.pl.vsink, a.pl.vring, vnew))[dg]
                           : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int tok = base + 16 * r + tl;
      if (tok < ntok) {
        const uint32_t ww[4] = {vb[r].x, vb[r].y, vb[r].z, vb[r].w};
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const float pw = scw[gg * WINDOW_MAX + tok];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[gg][e] = fmaf(pw, bf16_to_f32((uint16_t)(ww[e >> 1] >> ((e & 1) * 16))), acc[gg][e]);
        }
      }
    }
  }
  // the four token lanes of a wave are 16 lanes apart
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[gg][e] += __shfl_xor(acc[gg][e], 16);
      acc[gg][e] += __shfl_xor(acc[gg][e], 32);
    }
  if (lane < 16)
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
#pragma unroll
      for (int e = 0; e < 8; ++e) part[(wv * G + gg) * D + dg * 8 + e] = acc[gg][e];
  __syncthreads();
  if (tid < D)
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
      obuf[gg * D + tid] = (part[gg * D + tid] + part[(G + gg) * D + tid]) +
                           (part[(2 * G + gg) * D + tid] + part[(3 * G + gg) * D + tid]);
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    m_out[gg] = mx[gg];
    l_out[gg] = ls[gg];
  }
}

// ---------------------------------------------------------------- query block

// A thread's share of one (sequence, KV head) query block (16-byte words).
template <int G>
struct PrepIn {
  uint4 v[(prep_words(G) / 4 + 255) / 256];
};

// Issues the loads of unit u's query block.  Callers issue their first code
// loads after this, so that waiting for the block does not wait for the codes.
template <int G>
__device__ __forceinline__ void prep_load(const DecodeArgs& a, int u, PrepIn<G>& in) {
  const uint4* src = (const uint4*)(a.prep + (int64_t)u * prep_words(G));
#pragma unroll
  for (int n = 0; n < (prep_words(G) / 4 + 255) / 256; ++n) {
    const int x = (int)threadIdx.x + 256 * n;
    in.v[n] = x < prep_words(G) / 4 ? src[x] : make_uint4(0u, 0u, 0u, 0u);
  }
}

// Places the block in LDS where the query preparation leaves it: q', scales
// and digit words from O_QF on, the new entry at O_UNION + O_NEW.
template <int BITS, int G>
__device__ __forceinline__ void prep_store(uint32_t* sm, const PrepIn<G>& in) {
  using C = SplitCfg<BITS, G>;
  constexpr int NQ4 = (prep_words(G) - D) / 4;
#pragma unroll
  for (int n = 0; n < (prep_words(G) / 4 + 255) / 256; ++n) {
    const int x = (int)threadIdx.x + 256 * n;
    if (x < NQ4)
      ((uint4*)(sm + C::O_QF))[x] = in.v[n];
    else if (x < prep_words(G) / 4)
      ((uint4*)(sm + C::O_UNION + C::O_NEW))[x - NQ4] = in.v[n];
  }
  __syncthreads();
}

// ---------------------------------------------------------------- kernels

// One workgroup per (KV head, sequence): the query preparation of the split
// kernel done once per unit (q' = T_K^{-T} q and its digit words; in a decode
// step also the new entry, T_K k and v in bfloat16), written to the unit's
// query block for every split workgroup to copy.
template <int IO_BF16, int BITS, int G>
__global__ __launch_bounds__(256) void prep_kernel(DecodeArgs a) {
  using C = SplitCfg<BITS, G>;
  extern __shared__ uint4 smem4[];
  // T_K^{-T} of the head, rows padded to D + 4 floats (a lane's 16-byte
  // reads of rows i, i + 1, ... then fall in different banks)
  constexpr int TR = D + 4;
  __shared__ __align__(16) float tl[D * TR];
  uint32_t* sm = (uint32_t*)smem4;
  const int h = blockIdx.x, si = blockIdx.y, tid = threadIdx.x;
  QueryIn<G> qin;
  // The matrix in whole 16-byte chunks, chunk x = tid + 256 c (row x / 32):
  // every load instruction of a wave reads two whole rows (compensate_load's
  // layout has each lane read its own row, 64 rows per instruction), then
  // each thread takes its half row from LDS.
  {
    const float4* tg = (const float4*)(a.tq + (int64_t)h * D * D);
    float4 tv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) tv[c] = tg[tid + 256 * c];
    compensate_load_q<IO_BF16, G>(a, h, si, qin);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int x = tid + 256 * c;
      *(float4*)(tl + (x >> 5) * TR + 4 * (x & 31)) = tv[c];
    }
    __syncthreads();
    const float* tr = tl + (tid & (D - 1)) * TR + 64 * (tid >> 7);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const float4 t4 = *(const float4*)(tr + 4 * c);
      qin.t[4 * c] = t4.x;
      qin.t[4 * c + 1] = t4.y;
      qin.t[4 * c + 2] = t4.z;
      qin.t[4 * c + 3] = t4.w;
    }
  }
  // (G >= 4: the split kernel's window workgroup transforms the new entry,
  // which keeps this launch's chain short)
  if (!C::HS && a.k_new) new_entry<IO_BF16, BITS, G>(a, h, si, sm);
  compensate_query<IO_BF16, BITS, G>(a, h, si, sm, qin);
  uint4* dst = (uint4*)(a.prep + (int64_t)(si * a.g.n_kv + h) * prep_words(G));
  constexpr int NQ4 = (prep_words(G) - D) / 4;
  for (int x = threadIdx.x; x < prep_words(G) / 4; x += 256)
    dst[x] = x < NQ4 ? ((const uint4*)(sm + C::O_QF))[x]
                     : ((const uint4*)(sm + C::O_UNION + C::O_NEW))[x - NQ4];
}


// First sub-chunk (relative) of workgroup j's run when one workgroup per CU
// shares out nsub sub-chunks: workgroup 0 weighs LIGHT / 16 of the others.
constexpr int LIGHT = 14;
__device__ __forceinline__ int run_start(int64_t nsub, int j, int n) {
  if (j == 0) return 0;
  const int64_t total = LIGHT + 16 * (int64_t)(n - 1);
  return (int)((nsub * (LIGHT + 16 * (int64_t)(j - 1))) / total);
}

// Waves per SIMD the register allocation must allow: three at G = 4 with the
// query block from the prep kernel (the matrix-core path then needs 123-168
// registers, so four fit at 2 bits), two otherwise (G <= 2 keeps two sub-chunks of codes and the
// query digits in registers; G = 8, and the in-workgroup query preparation
// with two sub-chunks' loads in flight, need more than 168).
template <int G, bool PREP>
constexpr int split_waves() { return G == 4 && PREP ? 3 : 2; }

// PREP: the query block comes from the prep kernel (else every workgroup
// prepares the query itself).
template <int IO_BF16, int BITS, int G, bool PREP>
__global__ __launch_bounds__(256, (split_waves<G, PREP>())) void split_kernel(DecodeArgs a) {
  using C = SplitCfg<BITS, G>;
  extern __shared__ uint4 smem4[];
  uint32_t* sm = (uint32_t*)smem4;
  float* obuf = (float*)(sm + C::O_OBUF);

  const Geometry& g = a.g;
  const int tid = threadIdx.x;
  const int nsp = a.n_splits + 1;  // workgroups per (sequence, KV head)
  // Block order: the window workgroups first (dispatched first, they are the
  // oldest waves on their SIMDs and win issue arbitration, which keeps their
  // serial chain short), then the quantized workgroups unit by unit.
  int j, u;
  int nsu = a.n_splits;  // this unit's quantized workgroups
  const int units = a.n_seq * a.g.n_kv;
  if (a.balanced) {
    if ((int)blockIdx.x < units) {
      u = blockIdx.x;
      j = a.n_splits;
    } else {
      // the last sequence whose range starts at or before r (sequences
      // without quantized workgroups have empty ranges)
      const int r = blockIdx.x - units;
      int s0 = 0, s1 = a.n_seq;
      while (s1 - s0 > 1) {
        const int mid = (s0 + s1) >> 1;
        if (a.s.wg0[mid] <= r) s0 = mid;
        else s1 = mid;
      }
      nsu = (a.s.wg0[s0 + 1] - a.s.wg0[s0]) / a.g.n_kv;
      const int rr = r - a.s.wg0[s0];
      u = s0 * a.g.n_kv + rr / nsu;
      j = rr % nsu;
    }
  } else if (a.contig == 2) {
    // One quantized workgroup per CU: the quantized workgroups first, so that
    // the dispatcher spreads them one per CU, then the window workgroups.
    // Block b < units is unit b's workgroup 0, which takes a smaller share of
    // the sub-chunks: the dispatcher wraps the window workgroups, dispatched
    // last, onto the CUs of the first quantized workgroups of each XCD, and
    // those CUs carry the window's loads as well.
    const int nq = units * a.n_splits, b = blockIdx.x;
    if (b >= nq) {
      j = a.n_splits;
      u = a.xcd_map ? (b & 7) + 8 * ((b - nq) >> 3) : b - nq;
    } else if (b < units) {
      j = 0;
      u = b;
    } else {
      const int r = a.xcd_map ? (b - units) >> 3 : b - units;
      u = a.xcd_map ? (b & 7) + 8 * (r / (a.n_splits - 1)) : r / (a.n_splits - 1);
      j = 1 + r % (a.n_splits - 1);
    }
  } else if (a.xcd_map) {
    const int r = blockIdx.x >> 3, ng = units >> 3;
    if (r < ng) {
      u = (blockIdx.x & 7) + 8 * r;
      j = a.n_splits;
    } else {
      u = (blockIdx.x & 7) + 8 * ((r - ng) / a.n_splits);
      j = (r - ng) % a.n_splits;
    }
  } else if ((int)blockIdx.x < units) {
    u = blockIdx.x;
    j = a.n_splits;
  } else {
    u = (blockIdx.x - units) / a.n_splits;
    j = (blockIdx.x - units) % a.n_splits;
  }
  const int h = u % g.n_kv, si = u / g.n_kv;
  const int slot = a.s.slot[si], Lq = a.s.len[si], sq = a.s.squant[si];
  const int64_t unit = ((int64_t)a.layer * g.max_batch + slot) * g.n_kv + h;
  const QMap qm = qmap_of(g, a.layer, slot, h);
  const int qbase = si * g.n_q + h * G;
  // this head's T_K^{-T} (64 KB, read by the query preparation): the target
  // of the prefetches past a wave's last sub-chunk
  const uint8_t* spare = (const uint8_t*)(a.tq + (int64_t)h * D * D);

  // the quantized region [S, sq) in sub-chunks of TW positions, spread over
  // the 4 n_splits waves of this (sequence, KV head): interleaved (wave k
  // takes k, k + nw, ...), one contiguous run per wave, or one contiguous run
  // per workgroup shared out among its waves
  const int lo = g.S, hi = sq;
  const int c_first = lo / C::TW;
  const int c_end = hi > lo ? (hi + C::TW - 1) / C::TW : c_first;
  const int nw = 4 * a.n_splits;
  const int64_t nsub = c_end - c_first;
  // matrix-core path (G >= 4): workgroup j takes the contiguous run [mr0,
  // mr1) of the unit's 64-position sub-chunks, which its waves share out in
  // turn (k, k + 4, ...)
  const int mc_first = lo / C::MT, mc_end = hi > lo ? (hi + C::MT - 1) / C::MT : mc_first;
  const int64_t mnsub = mc_end - mc_first;
  const int nsd = nsu > 0 ? nsu : 1;
  const int mr0 = j < nsu ? mc_first + (int)((mnsub * j) / nsd) : mc_first;
  const int mr1 = j < nsu ? mc_first + (int)((mnsub * (j + 1)) / nsd) : mc_first;
  bool empty;
  if (j == a.n_splits) {
    const int ns = Lq < g.S ? Lq : g.S;
    empty = ns + (Lq > sq ? Lq - sq : 0) == 0;
  } else if (C::HS) {
    empty = mr1 == mr0;
  } else if (a.contig == 1) {
    empty = (nsub * (4 * j + 4)) / nw == (nsub * 4 * j) / nw;
  } else if (a.contig == 2) {
    empty = run_start(nsub, j + 1, a.n_splits) == run_start(nsub, j, a.n_splits);
  } else {
    empty = c_first + 4 * j >= c_end;
  }
  float m[G], l[G];
  uint16_t first_leaving = 0;
  if (!empty) {
    if (j == a.n_splits) {
      // a decode step's first ring entry to quantize after the attention
      // (position sq when it leaves the window), read now
      uint16_t first_lv = 0;
      if (a.k_new) {
        const int e1 = squant_of(Lq, g.S, g.R, g.F) < Lq - 1 ? squant_of(Lq, g.S, g.R, g.F) : Lq - 1;
        if (sq < e1) {
          const int64_t row = (unit * g.W + (sq - g.S) % g.W) * D + (tid & (D - 1));
          first_lv = tid >= D ? a.pl.vring[row] : a.pl.kring[row];
        }
      }
      if constexpr (PREP) {
        PrepIn<G> pin;
        prep_load<G>(a, u, pin);
        prep_store<BITS, G>(sm, pin);
        // G >= 4: the prep kernel leaves the new entry to this workgroup
        if (C::HS && a.k_new) new_entry<IO_BF16, BITS, G>(a, h, si, sm);
      } else {
        // the query inputs and the new entry's inputs in flight together
        QueryIn<G> qin;
        compensate_load<IO_BF16, G>(a, h, si, qin);
        if (a.k_new) new_entry<IO_BF16, BITS, G>(a, h, si, sm);
        compensate_query<IO_BF16, BITS, G>(a, h, si, sm, qin);
      }
      window_chunk<BITS, G>(a, unit, Lq, sq, sm, m, l);
      first_leaving = first_lv;
    } else if constexpr (C::HS) {
      const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform for the compiler
      const int c0 = mr0 + w;
      // the query inputs, then the first two sub-chunks' codes, in flight together
      MBuf<BITS> A, B;
      MQuery<C::NTL> qy;
      if constexpr (PREP) {
        // the lane's operands straight from the unit's query block (its
        // scales and operand words; q' and the new entry are the window's)
        const uint32_t* blk = a.prep + (int64_t)u * prep_words(G);
        mquery_load<C::NTL>(qy, (const float*)(blk + (C::O_QSC - C::O_QF)), blk + (C::O_QD - C::O_QF));
        mload<BITS>(A, a, qm, c0 < mr1 ? c0 * C::MT : -1, spare);
        mload<BITS>(B, a, qm, c0 + 4 < mr1 ? (c0 + 4) * C::MT : -1, spare);
      } else {
        QueryIn<G> qin;
        compensate_load<IO_BF16, G>(a, h, si, qin);
        mload<BITS>(A, a, qm, c0 < mr1 ? c0 * C::MT : -1, spare);
        mload<BITS>(B, a, qm, c0 + 4 < mr1 ? (c0 + 4) * C::MT : -1, spare);
        compensate_query<IO_BF16, BITS, G>(a, h, si, sm, qin);
        mquery_load<C::NTL>(qy, (const float*)(sm + C::O_QSC), sm + C::O_QD);
      }
      uint32_t* wbase = sm + C::O_UNION;
      float* part = (float*)(wbase + 4 * C::WAVE);  // [4 waves][G][D + 2]
      mquant_wave<BITS, C::NTL>(a, qm, c0, mr1, lo, hi, qy, (uint16_t*)(wbase + w * C::WAVE),
                                part + w * G * (D + 2), A, B, spare);
      __syncthreads();
      merge_waves<G>(part, obuf, m, l);
    } else {
      const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wi = 4 * j + w;
      int c0, cstride, cend;
      if (a.contig == 1) {
        c0 = c_first + (int)((nsub * wi) / nw);
        cend = c_first + (int)((nsub * (wi + 1)) / nw);
        cstride = 1;
      } else if (a.contig == 2) {
        c0 = c_first + run_start(nsub, j, a.n_splits) + w;
        cend = c_first + run_start(nsub, j + 1, a.n_splits);
        cstride = 4;
      } else {
        c0 = c_first + wi;
        cend = c_end;
        cstride = nw;
      }
      // the query inputs, then the first sub-chunk's codes, in flight together
      SubBuf<BITS, G> A, B;
      if constexpr (PREP) {
        PrepIn<G> pin;
        prep_load<G>(a, u, pin);
        load_first<BITS, G>(A, a, qm, c0, cend, spare);
        load_first<BITS, G>(B, a, qm, c0 + cstride, cend, spare);
        prep_store<BITS, G>(sm, pin);
      } else {
        QueryIn<G> qin;
        compensate_load<IO_BF16, G>(a, h, si, qin);
        load_first<BITS, G>(A, a, qm, c0, cend, spare);
        load_first<BITS, G>(B, a, qm, c0 + cstride, cend, spare);
        compensate_query<IO_BF16, BITS, G>(a, h, si, sm, qin);
      }
      uint32_t* wbase = sm + C::O_UNION;
      float* part = (float*)(wbase + 4 * C::WAVE);  // [4 waves][G][D + 2]
      quant_wave<BITS, G, CPOL_NT, G == 1>(a, qm, c0, cstride, cend, lo, hi,
                                           (const float*)(sm + C::O_QSC), sm + C::O_QD,
                                           wbase + w * C::WAVE, part + w * G * (D + 2), D + 2, A,
                                           B, spare);
      __syncthreads();
      merge_waves<G>(part, obuf, m, l);
    }
  }
  __syncthreads();
  if (tid < D) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      float* dst = a.wsp + ((int64_t)(qbase + gg) * nsp + j) * PS;
      dst[tid] = empty ? 0.f : obuf[gg * D + tid];
      if (tid == 0) {
        dst[D] = empty ? -INFINITY : m[gg];
        dst[D + 1] = empty ? 0.f : l[gg];
      }
    }
  }
  if (a.k_new && j == a.n_splits) step_append<BITS, G>(a, unit, qm, Lq, sq, sm, first_leaving);
}

// One workgroup per (sequence, query head): log-sum-exp merge of the
// partials.  Thread = (4 dimensions, partial residue mod 8).
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  // partials per residue class mod 8: n_splits <= 64, so at most 65 partials
  constexpr int KMAX = 9;
  __shared__ __align__(16) float racc[8][D];
  __shared__ float red[64];
  const int jq = blockIdx.x, si = blockIdx.y, tid = threadIdx.x;
  const int nsp = a.n_splits + 1;
  // partials written: the sequence's quantized workgroups 0 .. nq - 1 and the
  // window's, n_splits (a balanced grid gives a sequence nq <= n_splits)
  const int nq = a.balanced ? (a.s.wg0[si + 1] - a.s.wg0[si]) / a.g.n_kv : a.n_splits;
  auto written = [&](int y) { return y < nq || y == a.n_splits; };
  const float* src = a.wsp + ((int64_t)si * a.g.n_q + jq) * nsp * PS;
  const int d4 = (tid & 31) * 4, rsd = tid >> 5;
  // every load in flight at once: (m, l) of partial tid, and this thread's
  // four dimensions of partials rsd, rsd + 8, ... with their (m, l)
  float mt = -INFINITY, lt = 0.f;
  if (written(tid)) {
    mt = src[tid * PS + D];
    lt = src[tid * PS + D + 1];
  }
  float4 v[KMAX];
  float my[KMAX], ly[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int y = rsd + 8 * k;
    v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    my[k] = 0.f;
    ly[k] = 0.f;
    if (written(y)) {
      v[k] = *(const float4*)(src + (int64_t)y * PS + d4);
      my[k] = src[y * PS + D];
      ly[k] = src[y * PS + D + 1];
    }
  }
  float M[1] = {lt > 0.f ? mt : -INFINITY};
  block_reduce<1, true>(M, red);
  float Ls[1] = {lt > 0.f ? lt * exp2f(mt - M[0]) : 0.f};
  float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const float fy = ly[k] > 0.f ? exp2f(my[k] - M[0]) : 0.f;
    o4.x = fmaf(v[k].x, fy, o4.x);
    o4.y = fmaf(v[k].y, fy, o4.y);
    o4.z = fmaf(v[k].z, fy, o4.z);
    o4.w = fmaf(v[k].w, fy, o4.w);
  }
  block_reduce<1, false>(Ls, red);
  *(float4*)(&racc[rsd][d4]) = o4;
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) o += racc[x][tid];
    a.out[((int64_t)si * a.g.n_q + jq) * D + tid] = o / Ls[0];
  }
}

// Workgroups per (sequence, KV head) so that the grid (plus the window
// workgroups) fits the GPU's resident capacity once; never more than the host
// bound in a.n_splits.
template <int IO_BF16, int BITS, int G>
hipError_t launch_split(DecodeArgs& a, hipStream_t st) {
  // resident workgroups of the two kernel variants (in-workgroup query
  // preparation, query block from the prep kernel)
  static int slots = 0, slots_p = 0, cus = 0;
  const size_t lds = (size_t)SplitCfg<BITS, G>::TOTAL * 4;
  if (slots == 0) {
    int dev = 0, per = 0, per_p = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, split_kernel<IO_BF16, BITS, G, false>, 256,
                                                       lds);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_p, split_kernel<IO_BF16, BITS, G, true>, 256,
                                                       lds);
    if (e != hipSuccess) return e;
    slots_p = cus * (per_p > 0 ? per_p : 1);
    slots = cus * (per > 0 ? per : 1);
  }
  // Layouts, chosen per launch:
  //  - G >= 4 (matrix-core path): one wave of workgroups, the quantized ones
  //    shared out among the sequences in proportion to their 64-position
  //    sub-chunks (balanced grid, below);
  //  - G <= 2 with at most half as many units as CUs: one quantized
  //    workgroup per CU (below), query preparation in every workgroup;
  //  - otherwise, for long single launches with few units: the grid fills the
  //    resident capacity once, query preparation in every workgroup;
  //  - otherwise the query is prepared once per unit in the prep kernel and
  //    the grid is oversubscribed ~6x, so that the dispatcher balances
  //    workgroups of unequal length (ragged batches, many units) and the
  //    window workgroup's chain stays short.
  const int units = a.n_seq * a.g.n_kv;
  bool prep = false;
  int grid = 0;
  a.balanced = 0;
  if (SplitCfg<BITS, G>::HS) {
    // A workgroup takes four sub-chunks at a time, so an oversubscribed grid
    // would leave it runs too short for its fixed costs; one wave of
    // workgroups with shares in proportion to the sequences' lengths keeps
    // the ragged batch balanced instead (36-layer ragged batch: 2.80 ms per
    // step with ~6x oversubscription, 2.40 with 1x).  The prep kernel
    // prepares the query blocks whenever the longest unit has 16 or more
    // sub-chunks (the preparation in every workgroup, behind its first code
    // loads, measured no faster).  At least four sub-chunks (one per wave)
    // per workgroup, at most a.n_splits per KV head.
    prep = a.max_sub >= 16;
    const int sl = prep ? slots_p : slots;
    constexpr int MT = SplitCfg<BITS, G>::MT;
    int64_t total = 0;
    int msub[MAXSEQ];
    for (int i = 0; i < a.n_seq; ++i) {
      const int lo = a.g.S, hi = a.s.squant[i];
      const int first = lo / MT, end = hi > lo ? (hi + MT - 1) / MT : first;
      msub[i] = end - first;
      total += (int64_t)msub[i] * a.g.n_kv;
    }
    // sub-chunks per workgroup: the smallest share whose rounded-up counts
    // fit the slots left by the window workgroups (a second wave of
    // workgroups would start only when the windows end)
    const int qwg = sl - units > units ? sl - units : units;
    int64_t per = (total + qwg - 1) / qwg;
    if (per < 4) per = 4;
    for (;;) {
      int64_t n = 0;
      for (int i = 0; i < a.n_seq; ++i) {
        const int64_t ni = (msub[i] + per - 1) / per;
        n += (ni < a.n_splits ? ni : a.n_splits) * a.g.n_kv;
      }
      if (n <= qwg) break;
      per += 1 + per / 16;
    }
    int acc = 0, nmax = 0;
    for (int i = 0; i < a.n_seq; ++i) {
      int n = (int)((msub[i] + per - 1) / per);
      if (n > a.n_splits) n = a.n_splits;
      a.s.wg0[i] = acc;
      acc += n * a.g.n_kv;
      if (n > nmax) nmax = n;
    }
    a.s.wg0[a.n_seq] = acc;
    a.n_splits = nmax;
    a.balanced = 1;
    grid = units + acc;
  } else if (2 * units <= cus) {
    // Few units (long contexts, G <= 2): one quantized workgroup per CU, each
    // on one contiguous run of its unit's sub-chunks, with the query
    // preparation in every workgroup.  Four waves per CU keep fewer bytes in
    // flight than three workgroups per CU, and a contiguous run per CU keeps
    // each CU's addresses together; together they stream faster (128K MHA,
    // one layer of 32 KV heads: 69 -> 64 us per launch; 64K: 47 -> 41 us).
    int fill = cus / units;
    if (a.n_splits > fill) a.n_splits = fill;
    a.contig = 2;
  } else if (a.n_splits > 0) {
    int fill = (slots - units) / units;
    if (fill < 1) fill = 1;
    const double bytes = (double)a.total_sub * SplitCfg<BITS, G>::TW * (32.0 * BITS + 8.0);
    prep = a.max_sub >= 16 && (bytes < 240e6 || 9 * units > slots);
    if (prep) {
      const int target = (6 * slots_p) / units - 1;
      if (target > fill) fill = target;
    }
    if (a.n_splits > fill) a.n_splits = fill;
  }
  a.xcd_map = a.xcd_map && units % 8 == 0;
  if (!a.balanced) grid = (a.n_splits + 1) * units;
  if (prep) {
    hipLaunchKernelGGL((prep_kernel<IO_BF16, BITS, G>), dim3(a.g.n_kv, a.n_seq), dim3(256), lds, st, a);
    hipLaunchKernelGGL((split_kernel<IO_BF16, BITS, G, true>), dim3(grid), dim3(256), lds, st, a);
  } else {
    hipLaunchKernelGGL((split_kernel<IO_BF16, BITS, G, false>), dim3(grid), dim3(256), lds, st, a);
  }
  return hipGetLastError();
}

template <int IO_BF16, int BITS>
hipError_t launch_split_g(DecodeArgs& a, hipStream_t st) {
  switch (a.g.G) {
    case 1: return launch_split<IO_BF16, BITS, 1>(a, st);
    case 2: return launch_split<IO_BF16, BITS, 2>(a, st);
    case 4: return launch_split<IO_BF16, BITS, 4>(a, st);
    default: return launch_split<IO_BF16, BITS, 8>(a, st);
  }
}

}  // namespace

hipError_t launch_decode(DecodeArgs& a, int io_bf16, hipStream_t st, hipEvent_t ev_start,
                         hipEvent_t ev_stop, hipEvent_t ev_cstart, hipEvent_t ev_cstop) {
  hipError_t e;
  if (ev_start && (e = hipEventRecord(ev_start, st)) != hipSuccess) return e;
  if (io_bf16)
    e = a.g.bits == 2 ? launch_split_g<1, 2>(a, st)
      : a.g.bits == 3 ? launch_split_g<1, 3>(a, st) : launch_split_g<1, 4>(a, st);
  else
    e = a.g.bits == 2 ? launch_split_g<0, 2>(a, st)
      : a.g.bits == 3 ? launch_split_g<0, 3>(a, st) : launch_split_g<0, 4>(a, st);
  if (e != hipSuccess) return e;
  if (ev_stop && (e = hipEventRecord(ev_stop, st)) != hipSuccess) return e;
  if (ev_cstart && (e = hipEventRecord(ev_cstart, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(a.g.n_q, a.n_seq), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev_cstop && (e = hipEventRecord(ev_cstop, st)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace wkv
