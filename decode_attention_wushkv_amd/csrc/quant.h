// Device-side helpers of the quantizer shared by the append kernels and the
// fused decode step: exact number-format conversions and the per-token
// percentile-clipped affine quantizer (WUSH-KV paper page, section 5.3;
// appendix B.3 for the level grid).
//
// Numerics: order statistics are exact (rank sort or selection of the 128
// bfloat16 values); the linear-interpolation percentile, the scale
// (hi - lo)/(2^b - 1) and its binary16 rounding are fp64 with no fused
// multiply-add; levels are round-half-to-even of the exact (x - z16)/s16,
// decided by exact comparisons with the level boundaries.
#pragma once

#include "common.h"

namespace wkv {
namespace {

// ---------------------------------------------------------------- formats

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Round m / 2^s to nearest, ties to even (1 <= s <= 63).
__device__ __forceinline__ uint64_t shift_rne(uint64_t m, int s) {
  uint64_t q = m >> s;
  uint64_t rem = m & ((1ull << s) - 1);
  uint64_t half = 1ull << (s - 1);
  if (rem > half || (rem == half && (q & 1))) q += 1;
  return q;
}

// fp64 -> bfloat16 bits, round to nearest even, gradual underflow, overflow to inf.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000);
  int ef = (int)((b >> 52) & 0x7FF);
  uint64_t mant = b & 0xFFFFFFFFFFFFFull;
  if (ef == 0x7FF) return sign | (mant ? 0x7FC0 : 0x7F80);
  if (ef == 0) return sign;  // fp64 subnormals lie far below bf16's smallest step
  int e = ef - 1023;
  uint64_t m = mant | (1ull << 52);
  if (e >= -126) {
    uint64_t r = shift_rne(m, 45);  // keep 8 significant bits
    if (r == 256) { r = 128; e += 1; }
    if (e > 127) return sign | 0x7F80;
    return sign | (uint16_t)((e + 127) << 7) | (uint16_t)(r & 0x7F);
  }
  int s = -(e + 81);  // value in units of 2^-133 is m * 2^(e + 81)
  if (s > 63) return sign;
  return sign | (uint16_t)shift_rne(m, s);  // r <= 128; 128 encodes 2^-126
}

// fp32 -> bfloat16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> binary16 bits, round to nearest even, saturating at +-65504.
__device__ __forceinline__ uint16_t f64_to_f16_sat(double x) {
  if (x != x) return 0x7E00;
  // round to odd into fp32 (13 more significant bits than binary16 and a wider
  // exponent range), so that the hardware round-to-nearest-even conversion to
  // binary16 gives the binary16 rounding of x itself
  const float f = (float)x;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != x) {
    if (fabs(back) > fabs(x)) u -= 1u;  // toward zero (f is not zero here)
    u |= 1u;
  }
  const uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)__uint_as_float(u));
  return (h & 0x7FFFu) == 0x7C00u ? (uint16_t)((h & 0x8000u) | 0x7BFFu) : h;  // saturate
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------- transform

// k'_i = sum_j T_ij k_j to fp64 accuracy (every fp32 x fp32 product is exact
// in fp64), in one fixed order shared by every path that stores a transformed
// key: four partial sums over dimensions [32 q, 32 q + 32), each a chain of
// fp64 FMAs in dimension order, added as (s0 + s1) + (s2 + s3).  t(j) and
// k(j) return T_ij and k_j.
template <typename TF, typename KF>
__device__ __forceinline__ double transform_entry(TF t, KF k) {
  double s[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int j = 0; j < D / 4; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      s[q] = fma((double)t(q * (D / 4) + j), (double)k(q * (D / 4) + j), s[q]);
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// ---------------------------------------------------------------- quantizer

// LDS scratch of the quantizer for up to two groups of 128 threads.
struct QLds {
  float vals[2][D];
  float sorted[2][D];
  int codes[2][D];
  double ss[2][2];  // RMS codec: sums of squares of the two halves of each group
};

// Sum of squares of a group in the order shared by every path: each half
// [64 h, 64 h + 64) summed in dimension order in fp64 (every square of a
// bfloat16 value is exact), then half 0 + half 1.  rms = sqrt(sum / 128).
__device__ __forceinline__ double rms_of_halves(double s0, double s1) {
#pragma clang fp contract(off)
  return sqrt((s0 + s1) / (double)D);
}

// Linear-interpolation percentile of the sorted group (fp64, no FMA).
__device__ __forceinline__ double percentile_sorted(const float* sorted, double p) {
#pragma clang fp contract(off)
  double h = p * (double)(D - 1);
  double jf = floor(h);
  int j = (int)jf;
  double f = h - jf;
  if (j >= D - 1) return (double)sorted[D - 1];
  double a = (double)sorted[j];
  double b = (double)sorted[j + 1];
  return a + f * (b - a);
}

// Level assignment.  The boundary between levels c and c + 1 is
// z16 + (c + 1/2) s16, exact in fp64 (both factors have at most 11
// significant bits).  A value takes a level above c when it lies above that
// boundary; a value exactly on it rounds to the even level, so the test is
// strict for even c.  This is round-half-to-even of the exact (x - z16) / s16,
// clamped to [0, levels], computed without a division.
__device__ __forceinline__ bool above_boundary(double x, double zd, double sd, int c) {
#pragma clang fp contract(off)
  const double t = zd + ((double)c + 0.5) * sd;
  return (c & 1) ? x >= t : x > t;
}

__device__ __forceinline__ int level_of(double x, double zd, double sd, int levels) {
  if (sd == 0.0) return 0;
  int c = 0;
  for (int k = 0; k < levels; ++k) c += above_boundary(x, zd, sd, k) ? 1 : 0;
  return c;
}

// Linear-interpolation percentile from the two order statistics around
// h = p (n - 1): x_j + f (x_{j+1} - x_j), f = h - floor(h) (fp64, no FMA).
__device__ __forceinline__ double interp(double xj, double xj1, double f) {
#pragma clang fp contract(off)
  return xj + f * (xj1 - xj);
}

// Scale and zero of a group with clip ends lo, hi: s = (hi - lo)/(2^b - 1),
// z = lo, both rounded to binary16 (saturating).
__device__ __forceinline__ void scale_zero(double lo, double hi, int bits, uint16_t* s16,
                                           uint16_t* z16) {
#pragma clang fp contract(off)
  const double levels = (double)((1 << bits) - 1);
  *s16 = f64_to_f16_sat((hi - lo) / levels);
  *z16 = f64_to_f16_sat(lo);
}

// Quantize groups of 128 values (clip ends from the percentiles or from the
// RMS, by the cache's codec): thread t holds element t % 128 of group
// t / 128 (x).  Returns this thread's code; *sz gets {s16 | z16 << 16} of its
// group.  Every thread of the workgroup must call it (it uses barriers).
__device__ __forceinline__ int quantize_group(float x, QLds& L, const Geometry& g, uint32_t* sz) {
#pragma clang fp contract(off)
  const int i = threadIdx.x & (D - 1), grp = threadIdx.x >> 7;
  const int bits = g.bits;
  float* vals = L.vals[grp];
  float* sorted = L.sorted[grp];
  vals[i] = x;
  __syncthreads();
  double lo, hi;
  if (g.codec == WUSHKV_CODEC_RMS) {
    if ((i & 63) == 0) {
      double ss = 0.0;
      for (int j = i; j < i + 64; ++j) {
        const double v = (double)vals[j];
        ss = fma(v, v, ss);
      }
      L.ss[grp][i >> 6] = ss;
    }
    __syncthreads();
    const double rms = rms_of_halves(L.ss[grp][0], L.ss[grp][1]);
    lo = -g.alpha * rms;
    hi = g.alpha * rms;
  } else {
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < D; ++j) {
      float y = vals[j];
      rank += (y < x) || (y == x && j < i);
    }
    sorted[rank] = x;
    __syncthreads();
    lo = percentile_sorted(sorted, g.p_lo);
    hi = percentile_sorted(sorted, g.p_hi);
  }
  uint16_t s16, z16;
  scale_zero(lo, hi, bits, &s16, &z16);
  const int c = level_of((double)x, f16_bits_to_f64(z16), f16_bits_to_f64(s16), (1 << bits) - 1);
  *sz = (uint32_t)s16 | ((uint32_t)z16 << 16);
  __syncthreads();  // vals / sorted may be reused by the next call
  return c;
}

// Accumulates value-code bits of one 16-byte row of one dimension (row index
// in units of D x 16 bytes of vcode) for consecutive positions and writes the
// row once (read-modify-write keeps other positions' bits).  Named fields
// rather than arrays keep the row in registers.
struct VRow {
  int64_t row;              // -1: empty
  uint32_t b0, b1, b2, b3;  // code bits
  uint32_t m0, m1, m2, m3;  // which bits are set
};
// Rows a value code goes to: lo (2- and 4-bit codes, the low plane of 3-bit
// codes) and hi (the high plane of 3-bit codes).
struct VRows {
  VRow lo, hi;
};

__device__ __forceinline__ void vrows_init(VRows& v) { v.lo.row = v.hi.row = -1; }

__device__ __forceinline__ void vrow_flush(VRow& r, const Planes& pl) {
  if (r.row < 0) return;
  uint4* p = (uint4*)(pl.vcode + (r.row * D + (threadIdx.x & (D - 1))) * 16);
  uint4 old = *p;
  old.x = (old.x & ~r.m0) | r.b0;
  old.y = (old.y & ~r.m1) | r.b1;
  old.z = (old.z & ~r.m2) | r.b2;
  old.w = (old.w & ~r.m3) | r.b3;
  *p = old;
  r.row = -1;
}

template <bool B3>
__device__ __forceinline__ void vrows_flush(VRows& v, const Planes& pl) {
  vrow_flush(v.lo, pl);
  if constexpr (B3) vrow_flush(v.hi, pl);
}

// Put the nb-bit field code at bit `bit` (0..127) of row `row`.
__device__ __forceinline__ void vrow_put(VRow& r, int64_t row, int bit, uint32_t code, int nb,
                                         const Planes& pl) {
  if (row != r.row) {
    vrow_flush(r, pl);
    r.row = row;
    r.b0 = r.b1 = r.b2 = r.b3 = r.m0 = r.m1 = r.m2 = r.m3 = 0u;
  }
  const int w = bit >> 5;
  const uint32_t cv = code << (bit & 31);
  const uint32_t mv = ((1u << nb) - 1u) << (bit & 31);
  r.b0 |= w == 0 ? cv : 0u;
  r.b1 |= w == 1 ? cv : 0u;
  r.b2 |= w == 2 ? cv : 0u;
  r.b3 |= w == 3 ? cv : 0u;
  r.m0 |= w == 0 ? mv : 0u;
  r.m1 |= w == 1 ? mv : 0u;
  r.m2 |= w == 2 ? mv : 0u;
  r.m3 |= w == 3 ? mv : 0u;
}

// The value code of the position at row prow of the per-position planes.
// B3: the cache holds 3-bit codes (a compile-time choice, so that the 2- and
// 4-bit kernels carry no high-plane accumulator).
template <bool B3>
__device__ __forceinline__ void vrows_add(VRows& v, int64_t prow, int code, const Planes& pl,
                                          const Geometry& g) {
  if constexpr (B3) {
    const int64_t blk = prow >> 7;
    const int t = (int)(prow & 127);
    vrow_put(v.lo, 3 * blk + (t >> 6), (t & 63) * 2, (uint32_t)code & 3u, 2, pl);
    vrow_put(v.hi, 3 * blk + 2, hi_bit(t), (uint32_t)code >> 2, 1, pl);
  } else {
    const int sh = g.bits == 2 ? 6 : 5;  // log2(vblock)
    vrow_put(v.lo, prow >> sh, (int)(prow & ((1 << sh) - 1)) * g.bits, (uint32_t)code, g.bits, pl);
  }
}

// Quantize key and value entries of position p and store codes and
// scale/zero.  128-thread workgroups: thread i holds dimension i of both (kx,
// vx) and the two groups run one after the other.  256-thread workgroups:
// threads 0..127 hold the key entry (kx), threads 128..255 the value entry
// (vx) and both groups run at once.
template <bool B3>
__device__ __forceinline__ void store_quantized(int p, float kx, float vx, QLds& L, VRows& vr, const Planes& pl,
                                const QMap& qm, const Geometry& g) {
  const int i = threadIdx.x & (D - 1);
  const bool two = blockDim.x == 2 * D;
  const bool is_v = two && threadIdx.x >= D;
  uint32_t ksz = 0, vsz = 0;
  int kc = 0, vc = 0;
  if (two) {
    uint32_t sz = 0;
    const int c = quantize_group(is_v ? vx : kx, L, g, &sz);
    kc = vc = c;
    ksz = vsz = sz;
  } else {
    kc = quantize_group(kx, L, g, &ksz);
    vc = quantize_group(vx, L, g, &vsz);
  }
  if (!is_v) L.codes[0][i] = kc;
  __syncthreads();
  const int words = g.code_bytes / 4;  // 8 (2-bit), 12 (3-bit) or 16 (4-bit)
  const int64_t row = qrow(qm, p);     // -1: unmapped page, nothing is stored
  if (threadIdx.x < words && row >= 0) {
    const int t = threadIdx.x;
    uint32_t w = 0;
    if (B3) {
      if (t < 8)  // low plane: elements 16 t + e at bits 2 e
        for (int e = 0; e < 16; ++e) w |= ((uint32_t)L.codes[0][16 * t + e] & 3u) << (2 * e);
      else        // high plane word t - 8
        for (int e = 32 * (t - 8); e < 32 * (t - 7); ++e)
          w |= ((uint32_t)L.codes[0][e] >> 2) << (hi_bit(e) & 31);
    } else {
      const int per = 32 / g.bits;
      for (int e = 0; e < per; ++e) w |= (uint32_t)L.codes[0][t * per + e] << (e * g.bits);
    }
    ((uint32_t*)(pl.kcode + row * g.code_bytes))[t] = w;
  }
  if (threadIdx.x == 0 && row >= 0) pl.ksz[row] = ksz;
  if (threadIdx.x == (two ? D : 0) && row >= 0) pl.vsz[row] = vsz;
  if ((!two || is_v) && row >= 0) vrows_add<B3>(vr, row, vc, pl, g);
  __syncthreads();  // codes[] reuse
}

}  // namespace
}  // namespace wkv
