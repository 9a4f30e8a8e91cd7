// Prefill append for bfloat16 inputs: the key transform of whole position
// tiles on the matrix cores, then selection, quantization and packing (WUSH-KV
// paper page, sections 4.2, 4.4, 5.3; appendix B.3 for the level grid).
//
// One workgroup (8 waves, two per SIMD, sharing one LDS copy of T_K and of
// the tiles) takes up to 1024 new positions of one (sequence, KV head), in
// tiles of 64 positions aligned to the value-code blocks.
//
// Transform.  k' = T_K k for the 64 keys of a tile is a [64 x 128] x
// [128 x 128] product.  T_K (fp32) is split exactly into three bfloat16 parts,
// T = T1 + T2 + T3 (8 + 8 + 8 significant bits), held as MFMA operands in
// registers for the whole workgroup; bfloat16 keys times bfloat16 parts are
// exact products, summed by the matrix cores in fp32: T1 products in eight
// v_mfma_f32_16x16x16_bf16 of 16 folded into one fp32 sum, T2 and T3 products
// in one v_mfma_f32_16x16x32_bf16 chain.  The fp32 error of the sum is below
// 20 ulp (2^-23 each) of A = sum_j |k_j| |T_ij|, which a fourth MFMA chain
// (|k| times |T1|) bounds.  An entry whose fp32 value lies within that bound of
// a bfloat16 rounding boundary is recomputed in fp64 with the arithmetic of the
// one-position paths (transform_entry; about 2 per cent of the entries, each by
// the wave that flagged it, four lanes to an entry), so the stored bfloat16
// keys are identical to theirs.
//
// Quantization.  Each group (one position's 128 key or value entries) is
// split over four lanes.  A lane scans its 32 entries keeping the three
// smallest and three largest (v_med3 insertion), the four merge them in two
// DPP rounds, and the order statistics around h = p (n - 1) give the
// linear-interpolation percentiles.  This covers clip percentiles whose
// interpolation needs only the three smallest and three largest values
// (p_lo (n - 1) < 2 and p_hi (n - 1) >= 125; the host falls back to the
// rank-sort kernel otherwise).
// With the RMS codec the clip ends are -alpha rms, +alpha rms instead (sum of
// squares per half-group in fp64, as in quant.h).  Scale, zero and levels
// follow quant.h exactly.  The four key waves quantize the tile's key groups
// while the four value waves quantize its value groups.  Key codes are stored
// by the group's lanes; value codes go to LDS as bytes, and during the next
// tile's transform one thread per 16-byte value-code row assembles its words
// from them and writes the row whole (no atomics: 16 lanes OR-ing into one
// word serialize).  Three barriers per tile.
#include <type_traits>

#include "quant.h"

namespace wkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int PT = PREFILL_TILE;  // positions per tile
constexpr int PCH = PREFILL_SPAN; // positions per workgroup
constexpr int NT = 512;           // threads per workgroup (8 waves)
constexpr int RS = 136;           // LDS row stride (bf16 elements) of the key / value tiles
constexpr int TS = 132;           // LDS row stride (floats) of T_K
constexpr int VCS = 132;          // LDS row stride (bytes) of the value-code bytes
constexpr int FIXMAX = PT * D;    // recomputation list capacity (every entry of a tile)
constexpr int FIXW = FIXMAX / (NT / 64);  // one wave's segment (its 16 dimensions of 64 rows)
// fp32 summation error bound of the transform relative to sum_j |k_j| |T_ij|,
// counting one ulp (2^-23) per rounding whatever order and rounding the
// matrix core uses inside an instruction: 15 roundings inside each 16-product
// T1 MFMA, 3 from the fold tree of the eight results, the T2 + T3 chain
// below 2^-8 of T (about half an ulp overall), the final additions: under 20
// ulp.
constexpr float kTransformErr = 20.0f * 0x1p-23f;

struct __align__(16) PLds {
  float t[D * TS];        // T_K rows (fp32)
  uint16_t k[PT * RS];    // input keys (bf16)
  uint16_t ka[PT * RS];   // their magnitudes |k|
  uint16_t v[PT * RS];    // values (bf16)
  uint16_t kq[PT * RS];   // transformed keys (bf16)
  uint16_t fix[FIXMAX];   // entries to recompute, one segment per wave: row << 7 | dimension
  uint8_t vc[PT * VCS];   // value codes of the tile, [position][dimension]
};

__device__ __forceinline__ __bf16 bf16_of_bits(uint32_t b) {
  return __builtin_bit_cast(__bf16, (uint16_t)b);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x4 as_bf16x4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(bf16x4, make_uint2(lo, hi));
}

// |x| of eight bfloat16 values, recomputed where it is used (a volatile
// v_and_b32 per dword, so that the compiler does not keep a copy of the
// magnitudes of the loop-invariant T1 operand in registers)
__device__ __forceinline__ bf16x8 abs_bf16x8(bf16x8 x) {
  const uint4 u = __builtin_bit_cast(uint4, x);
  uint4 r;
  asm volatile("v_and_b32 %0, 0x7fff7fff, %1" : "=v"(r.x) : "v"(u.x));
  asm volatile("v_and_b32 %0, 0x7fff7fff, %1" : "=v"(r.y) : "v"(u.y));
  asm volatile("v_and_b32 %0, 0x7fff7fff, %1" : "=v"(r.z) : "v"(u.z));
  asm volatile("v_and_b32 %0, 0x7fff7fff, %1" : "=v"(r.w) : "v"(u.w));
  return as_bf16x8(r);
}

// A pointer that is the same in every lane, read from the first active lane
// (kept in scalar registers; the compiler cannot re-associate it with a
// per-lane offset)
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const uint16_t*)((uint64_t)lo | ((uint64_t)hi << 32));
}

// float rounded down / up from a double (exact bounds for comparisons of
// float values against an fp64 boundary)
__device__ __forceinline__ float f32_down(double d) {
  float f = (float)d;
  if ((double)f > d) f = nextafterf(f, -INFINITY);
  return f;
}
__device__ __forceinline__ float f32_up(double d) {
  float f = (float)d;
  if ((double)f < d) f = nextafterf(f, INFINITY);
  return f;
}

// v_med3 insertion of x into the three smallest (a0 <= a1 <= a2) and three
// largest (b0 >= b1 >= b2) seen so far
__device__ __forceinline__ void sel_insert(float x, float& a0, float& a1, float& a2, float& b0,
                                           float& b1, float& b2) {
  a2 = __builtin_amdgcn_fmed3f(a1, a2, x);
  a1 = __builtin_amdgcn_fmed3f(a0, a1, x);
  a0 = fminf(a0, x);
  b2 = __builtin_amdgcn_fmed3f(b1, b2, x);
  b1 = __builtin_amdgcn_fmed3f(b0, b1, x);
  b0 = fmaxf(b0, x);
}

// Value of lane ^ 1 (CTRL 0xB1) or lane ^ 2 (CTRL 0x4E) by DPP quad_perm.
template <int CTRL>
__device__ __forceinline__ float partner(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double partner_d(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}

// Merges the partner lane's three smallest / largest into this lane's.
template <int CTRL>
__device__ __forceinline__ void merge_sel(float& a0, float& a1, float& a2, float& b0, float& b1,
                                          float& b2) {
  const float pa0 = partner<CTRL>(a0), pa1 = partner<CTRL>(a1), pa2 = partner<CTRL>(a2);
  const float pb0 = partner<CTRL>(b0), pb1 = partner<CTRL>(b1), pb2 = partner<CTRL>(b2);
  float d0 = b0, d1 = b1, d2 = b2;
  sel_insert(pa0, a0, a1, a2, d0, d1, d2);
  sel_insert(pa1, a0, a1, a2, d0, d1, d2);
  sel_insert(pa2, a0, a1, a2, d0, d1, d2);
  float e0 = INFINITY, e1 = INFINITY, e2 = INFINITY;
  sel_insert(pb0, e0, e1, e2, b0, b1, b2);
  sel_insert(pb1, e0, e1, e2, b0, b1, b2);
  sel_insert(pb2, e0, e1, e2, b0, b1, b2);
}

__device__ __forceinline__ float bf16_lane(const uint32_t* uw, int e) {
  return __uint_as_float((e & 1) ? (uw[e >> 1] & 0xFFFF0000u) : (uw[e >> 1] << 16));
}

// Level of x against the group's boundaries (2 and 3 bits: float bounds
// rounded for the strict / non-strict tests; 4 bits: an estimate checked
// exactly in fp64).  Round-half-to-even of the exact (x - z16)/s16.
template <int BITS>
__device__ __forceinline__ int level_f(float x, const float* bnd, float zf, float inv, double zd,
                                       double sd) {
  constexpr int LEV = (1 << BITS) - 1;
  if constexpr (BITS <= 3) {
    int code = 0;
#pragma unroll
    for (int c2 = 0; c2 < LEV; ++c2) code += (c2 & 1) ? (x >= bnd[c2] ? 1 : 0) : (x > bnd[c2] ? 1 : 0);
    return code;
  } else {
    if (sd == 0.0) return 0;
    int cc = (int)rintf((x - zf) * inv);
    cc = cc < 0 ? 0 : (cc > LEV ? LEV : cc);
    const double xd = (double)x;
    if (cc > 0 && !above_boundary(xd, zd, sd, cc - 1))
      cc -= 1;
    else if (cc < LEV && above_boundary(xd, zd, sd, cc))
      cc += 1;
    return cc;
  }
}

template <int BITS>
__global__ __launch_bounds__(NT, 1) void prefill_kernel(AppendArgs a) {
  __shared__ PLds L;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = blockIdx.y, si = blockIdx.z;
  const Geometry& g = a.g;
  const int L0 = a.s.len0[si], L1 = L0 + a.s.n_new[si];
  const int base = L0 - L0 % PT;
  const int c0 = max(L0, base + (int)blockIdx.x * PCH);
  const int c1 = min(L1, base + ((int)blockIdx.x + 1) * PCH);
  if (c0 >= c1) return;
  const int64_t unit = ((int64_t)a.layer * g.max_batch + a.s.slot[si]) * g.n_kv + h;
  const QMap qm = qmap_of(g, a.layer, a.s.slot[si], h);
  const int sq1 = squant_of(L1, g.S, g.R, g.F);
  const int qlo = max(L0, g.S), qhi = min(L1, sq1);  // new positions that are quantized
  constexpr int LEV = (1 << BITS) - 1;
  // positions per value-code row of 16 bytes per dimension (the low plane's
  // at 3 bits)
  constexpr int VB = BITS == 3 ? 64 : 128 / BITS;

  // percentile interpolation points (fp64 exactly as in quant.h)
  const double hlo = g.p_lo * (double)(D - 1), hhi = g.p_hi * (double)(D - 1);
  const int jlo = (int)floor(hlo), jhi = (int)floor(hhi);
  const double flo = hlo - floor(hlo), fhi = hhi - floor(hhi);

  // ---- T_K of this head into LDS; MFMA operands of this wave's 16 output dims
  {
    const float4* tg = (const float4*)(a.tk + (int64_t)h * D * D);
    for (int x = tid; x < D * D / 4; x += NT) {
      const int r = (4 * x) / D, c = (4 * x) % D;
      *(float4*)(L.t + r * TS + c) = tg[x];
    }
  }
  __syncthreads();
  // wave w: output dims 16 w .. 16 w + 15 of all the tile's rows, in four
  // blocks of 16 rows; lane: output dim i, k-slice 8 (lane / 16) .. + 8 of each
  // 32-step (A and B take the same slice, so the products pair up whatever
  // order the matrix core sums them in)
  const int i_out = 16 * w + (lane & 15);
  bf16x8 b1[4], b2[4], b3[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = L.t[i_out * TS + 32 * ks + 8 * (lane >> 4) + e];
      const uint32_t t1 = f32_to_bf16(t);
      const float r1 = t - bf16_bits_to_f32((uint16_t)t1);
      const uint32_t t2 = f32_to_bf16(r1);
      const float r2 = r1 - bf16_bits_to_f32((uint16_t)t2);
      const uint32_t t3 = f32_to_bf16(r2);  // exact: r2 has at most 8 significant bits
      b1[ks][e] = bf16_of_bits(t1);
      b2[ks][e] = bf16_of_bits(t2);
      b3[ks][e] = bf16_of_bits(t3);
    }
  }

  // ---- input tiles: global -> registers one tile ahead -> LDS
  const int64_t tok0 = a.s.tok0[si];
  const uint16_t* kin = (const uint16_t*)a.k;
  const uint16_t* vin = (const uint16_t*)a.v;
  constexpr int NPRE = 2 * PT * 16 / NT;  // 16-byte chunks per thread
  static_assert(NPRE == 4 && PT == 64, "tile load layout assumes 4 chunks per thread");
  uint4 pre[NPRE];
  // this thread's chunks: rows rr, rr + 32 of the key tile, then of the value
  // tile, 16-byte chunk tid % 16; offsets (elements) from the tile's first row
  const int rr = (tid >> 4) & 31;
  const int off0 = (rr * g.n_kv) * D + 8 * (tid & 15), off1 = off0 + 32 * g.n_kv * D;
  auto load_tile = [&](int p0) {
    // first input row of the tile (uniform)
    const int64_t e0 = ((tok0 + (p0 - L0)) * g.n_kv + h) * D;
    // uniform tile bases (scalar registers), so that each load is a scalar
    // base plus this thread's 32-bit offset
    const uint16_t* kt = uniform_ptr(kin + e0);
    const uint16_t* vt = uniform_ptr(vin + e0);
#pragma unroll
    for (int u = 0; u < NPRE; ++u) {
      const int r = rr + 32 * (u & 1), p = p0 + r;
      pre[u] = make_uint4(0u, 0u, 0u, 0u);
      if (p >= c0 && p < c1)
        pre[u] = *(const uint4*)((u >> 1 ? vt : kt) + (uint32_t)(u & 1 ? off1 : off0));
    }
  };
  int p0 = c0 - (c0 - base) % PT;
  load_tile(p0);

  // role of the wave after the transform: waves 0-3 the keys, waves 4-7 the
  // values; each group (one position's 128 key or value entries) is split
  // over four lanes, lane quarter qd holding dimensions [32 qd, 32 qd + 32)
  const bool vwave = w >= NT / 128;
  const int rt = tid & (NT / 2 - 1);  // thread index within the role
  const int tg = rt >> 2, qd = rt & 3;

  // quantization of group tg of the tile (ISV: values from L.v, else the
  // transformed keys from L.kq); key codes go straight to the key plane,
  // value codes as bytes to L.vc
  auto quant_group = [&](auto isv_tag, int p0, int64_t trow) {
    constexpr bool isv = decltype(isv_tag)::value;
    const int t = tg;
    const int p = p0 + t;
    const bool quant = p >= qlo && p < qhi;
    const uint16_t* row = (isv ? L.v : L.kq) + t * RS + 32 * qd;
    uint32_t uw[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 u4 = *(const uint4*)(row + 8 * c);
      uw[4 * c] = u4.x;
      uw[4 * c + 1] = u4.y;
      uw[4 * c + 2] = u4.z;
      uw[4 * c + 3] = u4.w;
    }
    double lo, hi;
    if (g.codec == WUSHKV_CODEC_RMS) {
      // sum of squares of each half [64 hh, 64 hh + 64) in dimension order
      // (quant.h's rms_of_halves): lanes 0, 1 run half 0's chain, lanes 2, 3
      // half 1's, reading the group's row from LDS; lane ^ 2 gives the other
      const uint16_t* hrow = (isv ? L.v : L.kq) + t * RS + 64 * (qd >> 1);
      double ss = 0.0;
#pragma unroll 2
      for (int c = 0; c < 8; ++c) {
        const uint4 u4 = *(const uint4*)(hrow + 8 * c);
        const uint32_t hw[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double x = (double)bf16_lane(hw, e);
          ss = fma(x, x, ss);
        }
      }
      const double other = partner_d<0x4E>(ss);
      const double rms = qd < 2 ? rms_of_halves(ss, other) : rms_of_halves(other, ss);
      lo = -g.alpha * rms;
      hi = g.alpha * rms;
    } else {
      float a0 = INFINITY, a1 = INFINITY, a2 = INFINITY;
      float bb0 = -INFINITY, bb1 = -INFINITY, bb2 = -INFINITY;
#pragma unroll
      for (int e = 0; e < 32; ++e) sel_insert(bf16_lane(uw, e), a0, a1, a2, bb0, bb1, bb2);
      merge_sel<0xB1>(a0, a1, a2, bb0, bb1, bb2);  // with lane ^ 1
      merge_sel<0x4E>(a0, a1, a2, bb0, bb1, bb2);  // with lane ^ 2
      // order statistics x(0..2) = a0..a2, x(127..125) = bb0..bb2
      const double lx0 = jlo == 0 ? a0 : a1, lx1 = jlo == 0 ? a1 : a2;
      lo = interp(lx0, lx1, flo);
      if (jhi >= D - 1)
        hi = bb0;
      else
        hi = interp(jhi == D - 2 ? bb1 : bb2, jhi == D - 2 ? bb0 : bb1, fhi);
    }
    uint16_t s16, z16;
    scale_zero(lo, hi, BITS, &s16, &z16);
    const double sd = f16_bits_to_f64(s16), zd = f16_bits_to_f64(z16);
    // level boundaries as floats: strict tests (even c) against the boundary
    // rounded down, non-strict (odd c) against it rounded up
    float bnd[BITS <= 3 ? LEV : 1];
    float inv = 0.f;
    const float zf = (float)zd;
    if constexpr (BITS <= 3) {
#pragma unroll
      for (int c = 0; c < LEV; ++c) {
        const double tb = zd + ((double)c + 0.5) * sd;
        bnd[c] = sd == 0.0 ? INFINITY : ((c & 1) ? f32_up(tb) : f32_down(tb));
      }
    } else {
      inv = sd == 0.0 ? 0.f : (float)(1.0 / sd);
    }
    if constexpr (!isv) {
      // key codes of this lane's 32 dimensions: 2 bits: 2 words; 3 bits:
      // 2 low-plane words and high-plane word qd; 4 bits: 4 words
      uint32_t packed[BITS == 3 ? 3 : BITS];
#pragma unroll
      for (int q = 0; q < (BITS == 3 ? 3 : BITS); ++q) packed[q] = 0u;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int code = level_f<BITS>(bf16_lane(uw, e), bnd, zf, inv, zd, sd);
        if constexpr (BITS == 3) {
          const uint32_t lv = ((uint32_t)code & 3u) << (2 * (e & 15));
          packed[0] |= e < 16 ? lv : 0u;
          packed[1] |= e < 16 ? 0u : lv;
          packed[2] |= ((uint32_t)code >> 2) << (hi_bit(32 * qd + e) & 31);
        } else {
          packed[(e * BITS) >> 5] |= (uint32_t)code << ((e * BITS) & 31);
        }
      }
      if (quant && trow >= 0) {
        uint8_t* kr = a.pl.kcode + (trow + t) * (16 * BITS);
        if constexpr (BITS == 3) {
          *(uint2*)(kr + 8 * qd) = make_uint2(packed[0], packed[1]);
          *(uint32_t*)(kr + 32 + 4 * qd) = packed[2];
        } else if constexpr (BITS == 2) {
          *(uint2*)(kr + 8 * qd) = make_uint2(packed[0], packed[1]);
        } else {
          *(uint4*)(kr + 16 * qd) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        }
      }
    } else {
      // value codes as bytes into the tile's [position][dimension] block
      uint32_t cw[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) cw[q] = 0u;
#pragma unroll
      for (int e = 0; e < 32; ++e)
        cw[e >> 2] |= (uint32_t)level_f<BITS>(bf16_lane(uw, e), bnd, zf, inv, zd, sd) << (8 * (e & 3));
      uint32_t* dst = (uint32_t*)(L.vc + t * VCS + 32 * qd);
#pragma unroll
      for (int q = 0; q < 8; ++q) dst[q] = cw[q];
    }
    if (qd == 0 && quant && trow >= 0)
      (isv ? a.pl.vsz : a.pl.ksz)[trow + t] = (uint32_t)s16 | ((uint32_t)z16 << 16);
  };

  // window copies of one tensor of the tile (positions kept in bfloat16)
  auto windows = [&](bool isv, int p0) {
    for (int x = rt; x < PT * 16; x += NT / 2) {
      const int r = x >> 4, c = x & 15;
      const int p = p0 + r;
      if (p < c0 || p >= c1 || (p >= qlo && p < qhi)) continue;
      const uint4 val = *(const uint4*)((isv ? L.v : L.kq) + r * RS + c * 8);
      uint16_t* dst;
      if (p < g.S)
        dst = (isv ? a.pl.vsink : a.pl.ksink) + (unit * g.S + p) * D;
      else
        dst = (isv ? a.pl.vring : a.pl.kring) + (unit * g.W + (p - g.S) % g.W) * D;
      ((uint4*)dst)[c] = val;
    }
  };

  // value-code rows of the tile at p0 (codes as bytes in L.vc), one thread
  // per row of 16 bytes (2 and 4 bits: block row of one dimension; 3 bits:
  // the tile's low-plane row, or its half of the block's high-plane row);
  // codes of positions outside the tile's quantized range are masked out
  auto rows = [&](int p0, int64_t trow) {
    constexpr int NROW = BITS == 3 ? 2 * D : (PT / VB) * D;
    for (int x = tid; x < NROW; x += NT) {
      if (trow < 0) break;
      const int dim = x & (D - 1), blk = x >> 7;  // blk: block (2, 4 bits) or plane (3 bits)
      if (BITS != 3 || blk == 0) {
        constexpr int WPOS = BITS == 4 ? 8 : 16;  // positions per word
        constexpr int SH = BITS == 4 ? 4 : 2;
        const int b0 = p0 + (BITS == 3 ? 0 : blk * VB);
        const int nb = BITS == 3 ? PT : VB;
        const int lo = max(b0, max(c0, qlo)), hi = min(b0 + nb, min(c1, qhi));
        if (lo >= hi) continue;
        uint32_t wd[4], m[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t word = 0u;
#pragma unroll
          for (int n = 0; n < WPOS; ++n) {
            const int t = (b0 - p0) + q * WPOS + n;
            const uint32_t code = L.vc[t * VCS + dim];
            word |= (BITS == 3 ? (code & 3u) : code) << (n * SH);
          }
          wd[q] = word;
          const int bl = (lo - b0) * SH - 32 * q, bh = (hi - b0) * SH - 32 * q;
          const int l2 = bl < 0 ? 0 : (bl > 32 ? 32 : bl), h2 = bh < 0 ? 0 : (bh > 32 ? 32 : bh);
          m[q] = h2 <= l2 ? 0u : ((h2 - l2 >= 32 ? 0xFFFFFFFFu : ((1u << (h2 - l2)) - 1u)) << l2);
        }
        uint4* dst;
        if constexpr (BITS == 3)
          dst = (uint4*)(a.pl.vcode + ((3 * (trow >> 7) + ((trow & 127) >> 6)) * D + dim) * 16);
        else
          dst = (uint4*)(a.pl.vcode + ((trow / VB + blk) * D + dim) * 16);
        uint4 row = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        if ((m[0] & m[1] & m[2] & m[3]) != 0xFFFFFFFFu) {
          const uint4 old = *dst;
          row.x = (old.x & ~m[0]) | (row.x & m[0]);
          row.y = (old.y & ~m[1]) | (row.y & m[1]);
          row.z = (old.z & ~m[2]) | (row.z & m[2]);
          row.w = (old.w & ~m[3]) | (row.w & m[3]);
        }
        *dst = row;
      } else {
        // 3 bits: high-plane words of the tile (positions 32 hw .. 32 hw + 31
        // at bit hi_bit(t)); 8 bytes, no other tile writes them
        const int lo = max(p0, max(c0, qlo)), hi = min(p0 + PT, min(c1, qhi));
        if (lo >= hi) continue;
        uint32_t wd[2];
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          uint32_t word = 0u;
#pragma unroll
          for (int n = 0; n < 32; ++n) {
            const int t = 32 * hw + n;
            const uint32_t code = L.vc[t * VCS + dim];
            word |= (code >> 2) << (hi_bit(t) & 31);
          }
          wd[hw] = word;
        }
        uint32_t m0 = 0xFFFFFFFFu, m1 = 0xFFFFFFFFu;
        if (lo > p0 || hi < p0 + PT) {
          m0 = m1 = 0u;
          for (int t = lo - p0; t < hi - p0; ++t) {
            const int hb = hi_bit(t);
            if (hb < 32) m0 |= 1u << hb;
            else m1 |= 1u << (hb - 32);
          }
        }
        const int sel = (int)((trow & 127) >> 6);
        uint2* dst = (uint2*)(a.pl.vcode + ((3 * (trow >> 7) + 2) * D + dim) * 16 + 8 * sel);
        uint2 row = make_uint2(wd[0], wd[1]);
        if ((m0 & m1) != 0xFFFFFFFFu) {
          const uint2 old = *dst;
          row.x = (old.x & ~m0) | (row.x & m0);
          row.y = (old.y & ~m1) | (row.y & m1);
        }
        *dst = row;
      }
    }
  };

  int64_t prev_trow = -1;  // the previous tile, whose value-code rows are still to be written
  int prev_p0 = -1;
  for (; p0 < c1; p0 += PT) {
    // quantized-plane row of the tile's first position (a tile never crosses
    // a page); -1 when its page is unmapped, and then no code is stored
    const int64_t trow = p0 + PT > qlo && p0 < qhi ? qrow(qm, p0) : -1;
#pragma unroll
    for (int u = 0; u < NPRE; ++u) {
      const int x = tid + NT * u;
      const int which = x >> 10, r = (x >> 4) & 63, c = x & 15;
      *(uint4*)((which ? L.v : L.k) + r * RS + c * 8) = pre[u];
      if (u < NPRE / 2)
        *(uint4*)(L.ka + r * RS + c * 8) =
            make_uint4(pre[u].x & 0x7FFF7FFFu, pre[u].y & 0x7FFF7FFFu, pre[u].z & 0x7FFF7FFFu,
                       pre[u].w & 0x7FFF7FFFu);
    }
    __syncthreads();
    if (p0 + PT < c1) load_tile(p0 + PT);
    if (prev_p0 >= 0) rows(prev_p0, prev_trow);  // L.vc still holds the previous tile's codes

    // ---- transform on the matrix cores (all waves); flag entries near a
    // rounding boundary
    {
      // the row blocks of 16 rows are computed two at a time (independent
      // MFMA chains keep the matrix core busy).  T1 products: two MFMAs of 16
      // products per 32-step (the lane's eight k values split in halves),
      // each from zero, folded in fp32 in a tree of depth 3; T2 and T3
      // products (below 2^-8 of T1's) in one chain; cab: |k| |T1| products
      // (|k| staged in LDS with the tile), which bound the partial sums
      f32x4 s01[4], q2[4], c23[4], cab[4];
#pragma unroll
      for (int rp = 0; rp < 4; rp += 2) {  // two row blocks at a time
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint4 bv = __builtin_bit_cast(uint4, b1[ks]);
          const bf16x8 b1a = abs_bf16x8(b1[ks]);
#pragma unroll
          for (int rb = rp; rb < rp + 2; ++rb) {
            const int ao = (16 * rb + (lane & 15)) * RS + 32 * ks + 8 * (lane >> 4);
            const uint4 av = *(const uint4*)(L.k + ao);
            const bf16x8 A = as_bf16x8(av);
            const bf16x8 Aab = as_bf16x8(*(const uint4*)(L.ka + ao));
            const f32x4 plo = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                as_bf16x4(av.x, av.y), as_bf16x4(bv.x, bv.y), f32x4{}, 0, 0, 0);
            const f32x4 phi = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                as_bf16x4(av.z, av.w), as_bf16x4(bv.z, bv.w), f32x4{}, 0, 0, 0);
            c23[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, b2[ks], ks == 0 ? f32x4{} : c23[rb], 0, 0, 0);
            c23[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, b3[ks], c23[rb], 0, 0, 0);
            cab[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aab, b1a, ks == 0 ? f32x4{} : cab[rb], 0, 0, 0);
            const f32x4 qk = plo + phi;
            if (ks == 0) s01[rb] = qk;
            else if (ks == 1) s01[rb] = s01[rb] + qk;
            else if (ks == 2) q2[rb] = qk;
            else s01[rb] = s01[rb] + (q2[rb] + qk);
          }
        }
      }
      // rows of this lane's entries inside [c0, c1): bit 4 rb + r
      uint32_t inr = 0u;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int t = 16 * (n >> 2) + 4 * (lane >> 4) + (n & 3);
        inr |= (uint32_t)((unsigned)(p0 + t - c0) < (unsigned)(c1 - c0)) << n;
      }
      uint32_t flags = 0u;  // bit 4 rb + r: entry (16 rb + 4 (lane / 16) + r, i) lies near a boundary
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * rb + 4 * (lane >> 4) + r;
          const float y = s01[rb][r] + c23[rb][r];
          const uint32_t bits = __float_as_uint(y);
          L.kq[t * RS + i_out] = (uint16_t)((bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16);
          // distance of y to the rounding boundary of its bfloat16 cell
          const int e = (int)((bits >> 23) & 0xFFu);
          const float ulp = __builtin_amdgcn_ldexpf(1.0f, (e > 0 ? e : 1) - 150);
          const float dist = fabsf((float)((int)(bits & 0xFFFFu) - 0x8000)) * ulp;
          // |T| <= |T1| (1 + 2^-8): cab (1 + 2^-7) bounds sum_j |k_j| |T_ij|
          // with room for the rounding of cab itself; 2^-110 covers products
          // below the smallest normal float
          const float err = fmaf(kTransformErr * 1.0079f, cab[rb][r], 0x1p-110f);
          flags |= (uint32_t)(fminf(dist, 16384.0f * ulp) <= err) << (4 * rb + r);
        }
      }
      flags &= inr;
      // the wave's flagged entries into its own segment of the list (exclusive
      // prefix of the per-lane counts from one ballot per count bit), then
      // recomputed four lanes to an entry, lane q running chain q
      const int cnt = __popc(flags);
      int before = 0, total = 0;
#pragma unroll
      for (int b = 0; b < 5; ++b) {
        const uint64_t m = __ballot((cnt >> b) & 1);
        before += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
        total += __popcll(m) << b;
      }
      uint16_t* fl = L.fix + w * FIXW;
      while (flags) {
        const int r = __ffs(flags) - 1;
        flags &= flags - 1u;
        const int t = 16 * (r >> 2) + 4 * (lane >> 4) + (r & 3);
        fl[before++] = (uint16_t)((t << 7) | i_out);
      }
      // the list's writes before any lane of the wave reads it
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // transform_entry's arithmetic: four fp64 FMA chains over dimensions
      // [32 q, 32 q + 32) in order, joined as (s0 + s1) + (s2 + s3)
      for (int base = 0; base < total; base += 16) {
        const int k = base + (lane >> 2), q = lane & 3;
        const int e = k < total ? fl[k] : 0;
        const int t = e >> 7, i = e & (D - 1);
        const float* tr = L.t + i * TS + 32 * q;
        const uint16_t* kr = L.k + t * RS + 32 * q;
        double sq = 0.0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4 ta = *(const float4*)(tr + 8 * c);
          const float4 tb = *(const float4*)(tr + 8 * c + 4);
          const uint4 kk = *(const uint4*)(kr + 8 * c);
          const float tv[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
          const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) sq = fma((double)tv[j], (double)bf16_lane(kw, j), sq);
        }
        const double pair = sq + partner_d<0xB1>(sq);  // lanes q = 0, 2: s0 + s1, s2 + s3
        const double y = pair + partner_d<0x4E>(pair);  // lane q = 0: (s0 + s1) + (s2 + s3)
        if (q == 0 && k < total) L.kq[t * RS + i] = f64_to_bf16(y);
      }
    }
    __syncthreads();

    // ---- windows and quantization: the key waves take the 64 key groups,
    // the value waves the 64 value groups
    if (!vwave) {
      windows(false, p0);
      quant_group(std::integral_constant<bool, false>{}, p0, trow);
    } else {
      windows(true, p0);
      quant_group(std::integral_constant<bool, true>{}, p0, trow);
    }
    __syncthreads();  // LDS tiles are rewritten by the next iteration
    prev_p0 = p0;
    prev_trow = trow;
  }
  if (prev_p0 >= 0) rows(prev_p0, prev_trow);
}

}  // namespace

hipError_t launch_prefill(const AppendArgs& a, int grid_x, int n_seq, hipStream_t st) {
  dim3 grid(grid_x, a.g.n_kv, n_seq);
  if (a.g.bits == 2)
    hipLaunchKernelGGL(prefill_kernel<2>, grid, dim3(NT), 0, st, a);
  else if (a.g.bits == 3)
    hipLaunchKernelGGL(prefill_kernel<3>, grid, dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_kernel<4>, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

bool prefill_supported(int codec, double p_lo, double p_hi) {
  if (codec == WUSHKV_CODEC_RMS) return true;
  const double hlo = p_lo * (double)(D - 1), hhi = p_hi * (double)(D - 1);
  return (int)floor(hlo) <= 1 && (int)floor(hhi) >= D - 3;
}

}  // namespace wkv
