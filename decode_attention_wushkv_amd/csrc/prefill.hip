// Prefill append for bfloat16 inputs: the key transform of whole position
// tiles on the matrix cores, then selection, quantization and packing (WUSH-KV
// paper page, sections 4.2, 4.4, 5.3; appendix B.3 for the level grid).
//
// One workgroup (4 waves) takes up to 1024 new positions of one (sequence,
// KV head), in tiles of 64 positions aligned to the value-code blocks.
//
// Transform.  k' = T_K k for the 64 keys of a tile is a [64 x 128] x
// [128 x 128] product.  T_K (fp32) is split exactly into three bfloat16 parts,
// T = T1 + T2 + T3 (8 + 8 + 8 significant bits), held as MFMA operands in
// registers for the whole workgroup; bfloat16 keys times bfloat16 parts are
// exact products, summed by v_mfma_f32_32x32x16_bf16 in fp32: T1 products in
// eight MFMAs of 16 folded into one fp32 sum, T2 and T3 products in one chain
// each.  A product of |k| and |T1| bounds A = sum_j |k_j| |T_ij|, and 2^-18 A
// bounds the fp32 error of the sum.  An entry whose fp32 value lies within that bound of
// a bfloat16 rounding boundary is recomputed in fp64 with the arithmetic of
// the one-position paths (transform_entry; a few per cent of the entries), so
// the stored bfloat16 keys are identical to theirs.
//
// Quantization.  Each group (one position's 128 key or value entries) is
// split over a lane pair.  A lane scans its 64 entries keeping the three
// smallest and three largest (v_med3 insertion), the pair merges them, and the
// order statistics around h = p (n - 1) give the linear-interpolation
// percentiles.  This covers clip percentiles whose interpolation needs only
// the three smallest and three largest values (p_lo (n - 1) < 2 and
// p_hi (n - 1) >= 125; the host falls back to the rank-sort kernel otherwise).
// With the RMS codec the clip ends are -alpha rms, +alpha rms instead (sum of
// squares per half-group in fp64, as in quant.h).  Scale, zero and levels
// follow quant.h exactly; value-code rows are
// assembled in LDS with atomic ORs and written as whole 16-byte rows.
#include "quant.h"

namespace wkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int PT = PREFILL_TILE;  // positions per tile
constexpr int PCH = PREFILL_SPAN; // positions per workgroup
constexpr int RS = 136;           // LDS row stride (bf16 elements) of the key / value tiles
constexpr int TS = 132;           // LDS row stride (floats) of T_K
constexpr int FIXMAX = PT * D;    // recomputation list capacity (every entry of a tile)
// fp32 summation error bound of the transform relative to sum_j |k_j| |T_ij|,
// counting one ulp (2^-23) per rounding: 15 roundings inside each 16-product
// T1 MFMA, 7 from folding the eight results together, the T2 chain below 2^-8
// of T (about half an ulp overall), the final additions; 24 ulp = 2^-18.4,
// and 2^-18 keeps a margin.
constexpr float kTransformErr = 3.814697265625e-06f;  // 2^-18

struct __align__(16) PLds {
  float t[D * TS];        // T_K rows (fp32)
  uint16_t k[PT * RS];    // input keys (bf16)
  uint16_t v[PT * RS];    // values (bf16)
  uint16_t kq[PT * RS];   // transformed keys (bf16)
  uint16_t fix[FIXMAX];   // entries to recompute: row << 7 | dimension
  uint32_t vrow[2 * D * 4];  // value-code rows of the tile: two blocks at 4 bits; at 3 bits
                             // the low-plane row and (words 0..1) the tile's half of the
                             // high-plane row
  int nfix;
};

__device__ __forceinline__ __bf16 bf16_of_bits(uint32_t b) {
  return __builtin_bit_cast(__bf16, (uint16_t)b);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 abs_bf16x8(bf16x8 x) {
  const uint4 u = __builtin_bit_cast(uint4, x);
  return as_bf16x8(make_uint4(u.x & 0x7FFF7FFFu, u.y & 0x7FFF7FFFu, u.z & 0x7FFF7FFFu,
                              u.w & 0x7FFF7FFFu));
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

__device__ __forceinline__ float partner(float x) {  // value of lane ^ 1
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

template <int BITS>
__global__ __launch_bounds__(256, 1) void prefill_kernel(AppendArgs a) {
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

  // ---- T_K of this head into LDS; MFMA operands of this wave's 32 output dims
  {
    const float4* tg = (const float4*)(a.tk + (int64_t)h * D * D);
    for (int x = tid; x < D * D / 4; x += 256) {
      const int r = (4 * x) / D, c = (4 * x) % D;
      *(float4*)(L.t + r * TS + c) = tg[x];
    }
  }
  __syncthreads();
  // lane: output dim i, k-slice 8 (lane / 32) .. + 8 of each 16-step
  const int i_out = 32 * w + (lane & 31);
  bf16x8 b1[8], b2[8], b3[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = L.t[i_out * TS + 16 * ks + 8 * (lane >> 5) + e];
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
  uint4 pre[8];
  auto load_tile = [&](int p0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int x = tid + 256 * u;  // 2 tensors x 64 rows x 16 chunks of 16 B
      const int which = x >> 10, r = (x >> 4) & 63, c = x & 15;
      const int p = p0 + r;
      pre[u] = make_uint4(0u, 0u, 0u, 0u);
      if (p >= c0 && p < c1) {
        const int64_t row = (tok0 + (p - L0)) * g.n_kv + h;
        pre[u] = ((const uint4*)((which ? vin : kin) + row * D))[c];
      }
    }
  };
  int p0 = c0 - (c0 - base) % PT;
  load_tile(p0);

  for (; p0 < c1; p0 += PT) {
    // quantized-plane row of the tile's first position (a tile never crosses
    // a page); -1 when its page is unmapped, and then no code is stored
    const int64_t trow = p0 + PT > qlo && p0 < qhi ? qrow(qm, p0) : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int x = tid + 256 * u;
      const int which = x >> 10, r = (x >> 4) & 63, c = x & 15;
      *(uint4*)((which ? L.v : L.k) + r * RS + c * 8) = pre[u];
    }
    for (int x = tid; x < 2 * D * 4; x += 256) L.vrow[x] = 0u;
    if (tid == 0) L.nfix = 0;
    __syncthreads();
    if (p0 + PT < c1) load_tile(p0 + PT);

    // ---- transform on the matrix cores; flag entries near a rounding boundary
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      uint4 av[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        av[ks] = *(const uint4*)(L.k + (32 * rb + (lane & 31)) * RS + 16 * ks + 8 * (lane >> 5));
      // T1 products: one MFMA per 16-step from zero, folded into s1 in fp32
      f32x16 s1 = f32x16{}, c2 = f32x16{}, c3 = f32x16{}, cab = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 A = as_bf16x8(av[ks]);
        const bf16x8 Aab = as_bf16x8(make_uint4(av[ks].x & 0x7FFF7FFFu, av[ks].y & 0x7FFF7FFFu,
                                                av[ks].z & 0x7FFF7FFFu, av[ks].w & 0x7FFF7FFFu));
        const f32x16 p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, b1[ks], f32x16{}, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, b2[ks], c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, b3[ks], c3, 0, 0, 0);
        cab = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aab, abs_bf16x8(b1[ks]), cab, 0, 0, 0);
        s1 = ks == 0 ? p1 : s1 + p1;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * rb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float y = s1[r] + (c2[r] + c3[r]);
        const uint32_t bits = __float_as_uint(y);
        L.kq[t * RS + i_out] = (uint16_t)((bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16);
        // distance of y to the rounding boundary of its bfloat16 cell
        const int e = (int)((bits >> 23) & 0xFFu);
        const float ulp = __builtin_amdgcn_ldexpf(1.0f, (e > 0 ? e : 1) - 150);
        const float dist = fabsf((float)((int)(bits & 0xFFFFu) - 0x8000)) * ulp;
        // |T| <= |T1| (1 + 2^-8): cab (1 + 2^-7) bounds sum_j |k_j| |T_ij| with
        // room for the rounding of cab itself
        const float err = kTransformErr * cab[r] * 1.0079f;
        const bool near = dist <= err || err >= 16384.0f * ulp;
        if (near && p0 + t >= c0 && p0 + t < c1) {
          const int slot = atomicAdd(&L.nfix, 1);
          L.fix[slot] = (uint16_t)((t << 7) | i_out);
        }
      }
    }
    __syncthreads();

    // ---- recompute flagged entries: fp64 FMAs in dimension order
    {
      const int nf = L.nfix;
      for (int x = tid; x < nf; x += 256) {
        const int t = L.fix[x] >> 7, i = L.fix[x] & (D - 1);
        const uint16_t* kr = L.k + t * RS;
        const float* tr = L.t + i * TS;
        const double acc = transform_entry([&](int j) { return tr[j]; },
                                           [&](int j) { return bf16_bits_to_f32(kr[j]); });
        L.kq[t * RS + i] = f64_to_bf16(acc);
      }
    }
    __syncthreads();

    // ---- windows: positions of the tile kept in bfloat16
    for (int x = tid; x < PT * 16 * 2; x += 256) {
      const int which = x >> 10, r = (x >> 4) & 63, c = x & 15;
      const int p = p0 + r;
      if (p < c0 || p >= c1 || (p >= qlo && p < qhi)) continue;
      const uint4 val = *(const uint4*)((which ? L.v : L.kq) + r * RS + c * 8);
      uint16_t* dst;
      if (p < g.S)
        dst = (which ? a.pl.vsink : a.pl.ksink) + (unit * g.S + p) * D;
      else
        dst = (which ? a.pl.vring : a.pl.kring) + (unit * g.W + (p - g.S) % g.W) * D;
      ((uint4*)dst)[c] = val;
    }

    // ---- groups: lane pair per (position, key or value); lane half hh holds
    // dimensions [64 hh, 64 hh + 64)
    {
      const int grp = tid >> 1, hh = tid & 1, t = grp & 63;
      const bool isv = grp >= 64;
      const int p = p0 + t;
      const bool quant = p >= qlo && p < qhi;
      const uint16_t* row = (isv ? L.v : L.kq) + t * RS + 64 * hh;
      double lo, hi;
      if (g.codec == WUSHKV_CODEC_RMS) {
        // sum of squares of this lane's half in dimension order, then the two
        // halves in order (quant.h's rms_of_halves)
        double ss = 0.0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint4 u4 = *(const uint4*)(row + 8 * c);
          const uint32_t uw[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double x = (double)__uint_as_float((e & 1) ? (uw[e >> 1] & 0xFFFF0000u)
                                                            : (uw[e >> 1] << 16));
            ss = fma(x, x, ss);
          }
        }
        const uint64_t sb = __builtin_bit_cast(uint64_t, ss);
        const uint64_t pb = (uint64_t)(uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)sb, 0xB1, 0xF, 0xF, false) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(sb >> 32), 0xB1, 0xF, 0xF, false) << 32);
        const double ps = __builtin_bit_cast(double, pb);
        const double rms = hh == 0 ? rms_of_halves(ss, ps) : rms_of_halves(ps, ss);
        lo = -g.alpha * rms;
        hi = g.alpha * rms;
      } else {
      float a0 = INFINITY, a1 = INFINITY, a2 = INFINITY;
      float bb0 = -INFINITY, bb1 = -INFINITY, bb2 = -INFINITY;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 u4 = *(const uint4*)(row + 8 * c);
        const uint32_t uw[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = __uint_as_float((e & 1) ? (uw[e >> 1] & 0xFFFF0000u) : (uw[e >> 1] << 16));
          sel_insert(x, a0, a1, a2, bb0, bb1, bb2);
        }
      }
      {  // merge with the other half of the group
        const float pa0 = partner(a0), pa1 = partner(a1), pa2 = partner(a2);
        const float pb0 = partner(bb0), pb1 = partner(bb1), pb2 = partner(bb2);
        float d0 = bb0, d1 = bb1, d2 = bb2;
        sel_insert(pa0, a0, a1, a2, d0, d1, d2);
        sel_insert(pa1, a0, a1, a2, d0, d1, d2);
        sel_insert(pa2, a0, a1, a2, d0, d1, d2);
        float e0 = INFINITY, e1 = INFINITY, e2 = INFINITY;
        sel_insert(pb0, e0, e1, e2, bb0, bb1, bb2);
        sel_insert(pb1, e0, e1, e2, bb0, bb1, bb2);
        sel_insert(pb2, e0, e1, e2, bb0, bb1, bb2);
      }
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
      float bnd[LEV];
      float inv = 0.f, zf = (float)zd;
      if (BITS <= 3) {
#pragma unroll
        for (int c = 0; c < LEV; ++c) {
          const double tb = zd + ((double)c + 0.5) * sd;
          bnd[c] = sd == 0.0 ? INFINITY : ((c & 1) ? f32_up(tb) : f32_down(tb));
        }
      } else {
        inv = sd == 0.0 ? 0.f : (float)(1.0 / sd);
      }
      // codes of this lane's 64 dimensions; at 3 bits words 0..3 hold the low
      // plane and words 4..5 the high plane
      uint32_t packed[BITS * 2];
#pragma unroll
      for (int q = 0; q < BITS * 2; ++q) packed[q] = 0u;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 u4 = *(const uint4*)(row + 8 * c);
        const uint32_t uw[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * c + e;  // dimension 64 hh + d
          const float x = __uint_as_float((e & 1) ? (uw[e >> 1] & 0xFFFF0000u) : (uw[e >> 1] << 16));
          int code;
          if (BITS <= 3) {
            code = 0;
#pragma unroll
            for (int c2 = 0; c2 < LEV; ++c2) code += (c2 & 1) ? (x >= bnd[c2] ? 1 : 0) : (x > bnd[c2] ? 1 : 0);
          } else if (sd == 0.0) {
            code = 0;
          } else {
            // estimate, then the exact boundary test on both sides
            int cc = (int)rintf((x - zf) * inv);
            cc = cc < 0 ? 0 : (cc > LEV ? LEV : cc);
            const double xd = (double)x;
            if (cc > 0 && !above_boundary(xd, zd, sd, cc - 1))
              cc -= 1;
            else if (cc < LEV && above_boundary(xd, zd, sd, cc))
              cc += 1;
            code = cc;
          }
          if (BITS == 3) {
            // selects rather than indexing keep the words in registers
            const uint32_t lv = ((uint32_t)code & 3u) << (2 * (d & 15));
            const int hb = hi_bit(d);
            const uint32_t hv = ((uint32_t)code >> 2) << (hb & 31);
            const int lw = d >> 4;
            packed[0] |= lw == 0 ? lv : 0u;
            packed[1] |= lw == 1 ? lv : 0u;
            packed[2] |= lw == 2 ? lv : 0u;
            packed[3] |= lw == 3 ? lv : 0u;
            packed[4] |= hb < 32 ? hv : 0u;
            packed[5] |= hb < 32 ? 0u : hv;
          } else {
            packed[(d * BITS) >> 5] |= (uint32_t)code << ((d * BITS) & 31);
          }
          if (isv && quant) {
            // value row of dimension 64 hh + d, position t of the tile
            const int dim = 64 * hh + d;
            if (BITS == 3) {
              atomicOr(&L.vrow[dim * 4 + (t >> 4)], ((uint32_t)code & 3u) << (2 * (t & 15)));
              // the tile is one half of its 128-position block: high-plane words
              // 2 (p0 / 64 % 2) and + 1, kept in words 0..1 of the second row
              const int hb = hi_bit(t);  // < 64: the half's bits are those of t
              atomicOr(&L.vrow[(D + dim) * 4 + (hb >> 5)], ((uint32_t)code >> 2) << (hb & 31));
            } else {
              const int blk = t / VB, pos = t % VB;
              atomicOr(&L.vrow[(blk * D + dim) * 4 + (pos * BITS >> 5)], (uint32_t)code << ((pos * BITS) & 31));
            }
          }
        }
      }
      if (quant && trow >= 0) {
        if (!isv) {
          if (BITS == 3) {
            uint8_t* kr = a.pl.kcode + (trow + t) * 48;
            *(uint4*)(kr + 16 * hh) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
            *(uint2*)(kr + 32 + 8 * hh) = make_uint2(packed[4], packed[5]);
          } else {
            uint4* kd = (uint4*)(a.pl.kcode + (trow + t) * (16 * BITS) + hh * 8 * BITS);
#pragma unroll
            for (int q = 0; q < BITS / 2; ++q)
              kd[q] = make_uint4(packed[4 * q], packed[4 * q + 1], packed[4 * q + 2], packed[4 * q + 3]);
          }
        }
        if (hh == 0) (isv ? a.pl.vsz : a.pl.ksz)[trow + t] = (uint32_t)s16 | ((uint32_t)z16 << 16);
      }
    }
    __syncthreads();

    // ---- value-code rows: one 16-byte row per (block, dimension); rows
    // partly outside the quantized positions of the tile keep their other bits
    if constexpr (BITS == 3) {
      // the tile's low-plane row (16 bytes per dimension) and its half of the
      // block's high-plane row (8 bytes: no other tile writes them)
      const int lo = max(p0, max(c0, qlo)), hi = min(p0 + PT, min(c1, qhi));
      const int64_t vb = 3 * (trow >> 7);
      const int sel = (int)((trow & 127) >> 6);
      for (int x = tid; x < 2 * D; x += 256) {
        const int which = x / D, dim = x % D;
        if (lo >= hi || trow < 0) continue;
        const uint32_t* src = &L.vrow[(which * D + dim) * 4];
        if (which == 0) {
          uint32_t m[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int bl = (lo - p0) * 2 - 32 * q, bh = (hi - p0) * 2 - 32 * q;
            const int l2 = bl < 0 ? 0 : (bl > 32 ? 32 : bl), h2 = bh < 0 ? 0 : (bh > 32 ? 32 : bh);
            m[q] = h2 <= l2 ? 0u : ((h2 - l2 >= 32 ? 0xFFFFFFFFu : ((1u << (h2 - l2)) - 1u)) << l2);
          }
          uint4* dst = (uint4*)(a.pl.vcode + ((vb + sel) * D + dim) * 16);
          uint4 row = make_uint4(src[0], src[1], src[2], src[3]);
          if ((m[0] & m[1] & m[2] & m[3]) != 0xFFFFFFFFu) {
            const uint4 old = *dst;
            row.x = (old.x & ~m[0]) | (row.x & m[0]);
            row.y = (old.y & ~m[1]) | (row.y & m[1]);
            row.z = (old.z & ~m[2]) | (row.z & m[2]);
            row.w = (old.w & ~m[3]) | (row.w & m[3]);
          }
          *dst = row;
        } else {
          uint32_t m0 = 0xFFFFFFFFu, m1 = 0xFFFFFFFFu;
          if (lo > p0 || hi < p0 + PT) {
            m0 = m1 = 0u;
            for (int t = lo - p0; t < hi - p0; ++t) {
              const int hb = hi_bit(t);
              if (hb < 32) m0 |= 1u << hb;
              else m1 |= 1u << (hb - 32);
            }
          }
          uint2* dst = (uint2*)(a.pl.vcode + ((vb + 2) * D + dim) * 16 + 8 * sel);
          uint2 row = make_uint2(src[0], src[1]);
          if ((m0 & m1) != 0xFFFFFFFFu) {
            const uint2 old = *dst;
            row.x = (old.x & ~m0) | (row.x & m0);
            row.y = (old.y & ~m1) | (row.y & m1);
          }
          *dst = row;
        }
      }
    } else {
      const int nblk = PT / VB;  // 1 (2 bits) or 2 (4 bits)
      for (int x = tid; x < nblk * D; x += 256) {
        const int blk = x / D, dim = x % D;
        const int b0 = p0 + blk * VB;
        const int lo = max(b0, max(c0, qlo)), hi = min(b0 + VB, min(c1, qhi));
        if (lo >= hi || trow < 0) continue;
        uint32_t m[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int bl = max(lo - b0, 0) * BITS - 32 * q, bh = (hi - b0) * BITS - 32 * q;
          const int l2 = bl < 0 ? 0 : (bl > 32 ? 32 : bl), h2 = bh < 0 ? 0 : (bh > 32 ? 32 : bh);
          m[q] = h2 <= l2 ? 0u : ((h2 - l2 >= 32 ? 0xFFFFFFFFu : ((1u << (h2 - l2)) - 1u)) << l2);
        }
        const uint32_t* src = &L.vrow[(blk * D + dim) * 4];
        uint4* dst = (uint4*)(a.pl.vcode + ((trow / VB + blk) * D + dim) * 16);
        uint4 row = make_uint4(src[0], src[1], src[2], src[3]);
        if ((m[0] & m[1] & m[2] & m[3]) != 0xFFFFFFFFu) {
          const uint4 old = *dst;
          row.x = (old.x & ~m[0]) | (row.x & m[0]);
          row.y = (old.y & ~m[1]) | (row.y & m[1]);
          row.z = (old.z & ~m[2]) | (row.z & m[2]);
          row.w = (old.w & ~m[3]) | (row.w & m[3]);
        }
        *dst = row;
      }
    }
    __syncthreads();  // LDS tiles are rewritten by the next iteration
  }
}

}  // namespace

hipError_t launch_prefill(const AppendArgs& a, int grid_x, int n_seq, hipStream_t st) {
  dim3 grid(grid_x, a.g.n_kv, n_seq);
  if (a.g.bits == 2)
    hipLaunchKernelGGL(prefill_kernel<2>, grid, dim3(256), 0, st, a);
  else if (a.g.bits == 3)
    hipLaunchKernelGGL(prefill_kernel<3>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_kernel<4>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

bool prefill_supported(int codec, double p_lo, double p_hi) {
  if (codec == WUSHKV_CODEC_RMS) return true;
  const double hlo = p_lo * (double)(D - 1), hhi = p_hi * (double)(D - 1);
  return (int)floor(hlo) <= 1 && (int)floor(hhi) >= D - 3;
}

}  // namespace wkv
