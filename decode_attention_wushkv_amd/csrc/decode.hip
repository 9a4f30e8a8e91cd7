// wushkv_decode_attn kernels: GQA decode attention over the mixed cache
// (WUSH-KV paper page: section 4.1 for the cache and GQA head sharing,
// section 4.2 / appendix B.1 for the T_K^{-T} query compensation, section
// 4.4 for the full-precision windows, appendix D.1 for the 1/sqrt(d) scale).
//
// Three launches per call:
//   qcomp   one workgroup per (sequence, KV head): q' = T_K^{-T} q for its G
//           query heads, prescaled by log2(e)/sqrt(d); sigma = sum_i q'_i (the
//           zero point factors out of a score: q'.(z + s c) = z sigma +
//           s (q'.c)); q' as a fixed-point vector (QDIG signed base-16
//           digits) for the integer dot products.
//   split   one workgroup per (sequence, KV head, chunk of the quantized
//           region) plus one for the bfloat16 sink + recent entries.
//             quantized chunk: every thread prefetches its share of the chunk's
//             key codes, value codes and scale/zero words into registers;
//             scores q'.c come from v_dot8 (4-bit x 4-bit) on the unpacked
//             codes and the query digits; the chunk max gives exp2 weights
//             w_t = p_t s_t, quantized to WDIG base-16 digits against the
//             chunk's largest value scale; o_i = sum_t w_t c_{t,i} is again
//             v_dot8 over the dim-major value codes and the weight digits;
//             o += sum_t p_t z_t.
//             window chunk: fp32 dot products over bfloat16 rows.
//           Each wave handles a quarter of its workgroup's chunk with its own
//           max; the workgroup merges the four and writes (o, m, l) per query
//           head.
//   combine one workgroup per (sequence, query head): log-sum-exp merge of the
//           chunk partials into the fp32 output.
#include "common.h"

namespace wkv {
namespace {

constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;
// Largest |q_i| representable by QDIG balanced base-16 digits in [-8, 7].
constexpr int pow16m1(int n) { return n == 0 ? 0 : 16 * pow16m1(n - 1) + 15; }
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

// Wave-wide sum / max: DPP within rows of 16 lanes, then the four row results
// read into scalars.
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

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Value of the neighbouring lane (lane ^ 1) via DPP quad_perm [1, 0, 3, 2].
__device__ __forceinline__ int swap_adjacent(int x) {
  return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
}

// ---------------------------------------------------------------- qcomp

template <int IO_BF16, int BITS>
__global__ __launch_bounds__(128) void qcomp_kernel(DecodeArgs a) {
  __shared__ float qv[8][D];
  __shared__ float red[2][2];
  __shared__ int8_t dig[QDIG][D];
  const int h = blockIdx.x, si = blockIdx.y, i = threadIdx.x;
  const int G = a.g.G, nq = a.g.n_q;
  const int lane = i & 63, wv = i >> 6;
  for (int g = 0; g < G; ++g) qv[g][i] = load_io<IO_BF16>(a.q, ((int64_t)si * nq + h * G + g) * D + i);
  float trow[D];
  const float4* tp = (const float4*)(a.tq + ((int64_t)h * D + i) * D);
#pragma unroll
  for (int c = 0; c < D / 4; ++c) {
    float4 t4 = tp[c];
    trow[4 * c] = t4.x;
    trow[4 * c + 1] = t4.y;
    trow[4 * c + 2] = t4.z;
    trow[4 * c + 3] = t4.w;
  }
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < D; ++j) acc = fmaf(trow[j], qv[g][j], acc);
    acc *= kLog2eOverSqrtD;
    float* rec = a.wsq + ((int64_t)si * nq + h * G + g) * QS;
    uint32_t* reci = (uint32_t*)rec;
    rec[i] = acc;
    float s = wave_sum(acc);
    float mx = wave_max(fabsf(acc));
    if (lane == 0) {
      red[wv][0] = s;
      red[wv][1] = mx;
    }
    __syncthreads();
    const float sigma = red[0][0] + red[1][0];
    const float maxabs = fmaxf(red[0][1], red[1][1]);
    const float sq = maxabs > 0.f ? (float)QMAX / maxabs : 1.f;
    int qi = (int)rintf(acc * sq);
    qi = qi > QMAX ? QMAX : (qi < -QMAX ? -QMAX : qi);
    const int qsum = wave_sum_i(qi);
    // balanced base-16 digits d_k in [-8, 7]: qi = sum_k 16^k d_k
    int r = qi;
#pragma unroll
    for (int k = 0; k < QDIG - 1; ++k) {
      int d = ((r + 8) & 15) - 8;
      dig[k][i] = (int8_t)d;
      r = (r - d) >> 4;
    }
    dig[QDIG - 1][i] = (int8_t)r;
    if (lane == 0) reci[QOFF_QSUM + wv] = (uint32_t)qsum;
    if (i == 0) {
      rec[QOFF_SIGMA] = sigma;
      rec[QOFF_INVS] = 1.f / sq;
    }
    __syncthreads();
    {
      // Word i of the digit block: group i / DIGP of 8 dimensions, digit
      // k = i % DIGP; nibble n holds that digit of one dimension of the group.
      //   2 bits: group = half * 8 + w * 2 + parity, dims 64 half + 16 w + 2 n + parity
      //   4 bits: group = half * 8 + w,              dims 64 half + 8 w + n
      const int grp16 = i / DIGP, k = i % DIGP, half = grp16 >> 3;
      int e0, step;
      if (BITS == 2) {
        e0 = 64 * half + 16 * ((grp16 >> 1) & 3) + (grp16 & 1);
        step = 2;
      } else {
        e0 = 64 * half + 8 * (grp16 & 7);
        step = 1;
      }
      uint32_t word = 0;
      if (k < QDIG)
#pragma unroll
        for (int n = 0; n < 8; ++n) word |= ((uint32_t)dig[k][e0 + step * n] & 15u) << (4 * n);
      reci[QOFF_LIMB + i] = word;
    }
    __syncthreads();
  }
}


// ---------------------------------------------------------------- split

template <int BITS, int G>
struct SplitCfg {
  static constexpr int TW = sub_len(BITS);     // positions per wave sub-chunk
  static constexpr int VB = 128 / BITS;        // positions per value-code block
  static constexpr int NBW = TW / VB;          // value blocks per sub-chunk (2)
  static constexpr int CB = 16 * BITS;         // key-code bytes per position
  static constexpr int ROWS = TW / 32;         // positions per lane pair
  static constexpr int KQ = CB / 32;           // uint4 per lane (half a position)
  static constexpr int GS = BITS == 2 ? 16 : 8;  // positions per 32-bit value-row word
  static constexpr int NG = TW / GS;           // value-row words per sub-chunk (8)
  static constexpr int WGW = BITS == 2 ? 2 * WDIG : WDIG;  // digit words per row word
  static constexpr int WGP = (WGW + 3) / 4 * 4;            // ... padded to 16 bytes
  static constexpr bool QREG = G <= 2;         // query digits held in registers
  // LDS words
  static constexpr int QLDS = QREG ? 0 : G * 16 * DIGP;
  static constexpr int WAVE = G * TW + G * NG * WGP;      // weights + digit words, per wave
  static constexpr int PART = 4 * G * (D + 2);            // wave partials (o, m, l)
  static constexpr int QUANT = QLDS + 4 * WAVE + PART;
  static constexpr int WIN = G * D + G * WINDOW_MAX;
  static constexpr int UNION = QUANT > WIN ? QUANT : WIN;
  static constexpr int TOTAL = G * D + 64 + UNION;        // obuf + reductions + union
};

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

// Orders this wave's LDS accesses before the following ones (lanes of one
// wave exchange data through LDS without a workgroup barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Registers holding one sub-chunk's codes: key codes (lane pair per
// position), scale/zero words, value rows of dimensions lane and lane + 64.
template <int BITS, int G>
struct SubBuf {
  using C = SplitCfg<BITS, G>;
  uint4 kc[C::ROWS][C::KQ];
  uint32_t ksz[C::ROWS], vsz[C::ROWS];
  uint4 vc[C::NBW][2];
};

template <int BITS, int G>
__device__ __forceinline__ void load_sub(SubBuf<BITS, G>& b, const DecodeArgs& a, int64_t unit,
                                         int pbase, int lo, int hi) {
  using C = SplitCfg<BITS, G>;
  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63, half = lane & 1, tq = lane >> 1;
  const uint8_t* kb = a.pl.kcode + (unit * g.cpos + pbase) * C::CB + half * (C::CB / 2);
#pragma unroll
  for (int r = 0; r < C::ROWS; ++r) {
    const int p = pbase + 32 * r + tq;
    const bool ok = p >= lo && p < hi;
#pragma unroll
    for (int q = 0; q < C::KQ; ++q)
      b.kc[r][q] = ok ? ((const uint4*)(kb + (int64_t)(32 * r + tq) * C::CB))[q] : make_uint4(0, 0, 0, 0);
    b.ksz[r] = ok ? a.pl.ksz[unit * g.cpos + p] : 0u;
    b.vsz[r] = ok ? a.pl.vsz[unit * g.cpos + p] : 0u;
  }
  const uint8_t* vb = a.pl.vcode + ((unit * g.ctx_blocks + pbase / C::VB) * D + lane) * 16;
#pragma unroll
  for (int k = 0; k < C::NBW; ++k) {
    const bool ok = pbase + k * C::VB < hi && pbase + (k + 1) * C::VB > lo;
    b.vc[k][0] = ok ? *(const uint4*)(vb + (int64_t)k * D * 16) : make_uint4(0, 0, 0, 0);
    b.vc[k][1] = ok ? *(const uint4*)(vb + (int64_t)k * D * 16 + 64 * 16) : make_uint4(0, 0, 0, 0);
  }
}

struct QueryRegs {
  float sig, inv, qsum;
};

// Scores, weights and value accumulation of one sub-chunk; folds the result
// into the wave's running (M, Lrun, O) (online softmax across sub-chunks).
template <int BITS, int G>
__device__ __forceinline__ void process_sub(const SubBuf<BITS, G>& b, int pbase, int lo, int hi,
                                            const uint4 (*qd)[8], const uint32_t* qlds,
                                            const QueryRegs* qr, uint32_t* wsm, float* M,
                                            float* Lrun, float (*O)[2]) {
  using C = SplitCfg<BITS, G>;
  const int lane = threadIdx.x & 63, half = lane & 1, tq = lane >> 1;

  // ---- scores (log2 domain)
  float sc[C::ROWS][G];
#pragma unroll
  for (int r = 0; r < C::ROWS; ++r) {
    uint32_t d[4 * C::KQ];
#pragma unroll
    for (int q = 0; q < C::KQ; ++q) {
      d[4 * q] = b.kc[r][q].x;
      d[4 * q + 1] = b.kc[r][q].y;
      d[4 * q + 2] = b.kc[r][q].z;
      d[4 * q + 3] = b.kc[r][q].w;
    }
    const float ks = f16_to_f32(b.ksz[r] & 0xFFFFu), kz = f16_to_f32(b.ksz[r] >> 16);
    const int p = pbase + 32 * r + tq;
    const bool ok = p >= lo && p < hi;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      int acc[QDIG];
#pragma unroll
      for (int k = 0; k < QDIG; ++k) acc[k] = 0;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint4 L = C::QREG ? qd[gg][x] : *(const uint4*)(qlds + (gg * 16 + half * 8 + x) * DIGP);
        const uint32_t Lk[4] = {L.x, L.y, L.z, L.w};
        int X;
        if constexpr (BITS == 2) {
          // x = 2 w + parity: parity 0 takes the even dimensions of code word w
          const uint32_t dw = d[x >> 1];
          X = (int)((x & 1) ? ((dw >> 2) & 0x33333333u) : (dw & 0x33333333u));
        } else {
          X = (int)(d[x] ^ 0x88888888u);  // code - 8 as a signed nibble
        }
#pragma unroll
        for (int k = 0; k < QDIG; ++k) acc[k] = __builtin_amdgcn_sdot8(X, (int)Lk[k], acc[k], false);
      }
      int dot = acc[QDIG - 1];
#pragma unroll
      for (int k = QDIG - 2; k >= 0; --k) dot = dot * 16 + acc[k];
      if (BITS == 4) dot += 8 * (int)qr[gg].qsum;
      dot += swap_adjacent(dot);
      sc[r][gg] = ok ? ks * ((float)dot * qr[gg].inv) + kz * qr[gg].sig : -INFINITY;
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
      pw[r][gg] = half ? 0.f : exp2f(sc[r][gg] - m[gg]);
      wmax[gg] = fmaxf(wmax[gg], pw[r][gg] * f16_to_f32(b.vsz[r] & 0xFFFFu));
    }
    wmax[gg] = wave_max(wmax[gg]);
  }
  uint32_t* wq = wsm;                 // [G][TW], positions of a row word grouped by parity
  uint32_t* wl = wsm + G * C::TW;     // [G][NG][WGP] digit words
  float lsum[G], zsum[G];
  wave_sync();  // previous sub-chunk's reads of wq / wl are done
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float wscale = wmax[gg] > 0.f ? (float)WMAX / wmax[gg] : 0.f;
    lsum[gg] = zsum[gg] = 0.f;
#pragma unroll
    for (int r = 0; r < C::ROWS; ++r) {
      const float vs = f16_to_f32(b.vsz[r] & 0xFFFFu), vz = f16_to_f32(b.vsz[r] >> 16);
      const int t = 32 * r + tq;
      const int slot = BITS == 2 ? ((t & ~15) | ((t & 1) << 3) | ((t & 15) >> 1)) : t;
      lsum[gg] += pw[r][gg];
      zsum[gg] = fmaf(pw[r][gg], vz, zsum[gg]);
      if (!half) wq[gg * C::TW + slot] = (uint32_t)rintf(pw[r][gg] * vs * wscale);
    }
    lsum[gg] = wave_sum(lsum[gg]);
    zsum[gg] = wave_sum(zsum[gg]);
  }
  wave_sync();

  // ---- weight digit words: group gi of GS positions, digit k; nibble n holds
  // digit k of position n of the group's (parity) set
  {
    constexpr int WPG = C::WGW;
    for (int x = lane; x < G * C::NG * WPG; x += 64) {
      const int gg = x / (C::NG * WPG), rem = x % (C::NG * WPG);
      const int gi = rem / WPG, r2 = rem % WPG;
      const int par = BITS == 2 ? r2 / WDIG : 0, k = r2 % WDIG;
      const uint4* src = (const uint4*)(wq + gg * C::TW + gi * C::GS + par * 8);
      const uint4 s0 = src[0], s1 = src[1];
      const uint32_t wv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) word |= ((wv[n] >> (4 * k)) & 15u) << (4 * n);
      wl[(gg * C::NG + gi) * C::WGP + par * WDIG + k] = word;
    }
  }
  wave_sync();

  // ---- o_i = sum_t w_t c_{t,i}: lane = dimensions lane, lane + 64
  uint32_t pa[G][2][WDIG];
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int k = 0; k < WDIG; ++k) pa[gg][e][k] = 0u;
#pragma unroll
  for (int kb = 0; kb < C::NBW; ++kb) {
    if (!(pbase + kb * C::VB < hi && pbase + (kb + 1) * C::VB > lo)) continue;
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
          if constexpr (BITS == 2) {
            const uint32_t E = rw[e][w] & 0x33333333u, Od = (rw[e][w] >> 2) & 0x33333333u;
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
    const float fo = exp2f(M[gg] - Mn), fn = exp2f(m[gg] - Mn);
    const float back = wmax[gg] / (float)WMAX;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float of = (float)pa[gg][e][WDIG - 1];
#pragma unroll
      for (int k = WDIG - 2; k >= 0; --k) of = fmaf(of, 16.f, (float)pa[gg][e][k]);
      O[gg][e] = fmaf(O[gg][e], fo, fmaf(of, back, zsum[gg]) * fn);
    }
    Lrun[gg] = fmaf(Lrun[gg], fo, lsum[gg] * fn);
    M[gg] = Mn;
  }
}

// One wave: sub-chunks c0, c0 + stride, ... (< c_end) of the quantized region
// [lo, hi), two sub-chunks of codes in flight; leaves its partial in po/pm/pl.
template <int BITS, int G>
__device__ void quant_wave(const DecodeArgs& a, int64_t unit, int qbase, int c0, int stride,
                           int c_end, int lo, int hi, const uint32_t* qlds, uint32_t* wsm, float* po,
                           float* pm, float* pl) {
  using C = SplitCfg<BITS, G>;
  const int lane = threadIdx.x & 63, half = lane & 1;
  uint4 qd[C::QREG ? G : 1][8];
  QueryRegs qr[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float* rec = a.wsq + (int64_t)(qbase + gg) * QS;
    qr[gg].sig = rec[QOFF_SIGMA];
    qr[gg].inv = rec[QOFF_INVS];
    qr[gg].qsum = (float)(int)__float_as_uint(rec[QOFF_QSUM + half]);
    if (C::QREG)
#pragma unroll
      for (int x = 0; x < 8; ++x)
        qd[C::QREG ? gg : 0][x] = *(const uint4*)((const uint32_t*)rec + QOFF_LIMB + (half * 8 + x) * DIGP);
  }
  float M[G], Lrun[G], O[G][2];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    M[gg] = -INFINITY;
    Lrun[gg] = 0.f;
    O[gg][0] = O[gg][1] = 0.f;
  }
  SubBuf<BITS, G> A, B;
  int c = c0;
  if (c < c_end) load_sub<BITS, G>(A, a, unit, c * C::TW, lo, hi);
  while (c < c_end) {
    int cn = c + stride;
    if (cn < c_end) load_sub<BITS, G>(B, a, unit, cn * C::TW, lo, hi);
    process_sub<BITS, G>(A, c * C::TW, lo, hi, qd, qlds, qr, wsm, M, Lrun, O);
    c = cn;
    if (c >= c_end) break;
    cn = c + stride;
    if (cn < c_end) load_sub<BITS, G>(A, a, unit, cn * C::TW, lo, hi);
    process_sub<BITS, G>(B, c * C::TW, lo, hi, qd, qlds, qr, wsm, M, Lrun, O);
    c = cn;
  }
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    po[gg * D + lane] = O[gg][0];
    po[gg * D + lane + 64] = O[gg][1];
    if (lane == 0) {
      pm[gg] = M[gg];
      pl[gg] = Lrun[gg];
    }
  }
}

template <int G>
__device__ void window_chunk(const DecodeArgs& a, int64_t unit, int qbase, int Lq, int sq,
                             uint32_t* sm, float* obuf, float* red, float (&m_out)[G],
                             float (&l_out)[G]) {
  const Geometry& g = a.g;
  const int tid = threadIdx.x, half = tid & 1;
  const int i = tid & (D - 1), grp = tid >> 7;
  float* qs = (float*)sm;        // [G][D]
  float* scw = qs + G * D;       // [G][WINDOW_MAX]
  const int ns = Lq < g.S ? Lq : g.S;
  const int ntok = ns + (Lq > sq ? Lq - sq : 0);
  for (int x = tid; x < G * D; x += 256) qs[x] = a.wsq[(int64_t)(qbase + x / D) * QS + (x % D)];
  __syncthreads();
  for (int tok = tid >> 1; tok < ntok; tok += 128) {
    const int p = tok < ns ? tok : sq + (tok - ns);
    const uint16_t* src = tok < ns ? a.pl.ksink + (unit * g.S + p) * D
                                   : a.pl.kring + (unit * g.W + (p - g.S) % g.W) * D;
    const uint4* s4 = (const uint4*)(src + half * 64);
    float dot[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) dot[gg] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 w = s4[c];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf16_to_f32((uint16_t)(ww[e >> 1] >> ((e & 1) * 16)));
#pragma unroll
        for (int gg = 0; gg < G; ++gg) dot[gg] = fmaf(qs[gg * D + half * 64 + c * 8 + e], x, dot[gg]);
      }
    }
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float d2 = dot[gg] + __shfl_xor(dot[gg], 1);
      if (!half) scw[gg * WINDOW_MAX + tok] = d2;
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
  block_reduce<G, false>(ls, red);
  __syncthreads();
  float acc[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) acc[gg] = 0.f;
  for (int tok = grp; tok < ntok; tok += 2) {
    const int p = tok < ns ? tok : sq + (tok - ns);
    const uint16_t* src = tok < ns ? a.pl.vsink + (unit * g.S + p) * D
                                   : a.pl.vring + (unit * g.W + (p - g.S) % g.W) * D;
    const float x = bf16_to_f32(src[i]);
#pragma unroll
    for (int gg = 0; gg < G; ++gg) acc[gg] = fmaf(scw[gg * WINDOW_MAX + tok], x, acc[gg]);
  }
  if (grp == 1)
#pragma unroll
    for (int gg = 0; gg < G; ++gg) obuf[gg * D + i] = acc[gg];
  __syncthreads();
  if (grp == 0)
#pragma unroll
    for (int gg = 0; gg < G; ++gg) obuf[gg * D + i] += acc[gg];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    m_out[gg] = mx[gg];
    l_out[gg] = ls[gg];
  }
}

template <int BITS, int G>
__global__ __launch_bounds__(256, G == 1 ? 3 : (G == 2 ? 2 : 1)) void split_kernel(DecodeArgs a) {
  using C = SplitCfg<BITS, G>;
  extern __shared__ uint4 smem4[];
  uint32_t* smem = (uint32_t*)smem4;
  float* obuf = (float*)smem;             // [G][D] workgroup partial o
  float* red = obuf + G * D;              // [64] reductions
  uint32_t* un = (uint32_t*)(red + 64);   // union

  const Geometry& g = a.g;
  const int j = blockIdx.x, h = blockIdx.y, si = blockIdx.z, tid = threadIdx.x;
  const int slot = a.s.slot[si], Lq = a.s.len[si], sq = a.s.squant[si];
  const int64_t unit = ((int64_t)a.layer * g.max_batch + slot) * g.n_kv + h;
  const int qbase = si * g.n_q + h * G;
  const int nsp = gridDim.x;

  float m[G], l[G];
  bool empty;
  if (j == a.n_splits) {
    const int ns = Lq < g.S ? Lq : g.S;
    empty = ns + (Lq > sq ? Lq - sq : 0) == 0;
    if (!empty) window_chunk<G>(a, unit, qbase, Lq, sq, un, obuf, red, m, l);
  } else {
    // sub-chunks of TW positions covering [S, sq); this workgroup's waves take
    // every (4 n_splits)-th one starting at 4 j + wave
    const int lo = g.S, hi = sq;
    const int c_first = lo / C::TW;
    const int c_end = hi > lo ? (hi + C::TW - 1) / C::TW : c_first;
    empty = c_first + 4 * j >= c_end;
    if (!empty) {
      uint32_t* qlds = un;
      float* part = (float*)(qlds + C::QLDS + 4 * C::WAVE);  // [4][G][D + 2]
      if (!C::QREG) {
        for (int x = tid; x < G * 16 * DIGP; x += 256)
          qlds[x] = ((const uint32_t*)(a.wsq + (int64_t)(qbase + x / (16 * DIGP)) * QS))
              [QOFF_LIMB + x % (16 * DIGP)];
        __syncthreads();
      }
      const int w = tid >> 6;
      float* pw = part + w * G * (D + 2);
      quant_wave<BITS, G>(a, unit, qbase, c_first + 4 * j + w, 4 * a.n_splits, c_end, lo, hi, qlds,
                          qlds + C::QLDS + w * C::WAVE, pw, pw + G * D, pw + G * D + G);
      __syncthreads();
      // merge the four wave partials (a wave without sub-chunks has l = 0)
      const int i = tid & (D - 1), hf = tid >> 7;
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float* px = part + x * G * (D + 2);
          if (px[G * D + G + gg] > 0.f) M = fmaxf(M, px[G * D + gg]);
        }
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float* px = part + x * G * (D + 2);
          const float f = px[G * D + G + gg] > 0.f ? exp2f(px[G * D + gg] - M) : 0.f;
          lsum = fmaf(px[G * D + G + gg], f, lsum);
          o = fmaf(px[gg * D + i], f, o);
        }
        if (hf == 0) obuf[gg * D + i] = o;
        m[gg] = M;
        l[gg] = lsum;
      }
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
}

// One workgroup per (sequence, query head): log-sum-exp merge of the chunk
// partials.  Thread = (4 dimensions, chunk residue mod 8).
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  __shared__ float scal[256];
  __shared__ __align__(16) float racc[8][D];
  __shared__ float red[64];
  const int jq = blockIdx.x, si = blockIdx.y, tid = threadIdx.x;
  const int nsp = a.n_splits + 1;
  const float* src = a.wsp + ((int64_t)si * a.g.n_q + jq) * nsp * PS;
  const int d4 = (tid & 31) * 4, rsd = tid >> 5;
  float M[1] = {-INFINITY};
  for (int x = tid; x < nsp; x += 256)
    if (src[x * PS + D + 1] > 0.f) M[0] = fmaxf(M[0], src[x * PS + D]);
  block_reduce<1, true>(M, red);
  float Ls[1] = {0.f};
  float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < nsp; c0 += 256) {
    __syncthreads();
    const int x = c0 + tid;
    float f = 0.f;
    if (x < nsp) {
      const float lx = src[x * PS + D + 1];
      f = lx > 0.f ? exp2f(src[x * PS + D] - M[0]) : 0.f;
      Ls[0] = fmaf(lx, f, Ls[0]);
    }
    scal[tid] = f;
    __syncthreads();
    const int n = nsp - c0 < 256 ? nsp - c0 : 256;
#pragma unroll 4
    for (int y = rsd; y < n; y += 8) {
      const float fy = scal[y];
      const float4 v = *(const float4*)(src + (int64_t)(c0 + y) * PS + d4);
      o4.x = fmaf(v.x, fy, o4.x);
      o4.y = fmaf(v.y, fy, o4.y);
      o4.z = fmaf(v.z, fy, o4.z);
      o4.w = fmaf(v.w, fy, o4.w);
    }
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
template <int BITS, int G>
hipError_t launch_split(DecodeArgs& a, hipStream_t st) {
  static int slots = 0;
  const size_t lds = (size_t)SplitCfg<BITS, G>::TOTAL * 4;
  if (slots == 0) {
    int dev = 0, cus = 0, per = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, split_kernel<BITS, G>, 256, lds);
    if (e != hipSuccess) return e;
    slots = cus * (per > 0 ? per : 1);
  }
  if (a.n_splits > 0) {
    const int units = a.n_seq * a.g.n_kv;
    int fill = (slots - units) / units;
    if (fill < 1) fill = 1;
    if (a.n_splits > fill) a.n_splits = fill;
  }
  dim3 gs(a.n_splits + 1, a.g.n_kv, a.n_seq);
  hipLaunchKernelGGL((split_kernel<BITS, G>), gs, dim3(256), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(DecodeArgs& a, int io_bf16, hipStream_t st, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
  dim3 gq(a.g.n_kv, a.n_seq);
  if (io_bf16) {
    if (a.g.bits == 2)
      hipLaunchKernelGGL((qcomp_kernel<1, 2>), gq, dim3(128), 0, st, a);
    else
      hipLaunchKernelGGL((qcomp_kernel<1, 4>), gq, dim3(128), 0, st, a);
  } else {
    if (a.g.bits == 2)
      hipLaunchKernelGGL((qcomp_kernel<0, 2>), gq, dim3(128), 0, st, a);
    else
      hipLaunchKernelGGL((qcomp_kernel<0, 4>), gq, dim3(128), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_start && (e = hipEventRecord(ev_start, st)) != hipSuccess) return e;
  const int G = a.g.G;
  if (a.g.bits == 2)
    e = G == 1 ? launch_split<2, 1>(a, st) : G == 2 ? launch_split<2, 2>(a, st)
      : G == 4 ? launch_split<2, 4>(a, st) : launch_split<2, 8>(a, st);
  else
    e = G == 1 ? launch_split<4, 1>(a, st) : G == 2 ? launch_split<4, 2>(a, st)
      : G == 4 ? launch_split<4, 4>(a, st) : launch_split<4, 8>(a, st);
  if (e != hipSuccess) return e;
  if (ev_stop && (e = hipEventRecord(ev_stop, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(a.g.n_q, a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace wkv
