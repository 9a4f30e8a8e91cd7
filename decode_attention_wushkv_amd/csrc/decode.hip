// wushkv_decode_attn kernels: GQA decode attention over the mixed cache
// (WUSH-KV paper page: section 4.1 for the cache and GQA head sharing,
// section 4.2 / appendix B.1 for the T_K^{-T} query compensation, section
// 4.4 for the full-precision windows, appendix D.1 for the 1/sqrt(d) scale).
//
// Three launches per call:
//   qcomp    q' = T_K^{-T} q per query head, prescaled by log2(e)/sqrt(d), and
//            sigma = sum_i q'_i (the zero point factors out of the score:
//            q'.(z + s c) = z sigma + s (q'.c)).
//   split    one workgroup per (sequence, KV head, 1024-position chunk of the
//            quantized region), plus one per (sequence, KV head) for the
//            bfloat16 sink + recent entries.  Pass 1 scores every position
//            of the chunk for the G query heads of the KV head, pass 2 turns
//            them into exp2 weights against the chunk max, pass 3 streams the
//            dim-major value codes: o_i = sum_t (p_t s_t) c_{t,i} +
//            sum_t p_t z_t.  Emits (o, m, l) per query head and chunk.
//   combine  log-sum-exp merge of the chunk partials into fp32 output.
#include "common.h"

namespace wkv {
namespace {

constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

template <int IO_BF16>
__device__ __forceinline__ float load_io(const void* base, int64_t idx) {
  if (IO_BF16) return bf16_to_f32(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// ---------------------------------------------------------------- qcomp

template <int IO_BF16>
__global__ __launch_bounds__(128) void qcomp_kernel(DecodeArgs a) {
  __shared__ float qv[8][D];
  __shared__ float red[8][2];
  const int h = blockIdx.x, si = blockIdx.y, i = threadIdx.x;
  const int G = a.g.G, nq = a.g.n_q;
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
    float* dst = a.wsq + ((int64_t)si * nq + h * G + g) * QS;
    dst[i] = acc;
    float s = wave_sum(acc);
    if ((i & 63) == 0) red[g][i >> 6] = s;
  }
  __syncthreads();
  if (i < G) a.wsq[((int64_t)si * nq + h * G + i) * QS + D] = red[i][0] + red[i][1];
}

// ---------------------------------------------------------------- split

struct SplitShared {
  float* qs;   // [G][D]
  float* sig;  // [8]
  float* sc;   // [G][SPLIT_LEN] scores, then weights
  float* vs;   // [SPLIT_LEN] value scale
  float* vz;   // [SPLIT_LEN] value zero
  float* red;  // [8 * 4 * 2] reductions + [G][D] pass-3 halves
};

__host__ __device__ inline size_t split_lds_floats(int G) {
  return (size_t)G * D + 8 + (size_t)G * SPLIT_LEN + 2 * SPLIT_LEN + 64 + (size_t)G * D;
}

// Block-wide (256 threads) max and sum helpers over per-thread partials.
__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <int BITS, int G>
__global__ __launch_bounds__(256) void split_kernel(DecodeArgs a) {
  extern __shared__ float dyn[];
  const Geometry& g = a.g;
  SplitShared sh;
  sh.qs = dyn;
  sh.sig = sh.qs + G * D;
  sh.sc = sh.sig + 8;
  sh.vs = sh.sc + G * SPLIT_LEN;
  sh.vz = sh.vs + SPLIT_LEN;
  sh.red = sh.vz + SPLIT_LEN;
  float* half_o = sh.red + 64;

  const int j = blockIdx.x, h = blockIdx.y, si = blockIdx.z;
  const int tid = threadIdx.x;
  const int slot = a.s.slot[si], Lq = a.s.len[si], sq = a.s.squant[si];
  const int64_t unit = ((int64_t)a.layer * g.max_batch + slot) * g.n_kv + h;
  const bool window = (j == a.max_splits);

  int t0 = 0, t1 = 0, ns = 0, ntok;
  if (window) {
    ns = Lq < g.S ? Lq : g.S;
    ntok = ns + (Lq > sq ? Lq - sq : 0);
  } else {
    t0 = j * SPLIT_LEN;
    if (t0 < g.S) t0 = g.S;
    t1 = (j + 1) * SPLIT_LEN;
    if (t1 > sq) t1 = sq;
    ntok = t1 - t0;
  }
  if (ntok <= 0) return;

  // Compensated queries of the G query heads of this KV head.
  const int qbase = si * g.n_q + h * G;
  for (int x = tid; x < G * D; x += 256) sh.qs[x] = a.wsq[(int64_t)(qbase + x / D) * QS + (x % D)];
  if (tid < G) sh.sig[tid] = a.wsq[(int64_t)(qbase + tid) * QS + D];
  __syncthreads();

  // ---- pass 1: scores (log2 domain), two lanes per position.
  const int half = tid & 1;
  for (int tok = tid >> 1; tok < ntok; tok += 128) {
    float dot[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) dot[gg] = 0.f;
    const float* q0 = sh.qs + half * 64;
    float ks = 1.f, kz = 0.f;
    if (window) {
      const int p = tok < ns ? tok : sq + (tok - ns);
      const uint16_t* src = tok < ns ? a.pl.ksink + (unit * g.S + p) * D
                                     : a.pl.kring + (unit * g.W + (p - g.S) % g.W) * D;
      const uint4* s4 = (const uint4*)(src + half * 64);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint4 w = s4[c];
        uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float x = bf16_to_f32((uint16_t)(ww[e >> 1] >> ((e & 1) * 16)));
          for (int gg = 0; gg < G; ++gg) dot[gg] = fmaf(q0[gg * D + c * 8 + e], x, dot[gg]);
        }
      }
    } else {
      const int p = t0 + tok;
      const uint32_t kszv = a.pl.ksz[unit * g.cpos + p];
      ks = f16_to_f32(kszv & 0xFFFFu);
      kz = f16_to_f32(kszv >> 16);
      const uint4* s4 = (const uint4*)(a.pl.kcode + (unit * g.cpos + p) * g.code_bytes +
                                       half * (g.code_bytes / 2));
      constexpr int NW = BITS == 2 ? 4 : 8;  // 32-bit words per half
      constexpr int PER = 32 / BITS;          // codes per word
      uint32_t ww[NW];
#pragma unroll
      for (int c = 0; c < NW / 4; ++c) {
        uint4 w = s4[c];
        ww[4 * c] = w.x;
        ww[4 * c + 1] = w.y;
        ww[4 * c + 2] = w.z;
        ww[4 * c + 3] = w.w;
      }
#pragma unroll
      for (int w = 0; w < NW; ++w) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          float x = (float)((ww[w] >> (e * BITS)) & ((1u << BITS) - 1u));
          for (int gg = 0; gg < G; ++gg) dot[gg] = fmaf(q0[gg * D + w * PER + e], x, dot[gg]);
        }
      }
      if (half) {
        const uint32_t vszv = a.pl.vsz[unit * g.cpos + p];
        sh.vs[tok] = f16_to_f32(vszv & 0xFFFFu);
        sh.vz[tok] = f16_to_f32(vszv >> 16);
      }
    }
    for (int gg = 0; gg < G; ++gg) {
      float d2 = dot[gg] + __shfl_xor(dot[gg], 1);
      if (!half) sh.sc[gg * SPLIT_LEN + tok] = ks * d2 + kz * sh.sig[gg];
    }
  }
  __syncthreads();

  // ---- pass 2: exp2 weights against the chunk max.
  float mg[G], lg[G], zg[G];
  for (int gg = 0; gg < G; ++gg) {
    float* sc = sh.sc + gg * SPLIT_LEN;
    float m = -INFINITY;
    for (int t = tid; t < ntok; t += 256) m = fmaxf(m, sc[t]);
    m = block_max(m, sh.red);
    float l = 0.f, z = 0.f;
    for (int t = tid; t < ntok; t += 256) {
      float pw = exp2f(sc[t] - m);
      l += pw;
      if (window) {
        sc[t] = pw;
      } else {
        z = fmaf(pw, sh.vz[t], z);
        sc[t] = pw * sh.vs[t];
      }
    }
    l = block_sum(l, sh.red);
    z = block_sum(z, sh.red);
    mg[gg] = m;
    lg[gg] = l;
    zg[gg] = z;
  }
  __syncthreads();

  // ---- pass 3: o_i = sum_t w_t v_{t,i}; lane = dimension, two position groups.
  const int i = tid & (D - 1), grp = tid >> 7;
  float acc[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) acc[gg] = 0.f;
  if (window) {
    for (int tok = grp; tok < ntok; tok += 2) {
      const int p = tok < ns ? tok : sq + (tok - ns);
      const uint16_t* src = tok < ns ? a.pl.vsink + (unit * g.S + p) * D
                                     : a.pl.vring + (unit * g.W + (p - g.S) % g.W) * D;
      float x = bf16_to_f32(src[i]);
      for (int gg = 0; gg < G; ++gg) acc[gg] = fmaf(sh.sc[gg * SPLIT_LEN + tok], x, acc[gg]);
    }
  } else {
    const int VB = 128 / BITS;
    const int bfirst = t0 / VB, blast = (t1 - 1) / VB;
    for (int b = bfirst + grp; b <= blast; b += 2) {
      const uint4 r = *(const uint4*)(a.pl.vcode + ((unit * g.ctx_blocks + b) * D + i) * 16);
      const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
      const int pb = b * VB;
#pragma unroll 4
      for (int u = 0; u < VB; ++u) {
        const int p = pb + u;
        if (p < t0 || p >= t1) continue;
        const int bit = u * BITS;
        float x = (float)((rw[bit >> 5] >> (bit & 31)) & ((1u << BITS) - 1u));
        for (int gg = 0; gg < G; ++gg) acc[gg] = fmaf(sh.sc[gg * SPLIT_LEN + (p - t0)], x, acc[gg]);
      }
    }
  }
  if (grp == 1)
    for (int gg = 0; gg < G; ++gg) half_o[gg * D + i] = acc[gg];
  __syncthreads();
  if (grp == 0) {
    for (int gg = 0; gg < G; ++gg) {
      float o = acc[gg] + half_o[gg * D + i] + zg[gg];
      float* dst = a.wsp + (((int64_t)(qbase + gg)) * (a.max_splits + 1) + j) * PS;
      dst[i] = o;
      if (i == 0) {
        dst[D] = mg[gg];
        dst[D + 1] = lg[gg];
      }
    }
  }
}

// ---------------------------------------------------------------- combine

__global__ __launch_bounds__(128) void combine_kernel(DecodeArgs a) {
  const int jq = blockIdx.x, si = blockIdx.y, i = threadIdx.x;
  const Geometry& g = a.g;
  const int Lq = a.s.len[si], sq = a.s.squant[si];
  const int nsplit = a.max_splits + 1;
  const float* base = a.wsp + ((int64_t)si * g.n_q + jq) * nsplit * PS;
  auto valid = [&](int j) -> bool {
    if (j == a.max_splits) {
      int ns = Lq < g.S ? Lq : g.S;
      return ns + (Lq > sq ? Lq - sq : 0) > 0;
    }
    int t0 = j * SPLIT_LEN;
    if (t0 < g.S) t0 = g.S;
    int t1 = (j + 1) * SPLIT_LEN;
    if (t1 > sq) t1 = sq;
    return t1 > t0;
  };
  float M = -INFINITY;
  for (int j = 0; j < nsplit; ++j)
    if (valid(j)) M = fmaxf(M, base[j * PS + D]);
  float l = 0.f, o = 0.f;
  for (int j = 0; j < nsplit; ++j) {
    if (!valid(j)) continue;
    float sc = exp2f(base[j * PS + D] - M);
    l = fmaf(base[j * PS + D + 1], sc, l);
    o = fmaf(base[j * PS + i], sc, o);
  }
  a.out[((int64_t)si * g.n_q + jq) * D + i] = o / l;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int io_bf16, hipStream_t st, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
  dim3 gq(a.g.n_kv, a.n_seq);
  if (io_bf16)
    hipLaunchKernelGGL(qcomp_kernel<1>, gq, dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL(qcomp_kernel<0>, gq, dim3(128), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 gs(a.max_splits + 1, a.g.n_kv, a.n_seq);
  size_t lds = split_lds_floats(a.g.G) * sizeof(float);
  if (ev_start && (e = hipEventRecord(ev_start, st)) != hipSuccess) return e;
#define WKV_SPLIT(B, GG) hipLaunchKernelGGL((split_kernel<B, GG>), gs, dim3(256), lds, st, a)
  if (a.g.bits == 2) {
    switch (a.g.G) {
      case 1: WKV_SPLIT(2, 1); break;
      case 2: WKV_SPLIT(2, 2); break;
      case 4: WKV_SPLIT(2, 4); break;
      default: WKV_SPLIT(2, 8); break;
    }
  } else {
    switch (a.g.G) {
      case 1: WKV_SPLIT(4, 1); break;
      case 2: WKV_SPLIT(4, 2); break;
      case 4: WKV_SPLIT(4, 4); break;
      default: WKV_SPLIT(4, 8); break;
    }
  }
#undef WKV_SPLIT
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_stop && (e = hipEventRecord(ev_stop, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(a.g.n_q, a.n_seq), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace wkv
