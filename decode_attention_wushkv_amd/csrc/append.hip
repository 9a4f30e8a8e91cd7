// wushkv_append kernels: key transform, window placement, per-token
// percentile-clipped affine quantization and packing (WUSH-KV paper page,
// sections 4.2, 4.4, 5.3; appendix B.3 for the level grid).
//
// One workgroup of 128 threads handles one (sequence, KV head) and a run of
// positions; thread i owns dimension i of every entry it touches.
//
// Numerics: k'_i = sum_j T[i][j] k_j in fp64 (transform_entry in quant.h),
// rounded once to bfloat16 (RNE); the quantizer is in quant.h.
#include "quant.h"

namespace wkv {
namespace {

template <int IO_BF16>
__device__ __forceinline__ float load_io(const void* base, int64_t idx) {
  if (IO_BF16) return bf16_bits_to_f32(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

template <int IO_BF16>
__device__ __forceinline__ uint16_t io_to_bf16(const void* base, int64_t idx) {
  if (IO_BF16) return ((const uint16_t*)base)[idx];
  return f32_to_bf16(((const float*)base)[idx]);
}

template <int IO_BF16, bool B3>
__global__ __launch_bounds__(128) void append_kernel(AppendArgs a) {
  __shared__ QLds L;
  __shared__ float kvec[D];
  const int i = threadIdx.x;
  const int chunk = blockIdx.x;
  const int h = blockIdx.y;
  const int si = blockIdx.z;
  const Geometry& g = a.g;
  const int slot = a.s.slot[si];
  const int L0 = a.s.len0[si];
  const int n = a.s.n_new[si];
  const int L1 = L0 + n;
  const int64_t unit = ((int64_t)a.layer * g.max_batch + slot) * g.n_kv + h;
  const QMap qm = qmap_of(g, a.layer, slot, h);
  const int sq0 = squant_of(L0, g.S, g.R, g.F);
  const int sq1 = squant_of(L1, g.S, g.R, g.F);

  VRows vr;
  vrows_init(vr);

  // Entries already in the ring that leave the recent window.
  if (a.mode != APPEND_CHUNKED) {
    const int e1 = sq1 < L0 ? sq1 : L0;
    for (int p = sq0; p < e1; ++p) {
      const int64_t row = (unit * g.W + (p - g.S) % g.W) * D + i;
      float kx = bf16_bits_to_f32(a.pl.kring[row]);
      float vx = bf16_bits_to_f32(a.pl.vring[row]);
      store_quantized<B3>(p, kx, vx, L, vr, a.pl, qm, g);
    }
    if (a.mode == APPEND_EVICT) {
      vrows_flush<B3>(vr, a.pl);
      return;
    }
  }
  __syncthreads();  // all ring reads above complete before any ring write below

  int c0 = L0, c1 = L1;
  if (a.mode == APPEND_CHUNKED) {
    const int base = L0 - L0 % CHUNK;
    c0 = base + chunk * CHUNK;
    c1 = c0 + CHUNK;
    if (c0 < L0) c0 = L0;
    if (c1 > L1) c1 = L1;
  }
  if (c0 >= c1) {
    vrows_flush<B3>(vr, a.pl);
    return;
  }

  // Row i of this head's key transform, kept in registers.
  float trow[D];
  {
    const float4* tp = (const float4*)(a.tk + ((int64_t)h * D + i) * D);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      float4 t4 = tp[c];
      trow[4 * c + 0] = t4.x;
      trow[4 * c + 1] = t4.y;
      trow[4 * c + 2] = t4.z;
      trow[4 * c + 3] = t4.w;
    }
  }

  for (int p = c0; p < c1; ++p) {
    const int64_t row = ((int64_t)a.s.tok0[si] + (p - L0)) * g.n_kv + h;
    kvec[i] = load_io<IO_BF16>(a.k, row * D + i);
    const uint16_t vb = io_to_bf16<IO_BF16>(a.v, row * D + i);
    __syncthreads();
    const double acc = transform_entry([&](int j) { return trow[j]; }, [&](int j) { return kvec[j]; });
    const uint16_t kb = f64_to_bf16(acc);
    if (p < g.S) {
      const int64_t o = (unit * g.S + p) * D + i;
      a.pl.ksink[o] = kb;
      a.pl.vsink[o] = vb;
    } else if (p >= sq1) {
      const int64_t o = (unit * g.W + (p - g.S) % g.W) * D + i;
      a.pl.kring[o] = kb;
      a.pl.vring[o] = vb;
    } else {
      store_quantized<B3>(p, bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), L, vr, a.pl, qm, g);
    }
    __syncthreads();  // kvec reuse
  }
  vrows_flush<B3>(vr, a.pl);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int io_bf16, int grid_x, int n_seq, hipStream_t st) {
  dim3 grid(grid_x, a.g.n_kv, n_seq);
  const bool b3 = a.g.bits == 3;
  if (io_bf16 && b3)
    hipLaunchKernelGGL((append_kernel<1, true>), grid, dim3(128), 0, st, a);
  else if (io_bf16)
    hipLaunchKernelGGL((append_kernel<1, false>), grid, dim3(128), 0, st, a);
  else if (b3)
    hipLaunchKernelGGL((append_kernel<0, true>), grid, dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL((append_kernel<0, false>), grid, dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace wkv
