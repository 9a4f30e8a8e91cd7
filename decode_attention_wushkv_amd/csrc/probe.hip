// Streaming-read reference kernel (instrumentation, not part of the method):
// reads a buffer once with 16-byte loads in a grid-stride loop, four loads in
// flight per thread, and folds it into one word per thread so the loads are
// not dead.  Its bandwidth is the practical read ceiling that the decode
// kernels are compared with.
#include "common.h"

namespace wkv {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, uint64_t n,
                                                          uint32_t* out) {
  uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, uint64_t bytes, int blocks, void* out,
                              hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, st, (const uint4*)buf,
                     bytes / 16, (uint32_t*)out);
  return hipGetLastError();
}

}  // namespace wkv
