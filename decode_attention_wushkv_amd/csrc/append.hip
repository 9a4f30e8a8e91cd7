// wushkv_append kernels: key transform, window placement, per-token
// percentile-clipped affine quantization and packing (WUSH-KV paper page,
// sections 4.2, 4.4, 5.3; appendix B.3 for the level grid).
//
// One workgroup of 128 threads handles one (sequence, KV head) and a run of
// positions; thread i owns dimension i of every entry it touches.
//
// Numerics (chosen so that every integer decision matches an fp64 evaluation
// of the method's definitions):
//   * k'_i = sum_j T[i][j] k_j accumulated with fp64 FMAs (fp32 T, fp32/bf16
//     k: every product is exact in fp64), rounded once to bfloat16 (RNE).
//   * Order statistics come from an exact rank sort of the 128 bfloat16
//     values; the linear-interpolation percentile, the scale (hi-lo)/(2^b-1),
//     its binary16 rounding and the code coordinate (x - z16)/s16 are fp64
//     with no fused multiply-add, rounded half to even.
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
__device__ uint16_t f64_to_bf16(double x) {
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
__device__ uint16_t f64_to_f16_sat(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000);
  int ef = (int)((b >> 52) & 0x7FF);
  uint64_t mant = b & 0xFFFFFFFFFFFFFull;
  if (ef == 0x7FF) return mant ? (uint16_t)0x7E00 : (uint16_t)(sign | 0x7BFF);
  if (ef == 0) return sign;
  int e = ef - 1023;
  uint64_t m = mant | (1ull << 52);
  if (e >= -14) {
    uint64_t r = shift_rne(m, 42);  // keep 11 significant bits
    if (r == 2048) { r = 1024; e += 1; }
    if (e > 15) return sign | 0x7BFF;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r & 0x3FF);
  }
  int s = 28 - e;  // value in units of 2^-24 is m * 2^(e - 28)
  if (s > 63) return sign;
  return sign | (uint16_t)shift_rne(m, s);  // r <= 1024; 1024 encodes 2^-14
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------- quantizer

struct Lds {
  float vals[D];
  float sorted[D];
  float kvec[D];
  int codes[D];
};

// Linear-interpolation percentile of the sorted group (fp64, no FMA).
__device__ double percentile_sorted(const float* sorted, double p) {
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

// Quantize the group whose element threadIdx.x is x.  Returns this thread's
// code; *sz gets {s16 | z16 << 16}.  Block-uniform call (uses barriers).
__device__ int quantize_group(float x, Lds& L, double p_lo, double p_hi, int bits, uint32_t* sz) {
#pragma clang fp contract(off)
  const int i = threadIdx.x;
  L.vals[i] = x;
  __syncthreads();
  int rank = 0;
#pragma unroll 8
  for (int j = 0; j < D; ++j) {
    float y = L.vals[j];
    rank += (y < x) || (y == x && j < i);
  }
  L.sorted[rank] = x;
  __syncthreads();
  const double lo = percentile_sorted(L.sorted, p_lo);
  const double hi = percentile_sorted(L.sorted, p_hi);
  const double levels = (double)((1 << bits) - 1);
  const double s = (hi - lo) / levels;
  const uint16_t s16 = f64_to_f16_sat(s);
  const uint16_t z16 = f64_to_f16_sat(lo);
  const double sd = f16_bits_to_f64(s16);
  const double zd = f16_bits_to_f64(z16);
  int c = 0;
  if (sd != 0.0) {
    double u = ((double)x - zd) / sd;
    double r = rint(u);
    r = r < 0.0 ? 0.0 : r;
    r = r > levels ? levels : r;
    c = (int)r;
  }
  *sz = (uint32_t)s16 | ((uint32_t)z16 << 16);
  __syncthreads();  // vals / sorted may be reused by the next call
  return c;
}

// Accumulates value-code bits of one dimension row for consecutive positions
// and writes each 16-byte row once (read-modify-write keeps other positions).
struct VRow {
  int blk;
  uint32_t buf[4];
  uint32_t msk[4];
};

__device__ __forceinline__ void vrow_flush(VRow& r, const Planes& pl, int64_t unit, const Geometry& g) {
  if (r.blk < 0) return;
  uint4* p = (uint4*)(pl.vcode + ((unit * g.ctx_blocks + r.blk) * D + threadIdx.x) * 16);
  uint4 old = *p;
  old.x = (old.x & ~r.msk[0]) | r.buf[0];
  old.y = (old.y & ~r.msk[1]) | r.buf[1];
  old.z = (old.z & ~r.msk[2]) | r.buf[2];
  old.w = (old.w & ~r.msk[3]) | r.buf[3];
  *p = old;
  r.blk = -1;
}

__device__ __forceinline__ void vrow_add(VRow& r, int p, int code, const Planes& pl, int64_t unit,
                                         const Geometry& g) {
  int blk = p / g.vblock;
  if (blk != r.blk) {
    vrow_flush(r, pl, unit, g);
    r.blk = blk;
#pragma unroll
    for (int w = 0; w < 4; ++w) r.buf[w] = r.msk[w] = 0u;
  }
  int bit = (p % g.vblock) * g.bits;
  uint32_t m = (1u << g.bits) - 1u;
  r.buf[bit >> 5] |= (uint32_t)code << (bit & 31);
  r.msk[bit >> 5] |= m << (bit & 31);
}

// Quantize key and value entries (bfloat16 values kx, vx of this thread's
// dimension) of position p and store codes and scale/zero.
__device__ void store_quantized(int p, float kx, float vx, Lds& L, VRow& vr, const Planes& pl,
                                int64_t unit, const Geometry& g) {
  const int i = threadIdx.x;
  uint32_t ksz, vsz;
  int kc = quantize_group(kx, L, g.p_lo, g.p_hi, g.bits, &ksz);
  int vc = quantize_group(vx, L, g.p_lo, g.p_hi, g.bits, &vsz);
  L.codes[i] = kc;
  __syncthreads();
  const int words = g.code_bytes / 4;  // 8 (2-bit) or 16 (4-bit)
  if (i < words) {
    const int per = 32 / g.bits;
    uint32_t w = 0;
    for (int e = 0; e < per; ++e) w |= (uint32_t)L.codes[i * per + e] << (e * g.bits);
    ((uint32_t*)(pl.kcode + (unit * g.cpos + p) * g.code_bytes))[i] = w;
  }
  if (i == 0) {
    pl.ksz[unit * g.cpos + p] = ksz;
    pl.vsz[unit * g.cpos + p] = vsz;
  }
  vrow_add(vr, p, vc, pl, unit, g);
  __syncthreads();  // codes[] reuse
}

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

template <int IO_BF16>
__global__ __launch_bounds__(128) void append_kernel(AppendArgs a) {
  __shared__ Lds L;
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
  const int sq0 = squant_of(L0, g.S, g.R, g.F);
  const int sq1 = squant_of(L1, g.S, g.R, g.F);

  VRow vr;
  vr.blk = -1;

  // Entries already in the ring that leave the recent window.
  if (a.mode != APPEND_CHUNKED) {
    const int e1 = sq1 < L0 ? sq1 : L0;
    for (int p = sq0; p < e1; ++p) {
      const int64_t row = (unit * g.W + (p - g.S) % g.W) * D + i;
      float kx = bf16_bits_to_f32(a.pl.kring[row]);
      float vx = bf16_bits_to_f32(a.pl.vring[row]);
      store_quantized(p, kx, vx, L, vr, a.pl, unit, g);
    }
    if (a.mode == APPEND_EVICT) {
      vrow_flush(vr, a.pl, unit, g);
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
    vrow_flush(vr, a.pl, unit, g);
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
    L.kvec[i] = load_io<IO_BF16>(a.k, row * D + i);
    const uint16_t vb = io_to_bf16<IO_BF16>(a.v, row * D + i);
    __syncthreads();
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < D; ++j) acc = fma((double)trow[j], (double)L.kvec[j], acc);
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
      store_quantized(p, bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), L, vr, a.pl, unit, g);
    }
    __syncthreads();  // kvec reuse
  }
  vrow_flush(vr, a.pl, unit, g);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int io_bf16, int grid_x, int n_seq, hipStream_t st) {
  dim3 grid(grid_x, a.g.n_kv, n_seq);
  if (io_bf16)
    hipLaunchKernelGGL(append_kernel<1>, grid, dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL(append_kernel<0>, grid, dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace wkv
