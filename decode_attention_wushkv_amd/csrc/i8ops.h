// Cache codes as operands of the int8 matrix-core instruction
// v_mfma_i32_16x16x64_i8 (shared by the chunked-step kernel and the split
// kernel's grouped-query path).
//
// A lane holds 16 bytes of an operand, the K indices of its lane group (lane
// / 16).  The contraction does not care which K index is which as long as
// both operands agree, so each helper below fixes an order ("operand byte"
// of an element) that makes the unpacking cheap, and the producer of the
// other operand (query digits, softmax-weight digits) writes its bytes in
// the same order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

typedef int v4i __attribute__((ext_vector_type(4)));

// 16 two-bit codes (a 32-bit word, element m at bits 2 m) as 16 operand
// bytes: byte e holds element 4 (e % 4) + e / 4.
__device__ __forceinline__ v4i unpack2(uint32_t d) {
  v4i r;
  r[0] = (int)(d & 0x03030303u);
  r[1] = (int)((d >> 2) & 0x03030303u);
  r[2] = (int)((d >> 4) & 0x03030303u);
  r[3] = (int)((d >> 6) & 0x03030303u);
  return r;
}

// Operand byte of element m (0 <= m < 16) in the order of unpack2.
__device__ __forceinline__ int opnd_byte(int m) { return 4 * (m & 3) + (m >> 2); }

// 16 four-bit codes (two words, element j in nibble j % 8 of word j / 8) as
// operand bytes: byte 4 q + b holds element 8 (q / 2) + 2 b + q % 2.
__device__ __forceinline__ v4i unpack4(uint32_t d0, uint32_t d1) {
  v4i r;
  r[0] = (int)(d0 & 0x0F0F0F0Fu);
  r[1] = (int)((d0 >> 4) & 0x0F0F0F0Fu);
  r[2] = (int)(d1 & 0x0F0F0F0Fu);
  r[3] = (int)((d1 >> 4) & 0x0F0F0F0Fu);
  return r;
}

// Operand byte of element m in the order of unpack4.
__device__ __forceinline__ int opnd_byte4(int m) { return 4 * (2 * (m >> 3) + (m & 1)) + ((m & 7) >> 1); }

// 16 three-bit codes: the low two bits as unpack2 orders them, the high bits
// from a high-plane word in which element i sits at bit
// 4 (i / 2) + sh + i % 2 (sh = 0 or 2, the plane's order of a 16-element group).
__device__ __forceinline__ v4i unpack3(uint32_t lo, uint32_t hw, int sh) {
  v4i r = unpack2(lo);
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] |= (int)(((hw >> (4 * (q >> 1) + sh + (q & 1))) & 0x01010101u) << 2);
  return r;
}

template <int BITS>
__device__ __forceinline__ int opnd_byte_b(int m) { return BITS == 4 ? opnd_byte4(m) : opnd_byte(m); }

__device__ __forceinline__ v4i mfma8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace wkv
