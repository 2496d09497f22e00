// MFMA helpers shared by the phase-2 kernels (gfx950, bf16 operands, fp32
// accumulation).  Operand layouts of v_mfma_f32_16x16x32_bf16 for lane l:
// A[m = l & 15][k = 8 (l >> 4) + e], B[k = 8 (l >> 4) + e][n = l & 15], e < 8;
// result D[m = 4 (l >> 4) + i][n = l & 15], i < 4.  The 16x16x16 form takes
// 4 consecutive k per lane (k = 4 (l >> 4) + e), so its result tile is laid
// out exactly like its own B operand.
#pragma once

#include "device_common.h"

namespace osdn {

__device__ __forceinline__ floatx4 mfma32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(bf16x4 a, bf16x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ bf16x4 ld4(const bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }

// two floats to a bf16 pair (v_cvt_pk_bf16_f32, round to nearest even);
// element 0 in the low half
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2{to_bf16(a), to_bf16(b)});
}
// the fp32 values of the two halves of a bf16 pair
__device__ __forceinline__ float pk_lo(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float pk_hi(uint32_t p) { return __builtin_bit_cast(float, p & 0xffff0000u); }

__device__ __forceinline__ bf16x4 pack4(floatx4 v) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(bf16x4, u2{pk2(v[0], v[1]), pk2(v[2], v[3])});
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split4(floatx4 v, bf16x4 &hi, bf16x4 &lo) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  uint32_t h0 = pk2(v[0], v[1]), h1 = pk2(v[2], v[3]);
  // keeps the compiler from converting element 0 a second time to unpack it
  asm("" : "+v"(h0), "+v"(h1));
  const uint32_t l0 = pk2(v[0] - pk_lo(h0), v[1] - pk_hi(h0));
  const uint32_t l1 = pk2(v[2] - pk_lo(h1), v[3] - pk_hi(h1));
  hi = __builtin_bit_cast(bf16x4, u2{h0, h1});
  lo = __builtin_bit_cast(bf16x4, u2{l0, l1});
}

}  // namespace osdn
