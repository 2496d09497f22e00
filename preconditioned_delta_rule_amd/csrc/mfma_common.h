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

__device__ __forceinline__ bf16x4 pack4(floatx4 v) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = to_bf16(v[i]);
  return r;
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split4(floatx4 v, bf16x4 &hi, bf16x4 &lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = to_bf16(v[i]);
    lo[i] = to_bf16(v[i] - to_f32(hi[i]));
  }
}

}  // namespace osdn
