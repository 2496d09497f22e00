// Device helpers shared by the gfx950 kernels: bf16 conversion, wave64
// cross-lane reductions, MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// One element of the readout o: float32 when the caller asked for float32
// outputs (o_f32), else rounded to the input type T.
template <typename T>
__device__ __forceinline__ void store_out(void *o, int64_t i, float x, int o_f32) {
  if (o_f32) static_cast<float *>(o)[i] = x;
  else static_cast<T *>(o)[i] = from_f32<T>(x);
}
// The same with the choice made at compile time (kernels that store inside a
// sequential loop take it as a template argument: no branch in the loop).
template <typename T, bool F32>
__device__ __forceinline__ void store_out_t(void *o, int64_t i, float x) {
  if constexpr (F32) static_cast<float *>(o)[i] = x;
  else static_cast<T *>(o)[i] = from_f32<T>(x);
}

// Sum over the 64 lanes of a wave; every lane receives the total.
// Rows of 16 lanes are reduced with DPP butterflies (xor 1, xor 2, half-row
// mirror, row mirror); rows are then combined with row broadcasts into lane
// 63, whose value is read back as a wave-uniform scalar.
__device__ __forceinline__ float wave_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)); // row_half_mirror
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)); // row_mirror
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0x142, 0xA, 0xF, false)); // row_bcast:15
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
           0, __builtin_bit_cast(int, x), 0x143, 0xC, 0xF, false)); // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Wave-uniform value (lets the compiler keep it in scalar registers).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace osdn
