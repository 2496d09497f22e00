// Helpers shared by the phase-1 kernels: per-lane token rows (EPL contiguous
// coordinates per lane), stores, lane broadcasts and a wave-wide transposed
// reduction.
#pragma once

#include "device_common.h"

namespace osdn {

template <typename TIn, int EPL> struct RowVec;
template <> struct RowVec<bf16, 1> { typedef bf16 type; };
template <> struct RowVec<bf16, 2> { typedef bf16x2 type; };
template <> struct RowVec<bf16, 4> { typedef bf16x4 type; };
template <> struct RowVec<float, 1> { typedef float type; };
template <> struct RowVec<float, 2> { typedef floatx2 type; };
template <> struct RowVec<float, 4> { typedef floatx4 type; };

// One token row of a lane: EPL elements kept as raw 32-bit words until used,
// so the compiler cannot hoist their conversion up to the (prefetch) load.
template <typename TIn, int EPL, bool FULL> struct Row {
  static constexpr int BYTES = EPL * (int)sizeof(TIn);
  static constexpr int WORDS = BYTES < 4 ? 1 : BYTES / 4;
  uint32_t w[WORDS];
  __device__ __forceinline__ void load(const TIn *p, int lane, int64_t K) {
    TIn x[EPL];
    if constexpr (FULL) {
      typedef typename RowVec<TIn, EPL>::type V;
      V v = *reinterpret_cast<const V *>(p + lane * EPL);
      if constexpr (EPL == 1) {
        x[0] = v;
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = v[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int64_t c = (int64_t)lane * EPL + e;
        x[e] = c < K ? p[c] : TIn(0.0f);
      }
    }
#pragma unroll
    for (int i = 0; i < WORDS; ++i) w[i] = 0;
    __builtin_memcpy(w, x, BYTES);
  }
  // Values as fp32, materialised at the point of use.
  __device__ __forceinline__ void get(float (&out)[EPL]) const {
    uint32_t t[WORDS];
#pragma unroll
    for (int i = 0; i < WORDS; ++i) {
      t[i] = w[i];
      asm volatile("" : "+v"(t[i]));
    }
    TIn x[EPL];
    __builtin_memcpy(x, t, BYTES);
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = to_f32(x[e]);
  }
};

template <typename TOut, int EPL, bool FULL>
__device__ __forceinline__ void store_row(TOut *p, int lane, int64_t K, const float (&x)[EPL]) {
  if constexpr (FULL) {
    typedef typename RowVec<TOut, EPL>::type V;
    V v;
    if constexpr (EPL == 1) {
      v = from_f32<TOut>(x[0]);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[e] = from_f32<TOut>(x[e]);
    }
    *reinterpret_cast<V *>(p + lane * EPL) = v;
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int64_t c = (int64_t)lane * EPL + e;
      if (c < K) p[c] = from_f32<TOut>(x[e]);
    }
  }
}

__device__ __forceinline__ float lane_bcast(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// Transposed reduction over the 64 lanes of a one-wave workgroup (the only
// kind that calls it; the exchange is ordered with wave_lds_sync): on entry
// every lane holds 64 partial values v[0..63]; on return lane l holds the
// combination over all lanes of entry l.  The transpose goes through LDS
// (buf: RS_PITCH * 64 floats): lane l writes its entries to row l, then
// reads column l.  With a row pitch of 65 words both the row writes and the
// column reads touch 64 distinct banks.  (Lane permutes would need a chain of
// dependent exchanges; here the 64 writes and the 64 reads each pipeline.)
constexpr int RS_PITCH = 65;

// Orders the LDS accesses of a one-wave workgroup around a cross-lane
// exchange.  The LDS unit executes one wave's operations in order, so only
// the compiler has to be kept from moving them; unlike __syncthreads this
// does not also wait for the wave's outstanding global loads.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

template <bool MAX>
__device__ __forceinline__ float reduce_scatter64(const float (&v)[64], int lane, float *buf) {
  wave_lds_sync();  // earlier readers of buf are done
#pragma unroll
  for (int j = 0; j < 64; ++j) buf[lane * RS_PITCH + j] = v[j];
  wave_lds_sync();
  float acc = buf[lane];
#pragma unroll
  for (int u = 1; u < 64; ++u) {
    const float x = buf[u * RS_PITCH + lane];
    acc = MAX ? fmaxf(acc, x) : acc + x;
  }
  wave_lds_sync();  // buf may be reused at once
  return acc;
}

}  // namespace osdn
