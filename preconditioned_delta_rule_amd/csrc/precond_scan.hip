// Phase 1 of OSDN: the online preconditioner sweep.
//
// Paper: "OSDN: Improving Delta Rule with Provable Online Preconditioning in
// Linear Attention", Section 4.2 (Eq.(4), Algorithm 1), Section 4.4 (Eq.(7),
// APF retention), Appendix B (non-beta-aware feedback).  Per (b,h) and token t:
//   emit k~_t = d (.) k_t, then
//   d <- clip(r_t d + eta b' (1 - b' <d, k_t^2>) / max(||k_t||^2, eps) k_t^2).
//
// Mapping: one wave64 per (b,h) sequence, d held in VGPRs (EPL coordinates
// per lane, contiguous so a token row is one coalesced load), the two K-long
// reductions per token done with DPP row butterflies plus row broadcasts.
// Keys of the next U tokens are loaded while the current U are processed.
#include "device_common.h"
#include "kernels.h"

namespace osdn {

template <typename TIn, int EPL> struct RowVec;
template <> struct RowVec<bf16, 1> { typedef bf16 type; };
template <> struct RowVec<bf16, 2> { typedef bf16x2 type; };
template <> struct RowVec<bf16, 4> { typedef bf16x4 type; };
template <> struct RowVec<float, 1> { typedef float type; };
template <> struct RowVec<float, 2> { typedef floatx2 type; };
template <> struct RowVec<float, 4> { typedef floatx4 type; };

template <typename TIn, int EPL, bool FULL>
__device__ __forceinline__ void load_row(const TIn *p, int lane, int64_t K, float (&x)[EPL]) {
  if constexpr (FULL) {
    typedef typename RowVec<TIn, EPL>::type V;
    V v = *reinterpret_cast<const V *>(p + lane * EPL);
    if constexpr (EPL == 1) {
      x[0] = to_f32(v);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = to_f32(v[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      int64_t c = (int64_t)lane * EPL + e;
      x[e] = c < K ? to_f32(p[c]) : 0.0f;
    }
  }
}

template <typename TIn, int EPL, bool FULL>
__device__ __forceinline__ void store_row(TIn *p, int lane, int64_t K, const float (&x)[EPL]) {
  if constexpr (FULL) {
    typedef typename RowVec<TIn, EPL>::type V;
    V v;
    if constexpr (EPL == 1) {
      v = from_f32<TIn>(x[0]);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[e] = from_f32<TIn>(x[e]);
    }
    *reinterpret_cast<V *>(p + lane * EPL) = v;
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      int64_t c = (int64_t)lane * EPL + e;
      if (c < K) p[c] = from_f32<TIn>(x[e]);
    }
  }
}

template <typename TIn, int EPL, bool FULL, bool HAS_R>
__global__ __launch_bounds__(64) void precond_scan_kernel(ScanArgs a) {
  constexpr int U = 8;  // tokens per prefetch group
  const int lane = threadIdx.x;
  const int64_t seq = blockIdx.x;  // (b,h), one wave each
  const int64_t H = a.H, T = a.T, K = a.K;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t tok0 = b * T * H + h;  // flat [B,T,H] index of token 0
  const int64_t stride = H * K;        // elements between consecutive tokens
  const TIn *kp = static_cast<const TIn *>(a.k) + tok0 * K;
  TIn *op = static_cast<TIn *>(a.k_tilde) + tok0 * K;
  const float *bp = a.beta + tok0;
  const float *rp = HAS_R ? a.r + tok0 : nullptr;

  float d[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    int64_t c = (int64_t)lane * EPL + e;
    d[e] = c < K ? (a.d1 ? a.d1[seq * K + c] : 1.0f) : 0.0f;
  }
  const float eta = a.eta, eps = a.eps, dmin = a.d_min, dmax = a.d_max;
  const bool clamp = a.clamp != 0, aware = a.beta_aware != 0;

  float kc[U][EPL], bc[U], rc[U];
  float kn[U][EPL], bn[U], rn[U];
  auto fetch = [&](int64_t t0, float (&kk)[U][EPL], float (&bb)[U], float (&rr)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t t = t0 + u;
      if (t < T) {
        load_row<TIn, EPL, FULL>(kp + t * stride, lane, K, kk[u]);
        bb[u] = bp[t * H];
        rr[u] = HAS_R ? rp[t * H] : 1.0f;
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kk[u][e] = 0.0f;
        bb[u] = 0.0f;
        rr[u] = 1.0f;
      }
    }
  };

  if (T > 0) fetch(0, kc, bc, rc);
  for (int64_t t0 = 0; t0 < T; t0 += U) {
    if (t0 + U < T) fetch(t0 + U, kn, bn, rn);
    const int nu = (int)((T - t0) < U ? (T - t0) : U);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < nu) {
        float w[EPL], s[EPL], pa = 0.0f, pn = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          w[e] = d[e] * kc[u][e];
          s[e] = kc[u][e] * kc[u][e];
          pn += s[e];
          pa += d[e] * s[e];
        }
        store_row<TIn, EPL, FULL>(op + (t0 + u) * stride, lane, K, w);
        const float norm = wave_sum(pn);
        const float align = wave_sum(pa);
        const float inv_n = 1.0f / fmaxf(norm, eps);
        const float bpr = aware ? bc[u] : 1.0f;
        const float c = eta * bpr * (1.0f - bpr * align) * inv_n;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float x = rc[u] * d[e] + c * s[e];
          if (clamp) x = fminf(fmaxf(x, dmin), dmax);
          d[e] = x;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bc[u] = bn[u];
      rc[u] = rn[u];
#pragma unroll
      for (int e = 0; e < EPL; ++e) kc[u][e] = kn[u][e];
    }
  }
  if (a.d_out) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      int64_t c = (int64_t)lane * EPL + e;
      if (c < K) a.d_out[seq * K + c] = d[e];
    }
  }
}

template <typename TIn, int EPL, bool FULL>
static hipError_t launch_epl(const ScanArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.H)), block(64);
  if (a.r)
    hipLaunchKernelGGL((precond_scan_kernel<TIn, EPL, FULL, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((precond_scan_kernel<TIn, EPL, FULL, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_typed(const ScanArgs &a, hipStream_t s) {
  if (a.K <= 64) return a.K == 64 ? launch_epl<TIn, 1, true>(a, s) : launch_epl<TIn, 1, false>(a, s);
  if (a.K <= 128) return a.K == 128 ? launch_epl<TIn, 2, true>(a, s) : launch_epl<TIn, 2, false>(a, s);
  return a.K == 256 ? launch_epl<TIn, 4, true>(a, s) : launch_epl<TIn, 4, false>(a, s);
}

hipError_t launch_precond_scan(const ScanArgs &a, bool is_bf16, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  return is_bf16 ? launch_typed<bf16>(a, s) : launch_typed<float>(a, s);
}

}  // namespace osdn
