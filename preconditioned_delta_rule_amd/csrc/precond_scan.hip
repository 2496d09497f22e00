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
// Only <d, k^2> sits on the token-to-token dependency chain: the step is
// written c = a_t - b_t <d, k^2> with a_t = eta b'/n, b_t = eta b'^2/n computed
// from the key alone.  Besides (or instead of) k~ in the input dtype the
// sweep can emit the residual (d - 1) (.) k in bf16: k + residual carries k~ to
// about 16 significant bits (exactly when d sits on a bound) for the chunk
// pass, at the byte cost of a bf16 k~.  d is carried with a compensation term (d_true =
// d - comp) so its fp32 rounding does not drift over long sequences: each step
// forms r d exactly as p + ep with an FMA and adds c s + ep - r comp to p with
// a Fast2Sum.  Keys of the next group of tokens are loaded (as raw
// bf16/f32 words) while the current group is processed; beta and r arrive as
// one lane-indexed vector load per group and are broadcast with readlane.
// With vector retention (diag(r_t) in place of r_t, Proposition A.3 of the
// appendix) r_t is a [K] row per token, loaded and held like the keys.
#include "kernels.h"
#include "profile.h"
#include "scan_common.h"

namespace osdn {

template <typename TIn, int EPL, bool FULL, bool HAS_R, bool RV, bool WKT, bool WRES>
__global__ __launch_bounds__(64) void precond_scan_kernel(ScanArgs a) {
  constexpr int G = 32;  // tokens per prefetch group
  const int lane = threadIdx.x;
  const int64_t seq = blockIdx.x;  // (b,h), one wave each
  const int64_t H = a.H, T = a.T, K = a.K;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t tok0 = b * T * H + h;  // flat [B,T,H] index of token 0
  const int64_t stride = H * K;        // elements between consecutive tokens
  const TIn *kp = static_cast<const TIn *>(a.k) + tok0 * K;
  TIn *op = WKT ? static_cast<TIn *>(a.k_tilde) + tok0 * K : nullptr;
  bf16 *rp_out = WRES ? static_cast<bf16 *>(a.kt_res) + tok0 * K : nullptr;
  const float *bp = a.beta + tok0;
  const float *rp = HAS_R ? a.r + tok0 : nullptr;
  const float *rvp = RV ? a.r + tok0 * K : nullptr;  // [B,T,H,K] rows

  float d[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int64_t c = (int64_t)lane * EPL + e;
    d[e] = c < K ? (a.d1 ? a.d1[seq * K + c] : 1.0f) : 0.0f;
    // re-define d after its load so no later wait has to cover the d1 loads
    asm volatile("" : "+v"(d[e]));
  }
  float comp[EPL];  // rounding error carried with d: the exact value is d - comp
#pragma unroll
  for (int e = 0; e < EPL; ++e) comp[e] = 0.0f;
  const float eta = a.eta, eps = a.eps, dmin = a.d_min, dmax = a.d_max;
  const bool clamp = a.clamp != 0, aware = a.beta_aware != 0;

  // two key buffers used in turn (no register copies of in-flight loads)
  Row<TIn, EPL, FULL> kA[G], kB[G];
  Row<float, EPL, FULL> vA[RV ? G : 1], vB[RV ? G : 1];  // retention rows (vector form)
  float bA = 0.0f, rA = 1.0f, bB = 0.0f, rB = 1.0f;  // lane u holds token u of the group
  auto fetch = [&](int64_t t0, Row<TIn, EPL, FULL> (&kk)[G], Row<float, EPL, FULL> (&vv)[RV ? G : 1],
                   float &bb, float &rr) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int64_t t = t0 + u < T ? t0 + u : T - 1;  // stay in bounds; unused past T
      kk[u].load(kp + t * stride, lane, K);
      if constexpr (RV) vv[u].load(rvp + t * stride, lane, K);
    }
    const int64_t tl = t0 + (lane < G ? lane : 0);
    const int64_t tc = tl < T ? tl : T - 1;
    bb = bp[tc * H];
    rr = HAS_R ? rp[tc * H] : 1.0f;
  };
  auto step = [&](int64_t t, const Row<TIn, EPL, FULL> &kr, const Row<float, EPL, FULL> &rrow, float bt,
                  float rs) {
    float k[EPL], w[EPL], s[EPL], rt[EPL], pa = 0.0f, pn = 0.0f;
    kr.get(k);
    if constexpr (RV) {
      rrow.get(rt);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) rt[e] = rs;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      s[e] = k[e] * k[e];
      pn += s[e];
      pa += d[e] * s[e];
    }
    if constexpr (WKT) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) w[e] = fmaf(-comp[e], k[e], d[e] * k[e]);  // (d - comp) k
      store_row<TIn, EPL, FULL>(op + t * stride, lane, K, w);
    }
    if constexpr (WRES) {
      float rres[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) rres[e] = ((d[e] - 1.0f) - comp[e]) * k[e];  // d - 1 is exact on [0.5, 2]
      store_row<bf16, EPL, FULL>(rp_out + t * stride, lane, K, rres);
    }
    // off the chain: step coefficients from the key and gates alone
    const float norm = wave_sum(pn);
    const float bpr = aware ? bt : 1.0f;
    const float ea = eta * bpr / fmaxf(norm, eps);  // c = ea - eb * <d, s>
    const float eb = ea * bpr;
    float p[EPL], q[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      p[e] = rt[e] * d[e];                                          // r d = p + ep exactly
      q[e] = fmaf(-rt[e], comp[e], fmaf(rt[e], d[e], -p[e]));       // ep - r comp
    }
    // on the chain
    const float align = wave_sum(pa);
    const float c = fmaf(-eb, align, ea);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float y = fmaf(c, s[e], q[e]);
      const float t = p[e] + y;
      float cn = (t - p[e]) - y;  // Fast2Sum error (|p| >= |y|)
      float x = t;
      if (clamp) {
        x = fminf(fmaxf(t, dmin), dmax);
        cn = x == t ? cn : 0.0f;  // a clamped coordinate is exact
      }
      d[e] = x;
      comp[e] = cn;
    }
  };
  auto process = [&](int64_t t0, const Row<TIn, EPL, FULL> (&kk)[G], const Row<float, EPL, FULL> (&vv)[RV ? G : 1],
                     float bv, float rv) {
    if (t0 + G <= T) {
      // full group: straight-line code, so load waits stay per token
#pragma unroll
      for (int u = 0; u < G; ++u) step(t0 + u, kk[u], vv[RV ? u : 0], lane_bcast(bv, u), lane_bcast(rv, u));
    } else {
      const int nu = (int)(T - t0);
#pragma unroll
      for (int u = 0; u < G; ++u)
        if (u < nu) step(t0 + u, kk[u], vv[RV ? u : 0], lane_bcast(bv, u), lane_bcast(rv, u));
    }
  };

  // Fetches are unconditional (addresses clamped to the last token) so the
  // code between them is straight-line and every load wait stays exact.
  if (T > 0) fetch(0, kA, vA, bA, rA);
  for (int64_t t0 = 0; t0 < T; t0 += 2 * G) {
    fetch(t0 + G, kB, vB, bB, rB);
    process(t0, kA, vA, bA, rA);
    if (t0 + G >= T) break;
    fetch(t0 + 2 * G, kA, vA, bA, rA);
    process(t0 + G, kB, vB, bB, rB);
  }
  if (a.d_out) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int64_t c = (int64_t)lane * EPL + e;
      if (c < K) a.d_out[seq * K + c] = d[e];
    }
  }
}

template <typename TIn, int EPL, bool FULL, bool HAS_R, bool RV>
static void launch_out(const ScanArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.H)), block(64);
  if (a.k_tilde && a.kt_res)
    hipLaunchKernelGGL((precond_scan_kernel<TIn, EPL, FULL, HAS_R, RV, true, true>), grid, block, 0, s, a);
  else if (a.kt_res)
    hipLaunchKernelGGL((precond_scan_kernel<TIn, EPL, FULL, HAS_R, RV, false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((precond_scan_kernel<TIn, EPL, FULL, HAS_R, RV, true, false>), grid, block, 0, s, a);
  prof_mark(s, "precond_scan_kernel");
}

template <typename TIn, int EPL, bool FULL>
static hipError_t launch_epl(const ScanArgs &a, hipStream_t s) {
  if (a.r && a.r_per_key)
    launch_out<TIn, EPL, FULL, false, true>(a, s);
  else if (a.r)
    launch_out<TIn, EPL, FULL, true, false>(a, s);
  else
    launch_out<TIn, EPL, FULL, false, false>(a, s);
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
