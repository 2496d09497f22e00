// Decode step of OSDN: a few new tokens through the recurrent form, carrying
// the state (S, d) from a previous call.
//
// Paper: "OSDN: Improving Delta Rule with Provable Online Preconditioning in
// Linear Attention", Appendix L (the fused single-token recurrence used at
// decode time, one launch per call), with the preconditioner step of Section
// 4.2 Eq.(4) / Section 4.4 Eq.(7) and the write of Section 4.3 Eq.(5), gated
// as in Appendix B.1.  Per (b,h) and token t, from the carried (S, d):
//   k~ = d (.) k_t   (before the update), then
//   d  = clip(r_t d + eta b' (1 - b' <d, k_t^2>) / max(|k_t|^2, eps) k_t^2)
//   Sb = alpha_t S;  S = Sb + beta_t (v_t - Sb k_t) k~^T;  o_t = S (q_scale q_t)
//
// Mapping: one workgroup per (b,h) holds the whole V x K fp32 state in VGPRs,
// one row of S per 8 lanes (16 coordinates each: K <= 128), so the two row
// dot products of a token are 3-step DPP reductions inside a group of 8 lanes
// and rows never exchange data.  Tokens are taken in blocks of 16: the
// workgroup stages the block's k, q, v, beta, r, alpha in LDS as fp32, wave 0
// runs the preconditioner over the block (d in VGPRs, two coordinates per
// lane) and leaves the write keys in LDS, then every row applies the block's
// updates and leaves its readouts in LDS for one coalesced store.  The state
// is read once at the start and written once at the end: a single-token call
// moves 2 * 4 V K bytes of state per (b,h) plus the token's rows.  Because
// one workgroup owns a (b,h), S_out may alias S0 and d_out may alias d1.
#include "kernels.h"
#include "profile.h"

namespace osdn {
namespace {

constexpr int DEC_TB = 16;   // tokens per staged block
constexpr int DEC_P = 128;   // LDS row pitch in floats (K, V <= 128)

template <int CTL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTL, 0xF, 0xF, false));
}

// Sum over aligned groups of 8 lanes; every lane of a group receives it.
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp<0xB1>(x);         // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);         // quad_perm [2,3,0,1]: quad sums
  return x + dpp<0x141>(x);  // row_half_mirror: lane i takes lane 7 - i of its 8
}

__device__ __forceinline__ floatx4 lds4(const float *p) { return *reinterpret_cast<const floatx4 *>(p); }

// KM = ceil(K / 32): lane (row, l8) holds coordinates 32 m + 4 l8 + c of its
// row for m < KM, c < 4, so one LDS or state load per m covers a row's 32
// consecutive floats with the 8 lanes of the row.
//
// LDS (dynamic, sized for TB = min(T, 16) staged tokens so a single-token
// call needs 2.5 KB): k, write keys, q, v and readouts [TB][128] fp32 each,
// then beta, r, alpha [TB].  At most 64 VGPRs, so two 1024-lane workgroups
// share a CU and one's state loads overlap the other's updates and stores.
// VEC (K % 4 == 0): state rows move as 16-byte vectors, else element-wise.
template <typename TIn, int KM, bool VEC, bool OF32>
__global__ __launch_bounds__(1024, 8) void decode_kernel(DecodeArgs a) {
  extern __shared__ floatx4 dec_smem[];
  const int TB = a.tb;
  typedef float Row[DEC_P];
  Row *sK = reinterpret_cast<Row *>(dec_smem);
  Row *sKt = sK + TB, *sQ = sKt + TB, *sV = sQ + TB, *sO = sV + TB;
  float *sB = reinterpret_cast<float *>(sO + TB), *sR = sB + TB, *sA = sR + TB;

  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  const int64_t seq = blockIdx.x;  // (b,h)
  const int64_t H = a.H, T = a.T, K = a.K, V = a.V;
  const int64_t b = seq / H, h = seq - b * H;
  const int row = tid >> 3, l8 = tid & 7;
  const bool active = row < V;

  // this lane's slice of its state row.  Loads are clamped in bounds (an
  // inactive row reads row V - 1, a slot past K reads within the row) and
  // not masked, so nothing waits on them before the first update: a slot
  // past K only ever meets zero keys, queries and write keys (inputs are
  // finite), and neither it nor an inactive row is stored.
  float S[KM][4];
#pragma unroll
  for (int m = 0; m < KM; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) S[m][c] = 0.0f;
  if (a.S0) {
    const float *src = a.S0 + (seq * V + (active ? row : V - 1)) * K;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const int j0 = 32 * m + 4 * l8;
      if constexpr (VEC) {
        const floatx4 x = *reinterpret_cast<const floatx4 *>(src + (j0 < K ? j0 : K - 4));
#pragma unroll
        for (int c = 0; c < 4; ++c) S[m][c] = x[c];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) S[m][c] = src[j0 + c < K ? j0 + c : K - 1];
      }
    }
  }

  // wave 0: d, coordinates lane and lane + 64
  float d[2] = {0.0f, 0.0f};
  if (tid < 64) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t j = lane + 64 * e;
      if (j < K) d[e] = a.d1 ? a.d1[seq * K + j] : 1.0f;
    }
  }

  const TIn *qp = static_cast<const TIn *>(a.q);
  const TIn *kp = static_cast<const TIn *>(a.k);
  const TIn *vp = static_cast<const TIn *>(a.v);
  const int64_t tok0 = b * T * H + h;  // flat [B,T,H] index of this (b,h)'s token 0
  const float eta = a.eta, eps = a.eps, dmin = a.d_min, dmax = a.d_max, qs = a.q_scale;
  const bool clamp = a.clamp != 0, aware = a.beta_aware != 0, gated = a.alpha != nullptr;

  // one block of up to TB tokens; the first block is peeled off the loop so
  // that a call of at most TB tokens is straight-line code and the waits on
  // the state and staging loads stay exact
  auto block = [&](int64_t t0) __attribute__((always_inline)) {
    const int nb = (int)(T - t0 < TB ? T - t0 : TB);
    // stage the block: every load is issued before any LDS write (addresses
    // clamped in bounds, values masked), so the block costs one round trip;
    // keys and queries are zero beyond K
    float bx, rx, ax;  // set and used only where tid < nb
    if (tid < nb) {
      const int64_t x = tok0 + (t0 + tid) * H;
      bx = a.beta[x];
      rx = (a.r ? a.r : a.beta)[x];
      ax = (gated ? a.alpha : a.beta)[x];
    }
    // one load per thread and pass: k, q, v rows of the block, flattened
    // (sK, sQ, sV sit at rows 0, 2 TB, 3 TB of the LDS block)
    const int per = nb * DEC_P;
    for (int e = tid; e < 3 * per; e += nt) {
      const int w = e / per, r = e - w * per;  // w: 0 k, 1 q, 2 v
      const int t = r / DEC_P, j = r - t * DEC_P;
      const int64_t tr = tok0 + (t0 + t) * H;
      float x;
      if (w == 0)
        x = to_f32(kp[tr * K + (j < K ? j : K - 1)]);
      else if (w == 1)
        x = qs * to_f32(qp[tr * K + (j < K ? j : K - 1)]);
      else
        x = to_f32(vp[tr * V + (j < V ? j : V - 1)]);
      sK[(w == 0 ? 0 : (w == 1 ? 2 : 3) * TB) + t][j] = j < (w == 2 ? V : K) ? x : 0.0f;
    }
    if (tid < nb) {
      sB[tid] = bx;
      sR[tid] = a.r ? rx : 1.0f;
      sA[tid] = gated ? ax : 1.0f;
    }
    __syncthreads();

    // wave 0: the preconditioner over the block, write keys into sKt
    if (tid < 64) {
      for (int t = 0; t < nb; ++t) {
        float k[2], s[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          k[e] = sK[t][lane + 64 * e];
          s[e] = k[e] * k[e];
        }
        const float norm = wave_sum(s[0] + s[1]);
        const float align = wave_sum(fmaf(d[0], s[0], d[1] * s[1]));
        const float bpr = aware ? sB[t] : 1.0f;
        const float ea = eta * bpr / fmaxf(norm, eps);
        const float c = fmaf(-ea * bpr, align, ea);  // eta b' (1 - b' <d, s>) / n
        const float rt = sR[t];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          sKt[t][lane + 64 * e] = d[e] * k[e];  // emitted before the update
          float x = fmaf(c, s[e], rt * d[e]);
          if (clamp) x = fminf(fmaxf(x, dmin), dmax);
          d[e] = lane + 64 * e < K ? x : 0.0f;
        }
      }
    }
    __syncthreads();

    // every row: the block's delta-rule updates and readouts
    for (int t = 0; t < nb; ++t) {
      if (gated) {
        const float at = sA[t];
#pragma unroll
        for (int m = 0; m < KM; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c) S[m][c] *= at;
      }
      float p = 0.0f;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const floatx4 kv = lds4(&sK[t][32 * m + 4 * l8]);
#pragma unroll
        for (int c = 0; c < 4; ++c) p = fmaf(S[m][c], kv[c], p);
      }
      p = group8_sum(p);  // (Sb k_t) of this row
      const float bu = sB[t] * ((active ? sV[t][row] : 0.0f) - p);
      float po = 0.0f;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const floatx4 wv = lds4(&sKt[t][32 * m + 4 * l8]);
        const floatx4 qv = lds4(&sQ[t][32 * m + 4 * l8]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          S[m][c] = fmaf(bu, wv[c], S[m][c]);
          po = fmaf(S[m][c], qv[c], po);
        }
      }
      po = group8_sum(po);
      if (active && l8 == 0) sO[t][row] = po;
    }
    __syncthreads();
    for (int e = tid; e < nb * (int)V; e += nt) {
      const int t = e / (int)V, i = e - t * (int)V;
      store_out_t<TIn, OF32>(a.o, (tok0 + (t0 + t) * H) * V + i, sO[t][i]);
    }
    // the next block's staging touches sK, sQ, sV, sB, sR, sA only, whose last
    // readers finished before the barrier above; sKt and sO are rewritten
    // after two more barriers
  };
  if (T > 0) block(0);
  for (int64_t t0 = TB; t0 < T; t0 += TB) block(t0);

  if (a.S_out && active) {
    float *dst = a.S_out + (seq * V + row) * K;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const int j0 = 32 * m + 4 * l8;
      if constexpr (VEC) {
        if (j0 < K) *reinterpret_cast<floatx4 *>(dst + j0) = floatx4{S[m][0], S[m][1], S[m][2], S[m][3]};
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (j0 + c < K) dst[j0 + c] = S[m][c];
      }
    }
  }
  if (a.d_out && tid < 64) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t j = lane + 64 * e;
      if (j < K) a.d_out[seq * K + j] = d[e];
    }
  }
}

template <typename TIn, bool VEC, bool OF32>
hipError_t launch_vec(DecodeArgs a, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.H));
  const dim3 block((unsigned)(((8 * a.V + 63) / 64) * 64));
  a.tb = (int)(a.T < DEC_TB ? (a.T > 0 ? a.T : 1) : DEC_TB);
  const size_t lds = (size_t)a.tb * (5 * DEC_P + 3) * sizeof(float);
  switch ((a.K + 31) / 32) {
    case 1: hipLaunchKernelGGL((decode_kernel<TIn, 1, VEC, OF32>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<TIn, 2, VEC, OF32>), grid, block, lds, s, a); break;
    case 3: hipLaunchKernelGGL((decode_kernel<TIn, 3, VEC, OF32>), grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL((decode_kernel<TIn, 4, VEC, OF32>), grid, block, lds, s, a); break;
  }
  prof_mark(s, "decode_kernel");
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t s) {
  // float32 readout for bf16 inputs: a variant (no branch at the stores)
  if (a.o_f32 && sizeof(TIn) == 2)
    return a.K % 4 == 0 ? launch_vec<TIn, true, true>(a, s) : launch_vec<TIn, false, true>(a, s);
  return a.K % 4 == 0 ? launch_vec<TIn, true, false>(a, s) : launch_vec<TIn, false, false>(a, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, bool is_bf16, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  return is_bf16 ? launch_typed<bf16>(a, s) : launch_typed<float>(a, s);
}

}  // namespace osdn
