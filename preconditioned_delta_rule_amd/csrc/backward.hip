// Backward pass of the OSDN forward: gradients of a loss through phase 2 (the
// delta rule with the preconditioned write key) and phase 1 (the clamped
// preconditioner recurrence).
//
// Paper: "OSDN: Improving Delta Rule with Provable Online Preconditioning in
// Linear Attention", Section 4.5 (the gradient reaches d through
// k~ = d (.) k and is swept back through the clamped recurrence), with the
// forward of Section 4.2 Eq.(4) / Section 4.4 Eq.(7) and Section 4.3 Eq.(5),
// gated as in Appendix B.1.  With G = dL/dS_t swept from t = T down to 1:
//   G += q_scale dout_t q_t^T;          dq_t  = q_scale S_t^T dout_t
//   w = G k~_t;  dv_t = beta_t w;       dbeta_t = u_t . w        (+ phase 1)
//   dk~_t = beta_t G^T u_t;             dk_t  = -beta_t Sb_t^T w  (+ phase 1)
//   dSb = G - beta_t w k_t^T;           dalpha_t = <dSb, S_{t-1}>;  G = alpha_t dSb
// then with g = dL/dd_{t+1}, the clamp's pass mask m and y the pre-clip step:
//   gy = m (.) g;  gc = s . gy;  dr_t = d_t . gy
//   dk_t += 2 k_t (.) (c gy - gc eta b'^2/n d_t - [|k|^2 > eps] gc c/n) + dk~_t (.) d_t
//   dbeta_t += gc eta (1 - 2 b' a)/n (beta-aware);  g = dk~_t (.) k_t + r_t gy - (eta b'^2/n)(s . gy) s
//
// Three kernels, each one workgroup (or wave) per (b,h):
//  bwd_record_kernel  the forward once more, token by token (the decode
//                     step's layout: a state row per 8 lanes), recording the
//                     residual u_t of every token and S, d every 16 tokens;
//  bwd_p2_kernel      the phase-2 sweep backwards in blocks of 16 tokens, the
//                     state held transposed (a key row of S^T per 8 lanes), so
//                     dq, dk~ and the read-key gradient are reductions inside
//                     8 lanes and only w = G k~ crosses rows (one LDS pass, two
//                     barriers per token); the states inside a block are
//                     rebuilt backwards from the block's end with the recorded
//                     residuals, S_{t-1} = (S_t - beta u k~^T) / alpha, and the
//                     write keys by replaying phase 1 from the recorded d;
//  bwd_p1_kernel      the phase-1 sweep backwards, one wave per (b,h), each
//                     block's d replayed forward from the recorded d first.
#include "kernels.h"
#include "profile.h"

namespace osdn {
namespace {

constexpr int BT = 16;   // tokens per block (and between recorded states)
constexpr int BP = 128;  // LDS row pitch in floats (K, V <= 128)

template <int CTL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTL, 0xF, 0xF, false));
}

// Sum over aligned groups of 8 lanes; every lane of a group receives it.
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp_mov<0xB1>(x);         // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);         // quad_perm [2,3,0,1]
  return x + dpp_mov<0x141>(x);  // row_half_mirror
}

// Sum over the 8 lanes l8, l8 + 8, ..., l8 + 56 of a wave (the same slot of
// its 8 row groups); every lane receives the sum of its slot.
__device__ __forceinline__ float rows8_sum(float x) {
  x += dpp_mov<0x128>(x);  // row_ror:8 -- the other half of the 16-lane row
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ floatx4 lds4(const float *p) { return *reinterpret_cast<const floatx4 *>(p); }

struct P1 {
  float eta, eps, dmin, dmax;
  bool clamp, aware;
};

// One preconditioner step on wave 0's two coordinates per lane (lane, lane +
// 64): returns the step scalar c and leaves y (before the clamp) in y[].
__device__ __forceinline__ float p1_step(const P1 &p, const float (&d)[2], const float (&k)[2], float beta, float r,
                                         float (&y)[2]) {
  float s[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) s[e] = k[e] * k[e];
  const float norm = wave_sum(s[0] + s[1]);
  const float align = wave_sum(fmaf(d[0], s[0], d[1] * s[1]));
  const float bpr = p.aware ? beta : 1.0f;
  const float ea = p.eta * bpr / fmaxf(norm, p.eps);
  const float c = fmaf(-ea * bpr, align, ea);  // eta b' (1 - b' <d, s>) / n
#pragma unroll
  for (int e = 0; e < 2; ++e) y[e] = fmaf(c, s[e], r * d[e]);
  return c;
}

__device__ __forceinline__ float p1_clip(const P1 &p, float y) {
  return p.clamp ? fminf(fmaxf(y, p.dmin), p.dmax) : y;
}

// ===================================================================== record
// KM = ceil(K / 32): lane (row i of S, l8) holds S[i][32 m + 4 l8 + c].
template <typename TIn, int KM>
__global__ __launch_bounds__(1024) void bwd_record_kernel(BwdArgs a) {
  __shared__ float sK[BT][BP], sKt[BT][BP], sV[BT][BP], sU[BT][BP];
  __shared__ float sB[BT], sR[BT], sA[BT];
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  const int64_t seq = blockIdx.x;
  const int64_t H = a.H, T = a.T, K = a.K, V = a.V;
  const int64_t b = seq / H, h = seq - b * H;
  const int row = tid >> 3, l8 = tid & 7;
  const bool active = row < V;
  const int64_t NB = (T + BT - 1) / BT;
  const P1 p{a.eta, a.eps, a.d_min, a.d_max, a.clamp != 0, a.beta_aware != 0};
  const bool gated = a.alpha != nullptr;

  float S[KM][4];
#pragma unroll
  for (int m = 0; m < KM; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 32 * m + 4 * l8 + c;
      S[m][c] = (a.S0 && active && j < K) ? a.S0[(seq * V + row) * K + j] : 0.0f;
    }
  float d[2] = {0.0f, 0.0f};
  if (tid < 64) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t j = lane + 64 * e;
      if (j < K) d[e] = a.d1 ? a.d1[seq * K + j] : 1.0f;
    }
  }
  const TIn *kp = static_cast<const TIn *>(a.k);
  const TIn *vp = static_cast<const TIn *>(a.v);
  const int64_t tok0 = b * T * H + h;

  auto record_state = [&](int64_t blk) {
    float *dst = a.ck + ((seq * (NB + 1) + blk) * V + (active ? row : 0)) * K;
    if (active) {
#pragma unroll
      for (int m = 0; m < KM; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 32 * m + 4 * l8 + c;
          if (j < K) dst[j] = S[m][c];
        }
    }
    if (tid < 64) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t j = lane + 64 * e;
        if (j < K) a.dck[(seq * (NB + 1) + blk) * K + j] = d[e];
      }
    }
  };

  for (int64_t blk = 0; blk < NB; ++blk) {
    const int64_t t0 = blk * BT;
    const int nb = (int)(T - t0 < BT ? T - t0 : BT);
    record_state(blk);
    const int per = nb * BP;
    for (int e = tid; e < 2 * per; e += nt) {
      const int w = e / per, r = e - w * per;
      const int t = r / BP, j = r - t * BP;
      const int64_t tr = tok0 + (t0 + t) * H;
      if (w == 0)
        sK[t][j] = j < K ? to_f32(kp[tr * K + j]) : 0.0f;
      else
        sV[t][j] = j < V ? to_f32(vp[tr * V + j]) : 0.0f;
    }
    if (tid < nb) {
      const int64_t x = tok0 + (t0 + tid) * H;
      sB[tid] = a.beta[x];
      sR[tid] = a.r ? a.r[x] : 1.0f;
      sA[tid] = gated ? a.alpha[x] : 1.0f;
    }
    __syncthreads();
    if (tid < 64) {
      for (int t = 0; t < nb; ++t) {
        const float k[2] = {sK[t][lane], sK[t][lane + 64]};
        float y[2];
        p1_step(p, d, k, sB[t], sR[t], y);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          sKt[t][lane + 64 * e] = d[e] * k[e];
          d[e] = lane + 64 * e < K ? p1_clip(p, y[e]) : 0.0f;
        }
      }
    }
    __syncthreads();
    for (int t = 0; t < nb; ++t) {
      if (gated) {
        const float at = sA[t];
#pragma unroll
        for (int m = 0; m < KM; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c) S[m][c] *= at;
      }
      float pr = 0.0f;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const floatx4 kv = lds4(&sK[t][32 * m + 4 * l8]);
#pragma unroll
        for (int c = 0; c < 4; ++c) pr = fmaf(S[m][c], kv[c], pr);
      }
      pr = group8_sum(pr);
      const float u = (active ? sV[t][row] : 0.0f) - pr;
      if (active && l8 == 0) sU[t][row] = u;
      const float bu = sB[t] * u;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const floatx4 wv = lds4(&sKt[t][32 * m + 4 * l8]);
#pragma unroll
        for (int c = 0; c < 4; ++c) S[m][c] = fmaf(bu, wv[c], S[m][c]);
      }
    }
    __syncthreads();
    for (int e = tid; e < nb * (int)V; e += nt) {
      const int t = e / (int)V, i = e - t * (int)V;
      a.u[(tok0 + (t0 + t) * H) * V + i] = sU[t][i];
    }
    // the next block's staging writes sK, sV, sB, sR, sA, read last before
    // the barrier above; sKt and sU are rewritten after two more barriers
  }
  record_state(NB);
}

// ============================================================ phase-2 reverse
// Transposed state: lane (key row j, l8) holds S[32 m + 4 l8 + c][j] and the
// same slots of G, VM = ceil(V / 32).
template <typename TIn, int VM>
__global__ __launch_bounds__(1024) void bwd_p2_kernel(BwdArgs a) {
  __shared__ float sQ[BT][BP], sK[BT][BP], sKt[BT][BP], sDo[BT][BP], sU[BT][BP];
  __shared__ float sDq[BT][BP], sDkt[BT][BP], sDkr[BT][BP], sDv[BT][BP];
  __shared__ float sWp[16][BP], sW[BP];
  __shared__ float sDa[BT][16], sDb[BT][2];
  __shared__ float sB[BT], sR[BT], sA[BT];
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6;
  const int nwaves = nt >> 6;
  const int64_t seq = blockIdx.x;
  const int64_t H = a.H, T = a.T, K = a.K, V = a.V;
  const int64_t b = seq / H, h = seq - b * H;
  const int row = tid >> 3, l8 = tid & 7;  // row = key index j
  const bool active = row < K;
  const int64_t NB = (T + BT - 1) / BT;
  const P1 p{a.eta, a.eps, a.d_min, a.d_max, a.clamp != 0, a.beta_aware != 0};
  const bool gated = a.alpha != nullptr;
  const float qs = a.q_scale;

  float G[VM][4], S[VM][4];
#pragma unroll
  for (int m = 0; m < VM; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = 32 * m + 4 * l8 + c;
      G[m][c] = (a.dS && active && i < V) ? a.dS[(seq * V + i) * K + row] : 0.0f;
    }

  const TIn *qp = static_cast<const TIn *>(a.q);
  const TIn *kp = static_cast<const TIn *>(a.k);
  const TIn *dop = static_cast<const TIn *>(a.dout);
  TIn *dqp = static_cast<TIn *>(a.dq);
  TIn *dvp = static_cast<TIn *>(a.dv);
  const int64_t tok0 = b * T * H + h;

  for (int64_t blk = NB - 1; blk >= 0; --blk) {
    const int64_t t0 = blk * BT;
    const int nb = (int)(T - t0 < BT ? T - t0 : BT);
    __syncthreads();  // the previous block's write-out is done with the LDS
    // the state after the block's last token
    {
      const float *src = a.ck + (seq * (NB + 1) + blk + 1) * V * K;
#pragma unroll
      for (int m = 0; m < VM; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 32 * m + 4 * l8 + c;
          S[m][c] = (active && i < V) ? src[(int64_t)i * K + row] : 0.0f;
        }
    }
    // stage q (scaled), k, dout, u of the block
    const int per = nb * BP;
    for (int e = tid; e < 4 * per; e += nt) {
      const int w = e / per, r = e - w * per;
      const int t = r / BP, j = r - t * BP;
      const int64_t tr = tok0 + (t0 + t) * H;
      if (w == 0)
        sQ[t][j] = j < K ? qs * to_f32(qp[tr * K + j]) : 0.0f;
      else if (w == 1)
        sK[t][j] = j < K ? to_f32(kp[tr * K + j]) : 0.0f;
      else if (w == 2)
        sDo[t][j] = j < V ? to_f32(dop[tr * V + j]) : 0.0f;
      else
        sU[t][j] = j < V ? a.u[tr * V + j] : 0.0f;
    }
    if (tid < nb) {
      const int64_t x = tok0 + (t0 + tid) * H;
      sB[tid] = a.beta[x];
      sR[tid] = a.r ? a.r[x] : 1.0f;
      sA[tid] = gated ? a.alpha[x] : 1.0f;
    }
    __syncthreads();
    // wave 0: the write keys of the block, replayed from the recorded d
    if (tid < 64) {
      float d[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t j = lane + 64 * e;
        d[e] = j < K ? a.dck[(seq * (NB + 1) + blk) * K + j] : 0.0f;
      }
      for (int t = 0; t < nb; ++t) {
        const float k[2] = {sK[t][lane], sK[t][lane + 64]};
        float y[2];
        p1_step(p, d, k, sB[t], sR[t], y);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          sKt[t][lane + 64 * e] = d[e] * k[e];
          d[e] = lane + 64 * e < K ? p1_clip(p, y[e]) : 0.0f;
        }
      }
    }
    __syncthreads();

    for (int t = nb - 1; t >= 0; --t) {
      const float qj = sQ[t][row], kj = sK[t][row], ktj = sKt[t][row];
      const float bt = sB[t];
      // readout: G += q_scale dout q^T, dq = q_scale S^T dout
      float pdq = 0.0f;
#pragma unroll
      for (int m = 0; m < VM; ++m) {
        const floatx4 dov = lds4(&sDo[t][32 * m + 4 * l8]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          G[m][c] = fmaf(qj, dov[c], G[m][c]);
          pdq = fmaf(S[m][c], dov[c], pdq);
        }
      }
      pdq = group8_sum(pdq);
      // w = G k~ (over key rows: across lanes and waves)
#pragma unroll
      for (int m = 0; m < VM; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float x = rows8_sum(G[m][c] * ktj);
          if (lane < 8) sWp[wv][32 * m + 4 * l8 + c] = x;
        }
      __syncthreads();
      if (tid < V) {
        float x = 0.0f;
        for (int q = 0; q < nwaves; ++q) x += sWp[q][tid];
        sW[tid] = x;
        sDv[t][tid] = bt * x;
      }
      if (wv < (int)((V + 63) >> 6)) {
        const float x = tid < V ? sU[t][tid] * sW[tid] : 0.0f;
        // sW[tid] was written by this same thread just above
        const float sum = wave_sum(x);
        if (lane == 0) sDb[t][wv] = sum;
      }
      __syncthreads();
      // dk~ = beta G^T u; the state before the write; dk_read = -beta Sb^T w
      float pdkt = 0.0f, pdkr = 0.0f;
#pragma unroll
      for (int m = 0; m < VM; ++m) {
        const floatx4 uv = lds4(&sU[t][32 * m + 4 * l8]);
        const floatx4 wvv = lds4(&sW[32 * m + 4 * l8]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pdkt = fmaf(G[m][c], uv[c], pdkt);
          S[m][c] = fmaf(-bt * ktj, uv[c], S[m][c]);  // Sb
          pdkr = fmaf(S[m][c], wvv[c], pdkr);
          G[m][c] = fmaf(-bt * kj, wvv[c], G[m][c]);  // dSb
        }
      }
      pdkt = group8_sum(pdkt);
      pdkr = group8_sum(pdkr);
      if (active && l8 == 0) {
        sDq[t][row] = pdq;  // q_scale is in sQ's staging only; applied on store
        sDkt[t][row] = bt * pdkt;
        sDkr[t][row] = -bt * pdkr;
      }
      // decay: S_{t-1} = Sb / alpha, dalpha = <dSb, S_{t-1}>, G = alpha dSb
      if (gated) {
        const float at = sA[t], inv = 1.0f / at;
        float pda = 0.0f;
#pragma unroll
        for (int m = 0; m < VM; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            S[m][c] *= inv;
            pda = fmaf(G[m][c], S[m][c], pda);
            G[m][c] *= at;
          }
        pda = wave_sum(pda);
        if (lane == 0) sDa[t][wv] = pda;
      }
    }
    __syncthreads();
    // write the block's gradients
    for (int e = tid; e < nb * (int)K; e += nt) {
      const int t = e / (int)K, j = e - t * (int)K;
      const int64_t tr = tok0 + (t0 + t) * H;
      dqp[tr * K + j] = from_f32<TIn>(qs * sDq[t][j]);
      a.dkt[tr * K + j] = sDkt[t][j];
      a.dkr[tr * K + j] = sDkr[t][j];
    }
    for (int e = tid; e < nb * (int)V; e += nt) {
      const int t = e / (int)V, i = e - t * (int)V;
      dvp[(tok0 + (t0 + t) * H) * V + i] = from_f32<TIn>(sDv[t][i]);
    }
    if (tid < nb) {
      const int64_t x = tok0 + (t0 + tid) * H;
      float db = 0.0f;
      for (int q = 0; q < (int)((V + 63) >> 6); ++q) db += sDb[tid][q];
      a.dbp2[x] = db;
      if (gated && a.dalpha) {
        float da = 0.0f;
        for (int q = 0; q < nwaves; ++q) da += sDa[tid][q];
        a.dalpha[x] = da;
      }
    }
  }
  if (a.dS0 && active) {
#pragma unroll
    for (int m = 0; m < VM; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 32 * m + 4 * l8 + c;
        if (i < V) a.dS0[(seq * V + i) * K + row] = G[m][c];
      }
  }
}

// ============================================================ phase-1 reverse
template <typename TIn>
__global__ __launch_bounds__(64) void bwd_p1_kernel(BwdArgs a) {
  __shared__ float sD[BT][BP], sK[BT][BP];
  __shared__ float sC[BT];
  const int lane = threadIdx.x;
  const int64_t seq = blockIdx.x;
  const int64_t H = a.H, T = a.T, K = a.K;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t NB = (T + BT - 1) / BT;
  const P1 p{a.eta, a.eps, a.d_min, a.d_max, a.clamp != 0, a.beta_aware != 0};
  const TIn *kp = static_cast<const TIn *>(a.k);
  TIn *dkp = static_cast<TIn *>(a.dk);
  const int64_t tok0 = b * T * H + h;

  float g[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t j = lane + 64 * e;
    g[e] = (a.dd && j < K) ? a.dd[seq * K + j] : 0.0f;
  }
  for (int64_t blk = NB - 1; blk >= 0; --blk) {
    const int64_t t0 = blk * BT;
    const int nb = (int)(T - t0 < BT ? T - t0 : BT);
    // replay d over the block from the recorded start, keeping d_t and c_t
    float d[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t j = lane + 64 * e;
      d[e] = j < K ? a.dck[(seq * (NB + 1) + blk) * K + j] : 0.0f;
    }
    for (int t = 0; t < nb; ++t) {
      const int64_t tr = tok0 + (t0 + t) * H;
      float k[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t j = lane + 64 * e;
        k[e] = j < K ? to_f32(kp[tr * K + j]) : 0.0f;
        sK[t][lane + 64 * e] = k[e];
        sD[t][lane + 64 * e] = d[e];
      }
      float y[2];
      const float c = p1_step(p, d, k, a.beta[tr], a.r ? a.r[tr] : 1.0f, y);
      if (lane == 0) sC[t] = c;
#pragma unroll
      for (int e = 0; e < 2; ++e) d[e] = lane + 64 * e < K ? p1_clip(p, y[e]) : 0.0f;
    }
    __syncthreads();
    for (int t = nb - 1; t >= 0; --t) {
      const int64_t tr = tok0 + (t0 + t) * H;
      const float bt = a.beta[tr], rt = a.r ? a.r[tr] : 1.0f, c = sC[t];
      const float bpr = p.aware ? bt : 1.0f;
      float dv[2], k[2], s[2], gy[2], dkt[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t j = lane + 64 * e;
        dv[e] = sD[t][lane + 64 * e];
        k[e] = sK[t][lane + 64 * e];
        s[e] = k[e] * k[e];
        const float y = fmaf(c, s[e], rt * dv[e]);
        // branch-free on purpose: with a short-circuit || on the uniform
        // clamp flag, the compiler dropped g from the passing lanes
        const bool pass = (y >= p.dmin) & (y <= p.dmax) | !p.clamp;
        gy[e] = pass ? g[e] : 0.0f;
        dkt[e] = j < K ? a.dkt[tr * K + j] : 0.0f;
      }
      const float nraw = wave_sum(s[0] + s[1]);
      const float align = wave_sum(fmaf(dv[0], s[0], dv[1] * s[1]));
      const float gc = wave_sum(fmaf(s[0], gy[0], s[1] * gy[1]));
      const float grr = wave_sum(fmaf(dv[0], gy[0], dv[1] * gy[1]));
      const float n = fmaxf(nraw, p.eps);
      const float dca = -p.eta * bpr * bpr / n;            // dc / d<d, s>
      const float dcn = nraw > p.eps ? -c / n : 0.0f;      // dc / dn
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t j = lane + 64 * e;
        const float ds = fmaf(c, gy[e], gc * fmaf(dca, dv[e], dcn));
        if (j < K) {
          const float dk = a.dkr[tr * K + j] + fmaf(2.0f * k[e], ds, dkt[e] * dv[e]);
          dkp[tr * K + j] = from_f32<TIn>(dk);
        }
        g[e] = j < K ? fmaf(dkt[e], k[e], fmaf(rt, gy[e], dca * s[e] * gc)) : 0.0f;
      }
      if (lane == 0) {
        float db = a.dbp2[tr];
        if (p.aware) db += gc * p.eta * (1.0f - 2.0f * bpr * align) / n;
        a.dbeta[tr] = db;
        if (a.dr) a.dr[tr] = grr;
      }
    }
    __syncthreads();  // sD, sK, sC are rewritten by the next block's replay
  }
  if (a.dd1) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t j = lane + 64 * e;
      if (j < K) a.dd1[seq * K + j] = g[e];
    }
  }
}

template <typename TIn>
hipError_t launch_typed(const BwdArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.H));
  const dim3 brec((unsigned)(((8 * a.V + 63) / 64) * 64));
  const dim3 bp2((unsigned)(((8 * a.K + 63) / 64) * 64));
  switch ((a.K + 31) / 32) {
    case 1: hipLaunchKernelGGL((bwd_record_kernel<TIn, 1>), grid, brec, 0, s, a); break;
    case 2: hipLaunchKernelGGL((bwd_record_kernel<TIn, 2>), grid, brec, 0, s, a); break;
    case 3: hipLaunchKernelGGL((bwd_record_kernel<TIn, 3>), grid, brec, 0, s, a); break;
    default: hipLaunchKernelGGL((bwd_record_kernel<TIn, 4>), grid, brec, 0, s, a); break;
  }
  prof_mark(s, "bwd_record_kernel");
  switch ((a.V + 31) / 32) {
    case 1: hipLaunchKernelGGL((bwd_p2_kernel<TIn, 1>), grid, bp2, 0, s, a); break;
    case 2: hipLaunchKernelGGL((bwd_p2_kernel<TIn, 2>), grid, bp2, 0, s, a); break;
    case 3: hipLaunchKernelGGL((bwd_p2_kernel<TIn, 3>), grid, bp2, 0, s, a); break;
    default: hipLaunchKernelGGL((bwd_p2_kernel<TIn, 4>), grid, bp2, 0, s, a); break;
  }
  prof_mark(s, "bwd_p2_kernel");
  hipLaunchKernelGGL((bwd_p1_kernel<TIn>), grid, dim3(64), 0, s, a);
  prof_mark(s, "bwd_p1_kernel");
  return hipGetLastError();
}

}  // namespace

size_t bwd_work_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t NB = (size_t)((T + BT - 1) / BT);
  const size_t BH = (size_t)(B * H), tok = (size_t)(B * T * H);
  return al(tok * V * 4) + al(BH * (NB + 1) * V * K * 4) + al(BH * (NB + 1) * K * 4) + 2 * al(tok * K * 4) +
         al(tok * 4);
}

void bwd_work_layout(BwdArgs &a, void *base) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t NB = (size_t)((a.T + BT - 1) / BT);
  const size_t BH = (size_t)(a.B * a.H), tok = (size_t)(a.B * a.T * a.H);
  char *p = static_cast<char *>(base);
  a.u = reinterpret_cast<float *>(p);
  p += al(tok * a.V * 4);
  a.ck = reinterpret_cast<float *>(p);
  p += al(BH * (NB + 1) * a.V * a.K * 4);
  a.dck = reinterpret_cast<float *>(p);
  p += al(BH * (NB + 1) * a.K * 4);
  a.dkt = reinterpret_cast<float *>(p);
  p += al(tok * a.K * 4);
  a.dkr = reinterpret_cast<float *>(p);
  p += al(tok * a.K * 4);
  a.dbp2 = reinterpret_cast<float *>(p);
}

hipError_t launch_bwd(const BwdArgs &a, bool is_bf16, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  return is_bf16 ? launch_typed<bf16>(a, s) : launch_typed<float>(a, s);
}

}  // namespace osdn
