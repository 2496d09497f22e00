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
// Every value row i of S (and of G) evolves on its own given the keys, so
// the two sweeps over S split a (b,h) into ceil(V/32) slices of 32 value
// rows, one workgroup each, and only sums over value rows (dq, dk~, the
// read-key gradient, dbeta, dalpha) are left as per-slice partials:
//  bwd_record_kernel  the forward once more, token by token (the decode
//                     step's layout: a state row per 8 lanes), recording the
//                     residual u_t of every token and S, d every 16 tokens;
//  bwd_p2_kernel      the phase-2 sweep backwards in blocks of 16 tokens, the
//                     slice's state held transposed (a key row per 8 lanes,
//                     4 value columns per lane), so dq, dk~ and the read-key
//                     gradient are reductions inside 8 lanes and only
//                     w = G k~ crosses key rows (one LDS pass, two barriers
//                     per token); the states inside a block are rebuilt
//                     backwards from the block's end with the recorded
//                     residuals, S_{t-1} = (S_t - beta u k~^T) / alpha, and the
//                     write keys by replaying phase 1 from the recorded d;
//  bwd_p1_kernel      the phase-1 sweep backwards, one wave per (b,h) with
//                     each block's d replayed forward from the recorded d,
//                     while nine more waves sum the slices' partials of the
//                     next block into LDS (and finish dq and dalpha).
#include "kernels.h"
#include "profile.h"

namespace osdn {
namespace {

constexpr int BT = 16;   // tokens per block (and between recorded states)
constexpr int BP = 128;  // LDS row pitch in floats (K, V <= 128)
constexpr int VS = 32;   // value rows per slice

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

// One [B,T,H,L] operand of a token block, columns [c0, c0 + n) staged into
// LDS rows (zero from column n on).
template <typename TSrc>
struct RowSrc {
  const TSrc *p;  // the tensor
  int64_t L;      // its last dimension
  int64_t c0, n;  // first column and number of columns staged
  float *dst;     // LDS rows of pitch P (the stage call's)
  float scale;
};

// Copies tokens [t0, t0 + nb) of a (b,h) (token row tr = tok0 + t H) from two
// operands into LDS rows of W columns (pitch P): every thread issues its 2 U
// loads (addresses clamped in bounds) before any LDS write, so a block costs
// one round trip when U nt >= nb W.
template <int U, int W, int P, typename TA, typename TB>
__device__ __forceinline__ void stage2(const RowSrc<TA> &A, const RowSrc<TB> &Bs, int64_t tok0, int64_t H,
                                       int64_t t0, int nb, int tid, int nt) {
  const int total = nb * W;
  for (int base = tid; base < total; base += U * nt) {
    float xa[U], xb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = min(base + u * nt, total - 1);
      const int t = e / W, j = e - t * W;
      const int64_t tr = tok0 + (t0 + t) * H;
      xa[u] = to_f32(A.p[tr * A.L + A.c0 + (j < A.n ? j : A.n - 1)]);
      xb[u] = to_f32(Bs.p[tr * Bs.L + Bs.c0 + (j < Bs.n ? j : Bs.n - 1)]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = base + u * nt;
      if (e < total) {
        const int t = e / W, j = e - t * W;
        A.dst[t * P + j] = j < A.n ? A.scale * xa[u] : 0.0f;
        Bs.dst[t * P + j] = j < Bs.n ? Bs.scale * xb[u] : 0.0f;
      }
    }
  }
}

// Gates of a token block (threads < nb): beta, r (1 without), alpha (1
// without), loaded unconditionally before the LDS writes.
__device__ __forceinline__ void stage_gates(const BwdArgs &a, float *sB, float *sR, float *sA, int64_t tok0,
                                            int64_t H, int64_t t0, int nb, int tid) {
  if (tid < nb) {
    const int64_t x = tok0 + (t0 + tid) * H;
    const float bx = a.beta[x];
    const float rx = (a.r ? a.r : a.beta)[x];
    const float ax = (a.alpha ? a.alpha : a.beta)[x];
    sB[tid] = bx;
    sR[tid] = a.r ? rx : 1.0f;
    sA[tid] = a.alpha ? ax : 1.0f;
  }
}

struct P1 {
  float eta, eps, dmin, dmax;
  bool clamp, aware;
};

// One preconditioner step on wave 0's two coordinates per lane (lane, lane +
// 64): returns the step scalar c and leaves y (before the clamp) in y[].
__device__ __forceinline__ float p1_step(const P1 &p, const float (&d)[2], const float (&k)[2], float beta, float r,
                                         float (&y)[2], float *norm_out = nullptr, float *align_out = nullptr) {
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
  if (norm_out) *norm_out = norm;
  if (align_out) *align_out = align;
  return c;
}

__device__ __forceinline__ float p1_clip(const P1 &p, float y) {
  return p.clamp ? fminf(fmaxf(y, p.dmin), p.dmax) : y;
}

// ===================================================================== record
// One workgroup per (b,h) and slice of 32 value rows; KM = ceil(K / 32):
// lane (row i of S, l8) holds S[i][32 m + 4 l8 + c].
template <typename TIn, int KM>
__global__ __launch_bounds__(256) void bwd_record_kernel(BwdArgs a) {
  __shared__ float sK[BT][BP], sKt[BT][BP], sV[BT][BP], sU[BT][VS];
  __shared__ float sB[BT], sR[BT], sA[BT];
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  const int NQ = a.nq;
  const int64_t seq = blockIdx.x / NQ;
  const int q = (int)(blockIdx.x - seq * NQ);
  const int64_t H = a.H, T = a.T, K = a.K, V = a.V;
  const int64_t b = seq / H, h = seq - b * H;
  const int rl = tid >> 3, l8 = tid & 7;
  const int row = VS * q + rl;
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
    if (active) {
      float *dst = a.ck + ((seq * (NB + 1) + blk) * V + row) * K;
#pragma unroll
      for (int m = 0; m < KM; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 32 * m + 4 * l8 + c;
          if (j < K) dst[j] = S[m][c];
        }
    }
    if (q == 0 && tid < 64) {
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
    stage_gates(a, sB, sR, sA, tok0, H, t0, nb, tid);
    stage2<8, BP, BP>(RowSrc<TIn>{kp, K, 0, K, &sK[0][0], 1.0f}, RowSrc<TIn>{vp, V, 0, V, &sV[0][0], 1.0f},
                      tok0, H, t0, nb, tid, nt);
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
      if (l8 == 0) sU[t][rl] = u;
      const float bu = sB[t] * u;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const floatx4 wv = lds4(&sKt[t][32 * m + 4 * l8]);
#pragma unroll
        for (int c = 0; c < 4; ++c) S[m][c] = fmaf(bu, wv[c], S[m][c]);
      }
    }
    __syncthreads();
    for (int e = tid; e < nb * VS; e += nt) {
      const int t = e / VS, il = e - t * VS;
      if (VS * q + il < V) a.u[(tok0 + (t0 + t) * H) * V + VS * q + il] = sU[t][il];
    }
    // the next block's staging writes sK, sV, sB, sR, sA, read last before
    // the barrier above; sKt and sU are rewritten after two more barriers
  }
  record_state(NB);
}

// ============================================================ phase-2 reverse
// One workgroup per (b,h) and slice of 32 value columns, the state held
// transposed: lane (key row j, l8) holds S[c0 + 4 l8 + c][j], c < 4, and the
// same slots of G.
template <typename TIn, bool OF32>
__global__ __launch_bounds__(1024) void bwd_p2_kernel(BwdArgs a) {
  __shared__ float sQ[BT][BP], sK[BT][BP], sKt[BT][BP], sDo[BT][VS], sU[BT][VS];
  __shared__ float sDq[BT][BP], sDkt[BT][BP], sDkr[BT][BP], sDv[BT][VS];
  __shared__ float sWp[2][16][VS];
  __shared__ float sDa[BT][16], sDb[BT];
  __shared__ float sB[BT], sR[BT], sA[BT];
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6;
  const int nwaves = nt >> 6;
  const int NQ = a.nq;
  const int64_t seq = blockIdx.x / NQ;
  const int q = (int)(blockIdx.x - seq * NQ);
  const int64_t H = a.H, T = a.T, K = a.K, V = a.V;
  const int64_t b = seq / H, h = seq - b * H;
  const int c0 = VS * q;
  const int ncol = (int)(V - c0 < VS ? V - c0 : VS);
  const int row = tid >> 3, l8 = tid & 7;  // row = key index j
  const bool active = row < K;
  const int64_t NB = (T + BT - 1) / BT;
  const int64_t tok = a.B * T * H;
  const P1 p{a.eta, a.eps, a.d_min, a.d_max, a.clamp != 0, a.beta_aware != 0};
  const bool gated = a.alpha != nullptr;
  const float qs = a.q_scale;

  float G[4], S[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int il = 4 * l8 + c;
    G[c] = (a.dS && active && il < ncol) ? a.dS[(seq * V + c0 + il) * K + row] : 0.0f;
  }

  const TIn *qp = static_cast<const TIn *>(a.q);
  const TIn *kp = static_cast<const TIn *>(a.k);
  const TIn *dop = static_cast<const TIn *>(a.dout);
  const int64_t tok0 = b * T * H + h;

  for (int64_t blk = NB - 1; blk >= 0; --blk) {
    const int64_t t0 = blk * BT;
    const int nb = (int)(T - t0 < BT ? T - t0 : BT);
    __syncthreads();  // the previous block's write-out is done with the LDS
    // the slice's state after the block's last token: loads clamped in
    // bounds and issued together, masked after
    {
      const float *src = a.ck + (seq * (NB + 1) + blk + 1) * V * K + (active ? row : K - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int il = 4 * l8 + c;
        S[c] = src[(uint32_t)((c0 + (il < ncol ? il : ncol - 1)) * K)];
      }
    }
    stage_gates(a, sB, sR, sA, tok0, H, t0, nb, tid);
    stage2<2, BP, BP>(RowSrc<TIn>{qp, K, 0, K, &sQ[0][0], qs}, RowSrc<TIn>{kp, K, 0, K, &sK[0][0], 1.0f}, tok0,
                      H, t0, nb, tid, nt);
    stage2<1, VS, VS>(RowSrc<TIn>{dop, V, c0, ncol, &sDo[0][0], 1.0f},
                      RowSrc<float>{a.u, V, c0, ncol, &sU[0][0], 1.0f}, tok0, H, t0, nb, tid, nt);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (!(active && 4 * l8 + c < ncol)) S[c] = 0.0f;
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
      // readout: G += q_scale dout q^T, dq partial = S^T dout
      const floatx4 dov = lds4(&sDo[t][4 * l8]);
      float pdq = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        G[c] = fmaf(qj, dov[c], G[c]);
        pdq = fmaf(S[c], dov[c], pdq);
      }
      pdq = group8_sum(pdq);
      // w = G k~ over key rows: across the lanes of a wave, then its waves.
      // Each wave sums the waves' partials itself, so one barrier per token
      // suffices; the partials alternate between two buffers by token.
      const int par = t & 1;
      {
        floatx4 x;
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = rows8_sum(G[c] * ktj);
        if (lane < 8) *reinterpret_cast<floatx4 *>(&sWp[par][wv][4 * l8]) = x;
      }
      __syncthreads();
      floatx4 wvv = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int w2 = 0; w2 < nwaves; ++w2) wvv += lds4(&sWp[par][w2][4 * l8]);
      const floatx4 uv = lds4(&sU[t][4 * l8]);
      if (wv == 0) {
        // w for this lane's columns, dv and the slice's part of
        // dbeta = u . w (u is zero past the slice; 8 row groups repeat it)
        float pb = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) pb = fmaf(uv[c], wvv[c], pb);
        if (lane < 8) *reinterpret_cast<floatx4 *>(&sDv[t][4 * l8]) = bt * wvv;
        pb = group8_sum(pb);
        if (lane == 0) sDb[t] = pb;
      }
      // dk~ = beta G^T u; the state before the write; dk_read = -beta Sb^T w
      float pdkt = 0.0f, pdkr = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pdkt = fmaf(G[c], uv[c], pdkt);
        S[c] = fmaf(-bt * ktj, uv[c], S[c]);  // Sb
        pdkr = fmaf(S[c], wvv[c], pdkr);
        G[c] = fmaf(-bt * kj, wvv[c], G[c]);  // dSb
      }
      pdkt = group8_sum(pdkt);
      pdkr = group8_sum(pdkr);
      if (active && l8 == 0) {
        sDq[t][row] = pdq;
        sDkt[t][row] = bt * pdkt;
        sDkr[t][row] = -bt * pdkr;
      }
      // decay: S_{t-1} = Sb / alpha, dalpha = <dSb, S_{t-1}>, G = alpha dSb
      if (gated) {
        const float at = sA[t], inv = 1.0f / at;
        float pda = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          S[c] *= inv;
          pda = fmaf(G[c], S[c], pda);
          G[c] *= at;
        }
        pda = wave_sum(pda);
        if (lane == 0) sDa[t][wv] = pda;
      }
    }
    __syncthreads();
    // write the block's gradients: the slice's partials (fp32) and its dv
    for (int e = tid; e < nb * (int)K; e += nt) {
      const int t = e / (int)K, j = e - t * (int)K;
      const int64_t o = ((int64_t)q * tok + tok0 + (t0 + t) * H) * K + j;
      a.dqp[o] = sDq[t][j];
      a.dktp[o] = sDkt[t][j];
      a.dkrp[o] = sDkr[t][j];
    }
    for (int e = tid; e < nb * VS; e += nt) {
      const int t = e / VS, il = e - t * VS;
      if (il < ncol) store_out_t<TIn, OF32>(a.dv, (tok0 + (t0 + t) * H) * V + c0 + il, sDv[t][il]);
    }
    if (tid < nb) {
      const int64_t x = (int64_t)q * tok + tok0 + (t0 + tid) * H;
      a.dbp[x] = sDb[tid];
      if (gated) {
        float da = 0.0f;
        for (int w2 = 0; w2 < nwaves; ++w2) da += sDa[tid][w2];
        a.dap[x] = da;
      }
    }
  }
  if (a.dS0 && active) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int il = 4 * l8 + c;
      if (il < ncol) a.dS0[(seq * V + c0 + il) * K + row] = G[c];
    }
  }
}

// ============================================================ phase-1 reverse
// 640 lanes per (b,h): wave 0 runs the sweep over a block (d in VGPRs, two
// coordinates per lane) while waves 1-8 stage the next block (two waves each:
// keys; dk~ and the read-key part, each summed over the value slices; dq,
// summed, scaled and stored) and wave 9 its gates (and dalpha, summed and
// stored), into the other half of a double buffer.
template <typename TIn, bool OF32>
__global__ __launch_bounds__(640) void bwd_p1_kernel(BwdArgs a) {
  __shared__ float sK[2][BT][BP], sDkt[2][BT][BP], sDkr[2][BT][BP];
  __shared__ float sB[2][BT], sR[2][BT], sDb[2][BT];
  __shared__ float sD[BT][BP], sC[BT], sN[BT], sAl[BT];  // wave 0 only
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t seq = blockIdx.x;
  const int64_t H = a.H, T = a.T, K = a.K;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t NB = (T + BT - 1) / BT;
  const int64_t tok = a.B * T * H;
  const int NQ = a.nq;
  const P1 p{a.eta, a.eps, a.d_min, a.d_max, a.clamp != 0, a.beta_aware != 0};
  const TIn *kp = static_cast<const TIn *>(a.k);
  const int64_t tok0 = b * T * H + h;

  auto stage = [&](int64_t blk, int buf) {
    const int64_t t0 = blk * BT;
    const int nb = (int)(T - t0 < BT ? T - t0 : BT);
    const int grp = (wv - 1) >> 1;  // 0 k, 1 dk~, 2 read-key part, 3 dq, 4 gates
    const int gt = tid - 64 - 128 * grp;
    if (grp < 4) {
      float x[16];
      if (grp == 0) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = gt + 128 * u, t = e >> 7, j = e & 127;
          const int64_t tr = tok0 + (t0 + (t < nb ? t : nb - 1)) * H;
          x[u] = to_f32(kp[tr * K + (j < K ? j : K - 1)]);
        }
      } else {
        const float *src = grp == 1 ? a.dktp : (grp == 2 ? a.dkrp : a.dqp);
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = 0.0f;
        for (int qq = 0; qq < NQ; ++qq) {
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int e = gt + 128 * u, t = e >> 7, j = e & 127;
            const int64_t tr = tok0 + (t0 + (t < nb ? t : nb - 1)) * H;
            x[u] += src[((int64_t)qq * tok + tr) * K + (j < K ? j : K - 1)];
          }
        }
      }
      if (grp == 3) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = gt + 128 * u, t = e >> 7, j = e & 127;
          if (j < K && t < nb) store_out_t<TIn, OF32>(a.dq, (tok0 + (t0 + t) * H) * K + j, a.q_scale * x[u]);
        }
      } else {
        float(*dst)[BP] = grp == 0 ? sK[buf] : (grp == 1 ? sDkt[buf] : sDkr[buf]);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = gt + 128 * u, t = e >> 7, j = e & 127;
          dst[t][j] = (j < K && t < nb) ? x[u] : 0.0f;
        }
      }
    } else if (gt < nb) {
      const int64_t x = tok0 + (t0 + gt) * H;
      const float bx = a.beta[x], rx = (a.r ? a.r : a.beta)[x];
      float pb = 0.0f, pa = 0.0f;
      for (int qq = 0; qq < NQ; ++qq) {
        pb += a.dbp[(int64_t)qq * tok + x];
        if (a.alpha) pa += a.dap[(int64_t)qq * tok + x];
      }
      sB[buf][gt] = bx;
      sR[buf][gt] = a.r ? rx : 1.0f;
      sDb[buf][gt] = pb;
      if (a.dalpha) a.dalpha[x] = pa;
    }
  };

  float g[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t j = lane + 64 * e;
    g[e] = (a.dd && j < K) ? a.dd[seq * K + j] : 0.0f;
  }
  if (NB > 0 && wv > 0) stage(NB - 1, 0);
  __syncthreads();
  for (int64_t blk = NB - 1; blk >= 0; --blk) {
    const int buf = (int)((NB - 1 - blk) & 1);
    if (wv == 0) {
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
        const float k[2] = {sK[buf][t][lane], sK[buf][t][lane + 64]};
        sD[t][lane] = d[0];
        sD[t][lane + 64] = d[1];
        float y[2], nr, al;
        const float c = p1_step(p, d, k, sB[buf][t], sR[buf][t], y, &nr, &al);
        if (lane == 0) {
          sC[t] = c;
          sN[t] = nr;
          sAl[t] = al;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) d[e] = lane + 64 * e < K ? p1_clip(p, y[e]) : 0.0f;
      }
      for (int t = nb - 1; t >= 0; --t) {
        const int64_t tr = tok0 + (t0 + t) * H;
        const float bt = sB[buf][t], rt = sR[buf][t], c = sC[t];
        const float bpr = p.aware ? bt : 1.0f;
        float dv[2], k[2], s[2], gy[2], dkt[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          dv[e] = sD[t][lane + 64 * e];
          k[e] = sK[buf][t][lane + 64 * e];
          s[e] = k[e] * k[e];
          const float y = fmaf(c, s[e], rt * dv[e]);
          // branch-free on purpose: with a short-circuit || on the uniform
          // clamp flag, the compiler dropped g from the passing lanes
          const bool pass = (y >= p.dmin) & (y <= p.dmax) | !p.clamp;
          gy[e] = pass ? g[e] : 0.0f;
          dkt[e] = sDkt[buf][t][lane + 64 * e];
        }
        const float nraw = sN[t], align = sAl[t];
        const float gc = wave_sum(fmaf(s[0], gy[0], s[1] * gy[1]));
        const float grr = wave_sum(fmaf(dv[0], gy[0], dv[1] * gy[1]));
        const float n = fmaxf(nraw, p.eps);
        const float dca = -p.eta * bpr * bpr / n;        // dc / d<d, s>
        const float dcn = nraw > p.eps ? -c / n : 0.0f;  // dc / dn
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int64_t j = lane + 64 * e;
          const float ds = fmaf(c, gy[e], gc * fmaf(dca, dv[e], dcn));
          if (j < K) {
            const float dk = sDkr[buf][t][lane + 64 * e] + fmaf(2.0f * k[e], ds, dkt[e] * dv[e]);
            store_out_t<TIn, OF32>(a.dk, tr * K + j, dk);
          }
          g[e] = j < K ? fmaf(dkt[e], k[e], fmaf(rt, gy[e], dca * s[e] * gc)) : 0.0f;
        }
        if (lane == 0) {
          float db = sDb[buf][t];
          if (p.aware) db += gc * p.eta * (1.0f - 2.0f * bpr * align) / n;
          a.dbeta[tr] = db;
          if (a.dr) a.dr[tr] = grr;
        }
      }
    } else if (blk > 0) {
      stage(blk - 1, buf ^ 1);
    }
    __syncthreads();
  }
  if (a.dd1 && wv == 0) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t j = lane + 64 * e;
      if (j < K) a.dd1[seq * K + j] = g[e];
    }
  }
}

template <typename TIn>
hipError_t launch_typed(const BwdArgs &a, hipStream_t s) {
  const int64_t nseq = a.B * a.H;
  const dim3 gsplit((unsigned)(nseq * a.nq)), grid((unsigned)nseq);
  const dim3 bp2((unsigned)(((8 * a.K + 63) / 64) * 64));
  switch ((a.K + 31) / 32) {
    case 1: hipLaunchKernelGGL((bwd_record_kernel<TIn, 1>), gsplit, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((bwd_record_kernel<TIn, 2>), gsplit, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((bwd_record_kernel<TIn, 3>), gsplit, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((bwd_record_kernel<TIn, 4>), gsplit, dim3(256), 0, s, a); break;
  }
  prof_mark(s, "bwd_record_kernel");
  // float32 gradients for bf16 inputs: a variant of each reverse kernel
  const bool f32 = a.o_f32 && sizeof(TIn) == 2;
  if (f32)
    hipLaunchKernelGGL((bwd_p2_kernel<TIn, true>), gsplit, bp2, 0, s, a);
  else
    hipLaunchKernelGGL((bwd_p2_kernel<TIn, false>), gsplit, bp2, 0, s, a);
  prof_mark(s, "bwd_p2_kernel");
  if (f32)
    hipLaunchKernelGGL((bwd_p1_kernel<TIn, true>), grid, dim3(640), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_p1_kernel<TIn, false>), grid, dim3(640), 0, s, a);
  prof_mark(s, "bwd_p1_kernel");
  return hipGetLastError();
}

}  // namespace

size_t bwd_work_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t NB = (size_t)((T + BT - 1) / BT), NQ = (size_t)((V + VS - 1) / VS);
  const size_t BH = (size_t)(B * H), tok = (size_t)(B * T * H);
  return al(tok * V * 4) + al(BH * (NB + 1) * V * K * 4) + al(BH * (NB + 1) * K * 4) + 3 * al(NQ * tok * K * 4) +
         2 * al(NQ * tok * 4);
}

void bwd_work_layout(BwdArgs &a, void *base) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t NB = (size_t)((a.T + BT - 1) / BT), NQ = (size_t)((a.V + VS - 1) / VS);
  const size_t BH = (size_t)(a.B * a.H), tok = (size_t)(a.B * a.T * a.H);
  char *p = static_cast<char *>(base);
  a.nq = (int)NQ;
  a.u = reinterpret_cast<float *>(p);
  p += al(tok * a.V * 4);
  a.ck = reinterpret_cast<float *>(p);
  p += al(BH * (NB + 1) * a.V * a.K * 4);
  a.dck = reinterpret_cast<float *>(p);
  p += al(BH * (NB + 1) * a.K * 4);
  a.dqp = reinterpret_cast<float *>(p);
  p += al(NQ * tok * a.K * 4);
  a.dktp = reinterpret_cast<float *>(p);
  p += al(NQ * tok * a.K * 4);
  a.dkrp = reinterpret_cast<float *>(p);
  p += al(NQ * tok * a.K * 4);
  a.dbp = reinterpret_cast<float *>(p);
  p += al(NQ * tok * 4);
  a.dap = reinterpret_cast<float *>(p);
}

hipError_t launch_bwd(const BwdArgs &a, bool is_bf16, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  return is_bf16 ? launch_typed<bf16>(a, s) : launch_typed<float>(a, s);
}

}  // namespace osdn
