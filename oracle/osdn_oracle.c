/*
 * OSDN CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, sequential fp64 implementation of the OSDN forward pass, written
 * from the paper "OSDN: Improving Delta Rule with Provable Online Preconditioning
 * in Linear Attention" (Zhou, Li, Liu, Lin, Ge, Ye; arXiv:2605.13473):
 *
 *   phase 1  -- the online preconditioner sweep: Section 4.2, Eq.(4) and
 *               Algorithm 1; the retention-gated (APF) form of Section 4.4,
 *               Eq.(7); the non-beta-aware form of Appendix B (Eq.(12) text).
 *   phase 2  -- the token-by-token delta rule with the write key replaced by
 *               k~_t = d_t (.) k_t: Section 4.1 Eq.(2) / Section 4.3 Eq.(5),
 *               Appendix C Algorithm 2 part (2b); readout o_t = S_t q_t
 *               (Section 3); the Gated DeltaNet variant with the post-gate
 *               residual of Appendix B.1.
 *   OSKDA    -- the Kimi Delta Attention backbone with online scaling,
 *               Appendix B.2 and Table 3: K x V state, channel-wise decay,
 *               preconditioned key on the left (storage) side.
 *   vector retention -- diag(r_t) in place of the scalar r_t of Eq.(7),
 *               Appendix A.5 Proposition A.3.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this library.  It shares no code with the GPU path.
 *
 * Layouts: sequence tensors are [B,T,H,X] row-major, per-(b,h) vectors [B,H,X],
 * the memory state is [B,H,V,K] (V x K per head, Section 3).  All values fp64.
 * Every function returns 0 on success and a negative code on a bad argument.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static size_t at_bthx(int64_t b, int64_t t, int64_t h, int64_t x,
                      int64_t T, int64_t H, int64_t X) {
  return (size_t)(((b * T + t) * H + h) * X + x);
}

static size_t at_bth(int64_t b, int64_t t, int64_t h, int64_t T, int64_t H) {
  return (size_t)((b * T + t) * H + h);
}

int osdn_oracle_version(void) { return 1; }

/*
 * Phase 1 (Algorithm 1 with the per-step box clamp of Algorithm 2 line 12 and
 * the retention r of Eq.(7)).  For every (b,h), starting from d = d1 (ones when
 * d1 is NULL; d1 itself is not clamped):
 *
 *   k~_t   = d (.) k_t                       (emitted before the update)
 *   s      = k_t (.) k_t,  n = max(sum(s), eps)
 *   b'     = beta_t if beta_aware else 1
 *   c      = eta * b' * (1 - b' * <d, s>) / n
 *   d      = r_t * d + c * s                  (r_t = 1 when r is NULL;
 *                                             r_t a vector when r_per_key)
 *   d      = min(max(d, d_min), d_max)        (only when clamp != 0)
 *
 * r is [B,T,H] (one retention per token and head, Eq.(7)) or, with r_per_key,
 * [B,T,H,K] (the vector-retention extension diag(r_t) of Proposition A.3).
 * k_tilde [B,T,H,K] receives every k~_t, d_out [B,H,K] receives d_{T+1}.
 * d_traj (nullable, [B,H,T+1,K]) receives d_1 .. d_{T+1}.
 */
int osdn_oracle_precond_scan(int64_t B, int64_t T, int64_t H, int64_t K,
                             const double *k, const double *beta,
                             const double *r, int r_per_key, const double *d1, double eta,
                             double d_min, double d_max, int clamp, double eps,
                             int beta_aware, double *k_tilde, double *d_out,
                             double *d_traj, int threads) {
  if (B < 0 || T < 0 || H < 0 || K <= 0 || !k || !beta || !k_tilde || !d_out)
    return -1;
  if (threads <= 0) threads = 1;
  int64_t nseq = B * H;
#pragma omp parallel for num_threads(threads) schedule(dynamic, 1)
  for (int64_t bh = 0; bh < nseq; ++bh) {
    int64_t b = bh / H, h = bh % H;
    double *d = (double *)malloc(sizeof(double) * (size_t)K);
    double *s = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t i = 0; i < K; ++i) d[i] = d1 ? d1[bh * K + i] : 1.0;
    for (int64_t t = 0; t < T; ++t) {
      const double *kt = k + at_bthx(b, t, h, 0, T, H, K);
      double *out = k_tilde + at_bthx(b, t, h, 0, T, H, K);
      if (d_traj)
        for (int64_t i = 0; i < K; ++i)
          d_traj[((size_t)bh * (size_t)(T + 1) + (size_t)t) * (size_t)K + i] = d[i];
      /* emit the write key with the current d (Algorithm 1, before the update) */
      for (int64_t i = 0; i < K; ++i) out[i] = d[i] * kt[i];
      double norm = 0.0, align = 0.0;
      for (int64_t i = 0; i < K; ++i) {
        s[i] = kt[i] * kt[i];
        norm += s[i];
        align += d[i] * s[i];
      }
      double n = norm > eps ? norm : eps;
      double bt = beta[at_bth(b, t, h, T, H)];
      double bp = beta_aware ? bt : 1.0;
      double c = eta * bp * (1.0 - bp * align) / n;
      for (int64_t i = 0; i < K; ++i) {
        double rt = 1.0;
        if (r) rt = r_per_key ? r[at_bthx(b, t, h, i, T, H, K)] : r[at_bth(b, t, h, T, H)];
        double x = rt * d[i] + c * s[i];
        if (clamp) {
          if (x < d_min) x = d_min;
          if (x > d_max) x = d_max;
        }
        d[i] = x;
      }
    }
    for (int64_t i = 0; i < K; ++i) d_out[bh * K + i] = d[i];
    if (d_traj)
      for (int64_t i = 0; i < K; ++i)
        d_traj[((size_t)bh * (size_t)(T + 1) + (size_t)T) * (size_t)K + i] = d[i];
    free(d);
    free(s);
  }
  return 0;
}

/*
 * Phase 2, token by token (Algorithm 2 part (2b) / Eq.(5); Gated DeltaNet with
 * the post-gate residual of Appendix B.1 when alpha is given).  For every (b,h),
 * starting from S = S0 (zeros when S0 is NULL), S in R^{V x K}:
 *
 *   Sb  = alpha_t * S   (Sb = S when alpha is NULL)
 *   u_t = v_t - Sb k_t                 (read with the physical key)
 *   S   = Sb + beta_t u_t k~_t^T       (write with the preconditioned key)
 *   o_t = S (q_scale * q_t)            (readout after the write, Section 3)
 *
 * o [B,T,H,V], S_out [B,H,V,K].  Optional outputs (nullable):
 *   S_traj [B,H,T+1,V,K]  the states S_0 .. S_T;
 *   u_out  [B,T,H,V]      the pre-write residuals u_t.
 */
int osdn_oracle_delta_rule(int64_t B, int64_t T, int64_t H, int64_t K,
                           int64_t V, const double *q, const double *k,
                           const double *k_tilde, const double *v,
                           const double *beta, const double *alpha,
                           const double *S0, double q_scale, double *o,
                           double *S_out, double *S_traj, double *u_out,
                           int threads) {
  if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || !q || !k || !k_tilde ||
      !v || !beta || !o || !S_out)
    return -1;
  if (threads <= 0) threads = 1;
  int64_t nseq = B * H;
  size_t VK = (size_t)(V * K);
#pragma omp parallel for num_threads(threads) schedule(dynamic, 1)
  for (int64_t bh = 0; bh < nseq; ++bh) {
    int64_t b = bh / H, h = bh % H;
    double *S = (double *)malloc(sizeof(double) * VK);
    double *u = (double *)malloc(sizeof(double) * (size_t)V);
    for (size_t e = 0; e < VK; ++e) S[e] = S0 ? S0[(size_t)bh * VK + e] : 0.0;
    if (S_traj)
      for (size_t e = 0; e < VK; ++e) S_traj[(size_t)bh * (size_t)(T + 1) * VK + e] = S[e];
    for (int64_t t = 0; t < T; ++t) {
      const double *qt = q + at_bthx(b, t, h, 0, T, H, K);
      const double *kt = k + at_bthx(b, t, h, 0, T, H, K);
      const double *wt = k_tilde + at_bthx(b, t, h, 0, T, H, K);
      const double *vt = v + at_bthx(b, t, h, 0, T, H, V);
      double bt = beta[at_bth(b, t, h, T, H)];
      if (alpha) {
        double at = alpha[at_bth(b, t, h, T, H)];
        for (size_t e = 0; e < VK; ++e) S[e] *= at;
      }
      for (int64_t i = 0; i < V; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < K; ++j) acc += S[i * K + j] * kt[j];
        u[i] = vt[i] - acc;
      }
      if (u_out)
        for (int64_t i = 0; i < V; ++i) u_out[at_bthx(b, t, h, i, T, H, V)] = u[i];
      for (int64_t i = 0; i < V; ++i)
        for (int64_t j = 0; j < K; ++j) S[i * K + j] += bt * u[i] * wt[j];
      double *ot = o + at_bthx(b, t, h, 0, T, H, V);
      for (int64_t i = 0; i < V; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < K; ++j) acc += S[i * K + j] * (q_scale * qt[j]);
        ot[i] = acc;
      }
      if (S_traj)
        for (size_t e = 0; e < VK; ++e)
          S_traj[((size_t)bh * (size_t)(T + 1) + (size_t)(t + 1)) * VK + e] = S[e];
    }
    for (size_t e = 0; e < VK; ++e) S_out[(size_t)bh * VK + e] = S[e];
    free(S);
    free(u);
  }
  return 0;
}

/*
 * Phase 2 of OSKDA, token by token (Appendix B.2, the online-scaled KDA row of
 * Table 3).  The state keeps KDA's own K x V convention: S in R^{K x V} per
 * (b,h), starting from S0 [B,H,K,V] (zeros when NULL).  For every token:
 *
 *   Sb  = Diag(alpha_t) S        (row i scaled by alpha_t[i]; Sb = S when
 *                                 alpha is NULL)
 *   u_t = v_t - Sb^T k_t         (residual read with the physical key)
 *   S   = Sb + beta_t k~_t u_t^T (preconditioned key on the storage side)
 *   o_t = S^T (q_scale * q_t)
 *
 * alpha [B,T,H,K]; o [B,T,H,V]; S_out [B,H,K,V].
 */
int osdn_oracle_kda_rule(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                         const double *q, const double *k, const double *k_tilde,
                         const double *v, const double *beta, const double *alpha,
                         const double *S0, double q_scale, double *o,
                         double *S_out, int threads) {
  if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || !q || !k || !k_tilde ||
      !v || !beta || !o || !S_out)
    return -1;
  if (threads <= 0) threads = 1;
  int64_t nseq = B * H;
  size_t KV = (size_t)(K * V);
#pragma omp parallel for num_threads(threads) schedule(dynamic, 1)
  for (int64_t bh = 0; bh < nseq; ++bh) {
    int64_t b = bh / H, h = bh % H;
    double *S = (double *)malloc(sizeof(double) * KV);
    double *u = (double *)malloc(sizeof(double) * (size_t)V);
    for (size_t e = 0; e < KV; ++e) S[e] = S0 ? S0[(size_t)bh * KV + e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const double *qt = q + at_bthx(b, t, h, 0, T, H, K);
      const double *kt = k + at_bthx(b, t, h, 0, T, H, K);
      const double *wt = k_tilde + at_bthx(b, t, h, 0, T, H, K);
      const double *vt = v + at_bthx(b, t, h, 0, T, H, V);
      double bt = beta[at_bth(b, t, h, T, H)];
      if (alpha) {
        const double *at = alpha + at_bthx(b, t, h, 0, T, H, K);
        for (int64_t i = 0; i < K; ++i)
          for (int64_t j = 0; j < V; ++j) S[i * V + j] *= at[i];
      }
      for (int64_t j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * kt[i];
        u[j] = vt[j] - acc;
      }
      for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < V; ++j) S[i * V + j] += bt * wt[i] * u[j];
      double *ot = o + at_bthx(b, t, h, 0, T, H, V);
      for (int64_t j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < K; ++i) acc += S[i * V + j] * (q_scale * qt[i]);
        ot[j] = acc;
      }
    }
    for (size_t e = 0; e < KV; ++e) S_out[(size_t)bh * KV + e] = S[e];
    free(S);
    free(u);
  }
  return 0;
}

/*
 * Per-token diagnostics along the trajectory (Lemma 4.1 / Eq.(3), Corollary A.2,
 * Theorem D.7 proof).  Inputs are the phase-2 inputs plus the oracle outputs
 * S_traj [B,H,T+1,V,K] and u [B,T,H,V].  For every token it writes 6 values to
 * diag [B,T,H,6]:
 *   [0] a_t    = beta_t <d_t, k_t^2> = beta_t <k~_t, k_t>
 *   [1] n_t    = ||k_t||^2
 *   [2] f_pre  = 0.5 ||u_t||^2            (loss of the pre-write reference state)
 *   [3] f_post = 0.5 ||S_t k_t - v_t||^2  (loss after the write)
 *   [4] q_t    = f_post / f_pre, defined as 1 when u_t = 0 (Theorem D.7 proof)
 *   [5] h_t    = ((1 - a_t)^2 - 1) / (2 n_t), defined as 0 when u_t = 0 (Eq.(18))
 */
int osdn_oracle_diagnostics(int64_t B, int64_t T, int64_t H, int64_t K,
                            int64_t V, const double *k, const double *k_tilde,
                            const double *v, const double *beta,
                            const double *S_traj, const double *u,
                            double *diag) {
  if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || !k || !k_tilde || !v ||
      !beta || !S_traj || !u || !diag)
    return -1;
  size_t VK = (size_t)(V * K);
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h) {
      int64_t bh = b * H + h;
      for (int64_t t = 0; t < T; ++t) {
        const double *kt = k + at_bthx(b, t, h, 0, T, H, K);
        const double *wt = k_tilde + at_bthx(b, t, h, 0, T, H, K);
        const double *vt = v + at_bthx(b, t, h, 0, T, H, V);
        const double *ut = u + at_bthx(b, t, h, 0, T, H, V);
        const double *St = S_traj + ((size_t)bh * (size_t)(T + 1) + (size_t)(t + 1)) * VK;
        double bt = beta[at_bth(b, t, h, T, H)];
        double align = 0.0, n = 0.0;
        for (int64_t j = 0; j < K; ++j) {
          align += wt[j] * kt[j];
          n += kt[j] * kt[j];
        }
        double a = bt * align;
        double fpre = 0.0, fpost = 0.0;
        for (int64_t i = 0; i < V; ++i) {
          fpre += ut[i] * ut[i];
          double acc = 0.0;
          for (int64_t j = 0; j < K; ++j) acc += St[i * K + j] * kt[j];
          double e = acc - vt[i];
          fpost += e * e;
        }
        fpre *= 0.5;
        fpost *= 0.5;
        double *dg = diag + at_bthx(b, t, h, 0, T, H, 6);
        dg[0] = a;
        dg[1] = n;
        dg[2] = fpre;
        dg[3] = fpost;
        dg[4] = fpre > 0.0 ? fpost / fpre : 1.0;
        dg[5] = (fpre > 0.0 && n > 0.0) ? ((1.0 - a) * (1.0 - a) - 1.0) / (2.0 * n) : 0.0;
      }
    }
  return 0;
}
