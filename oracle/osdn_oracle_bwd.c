/*
 * OSDN CPU oracle, backward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, sequential fp64 reverse-mode differentiation of the OSDN forward
 * pass of osdn_oracle.c, written from the recurrences of "OSDN: Improving Delta
 * Rule with Provable Online Preconditioning in Linear Attention"
 * (arXiv:2605.13473): phase 1 is the preconditioner step of Section 4.2 Eq.(4)
 * with the retention of Section 4.4 Eq.(7) and the box clamp of Appendix C
 * Algorithm 2; phase 2 is the delta rule with write key k~_t = d_t (.) k_t of
 * Section 4.3 Eq.(5), gated as in Appendix B.1; the backward sweep through the
 * clamped preconditioner recurrence is the one Section 4.5 describes (the
 * gradient reaches d through k~ = d (.) k and flows back through each step).
 *
 * Forward, per (b,h), t = 1..T (as in osdn_oracle.c):
 *   k~_t = d_t (.) k_t;  s = k_t^2;  n = max(sum s, eps);  b' = beta_t or 1
 *   a = <d_t, s>;  c = eta b' (1 - b' a) / n;  y = r_t d_t + c s
 *   d_{t+1} = clip(y, d_min, d_max)  (y when clamp == 0)
 *   Sb_t = alpha_t S_{t-1};  u_t = v_t - Sb_t k_t;  S_t = Sb_t + beta_t u_t k~_t^T
 *   o_t = q_scale S_t q_t
 * For the loss L with dL/do_t = dout_t, dL/dS_T = dS, dL/dd_{T+1} = dd, the
 * reverse sweep, with G = dL/dS_t (starting from dS):
 *   G += q_scale dout_t q_t^T;           dq_t  = q_scale S_t^T dout_t
 *   w = G k~_t;  dv_t = beta_t w;        dbeta_t = u_t . w  (+ phase 1 below)
 *   dk~_t = beta_t G^T u_t;              dk_t  = -beta_t Sb_t^T w  (+ phase 1)
 *   dSb = G - beta_t w k_t^T;            dalpha_t = <dSb, S_{t-1}>;  G = alpha_t dSb
 * then, with g = dL/dd_{t+1} (starting from dd) and m the clamp's pass mask
 * (1 where d_min <= y <= d_max, or everywhere without clamp):
 *   gy = m (.) g;  gc = s . gy;          dr_t = d_t . gy
 *   ds = c gy - gc eta b'^2 / n d_t - [sum s > eps] gc c / n
 *   dk_t += 2 k_t (.) ds + dk~_t (.) d_t
 *   dbeta_t += gc eta (1 - 2 b' a) / n   (beta-aware only)
 *   g = dk~_t (.) k_t + r_t gy - (eta b'^2 / n) (s . gy) s
 * and finally dS0 = G, dd1 = g.
 *
 * The sweep recomputes the forward states of each 64-token stretch from a
 * stored state at its start (the recomputation repeats the forward arithmetic
 * exactly), so memory stays bounded at long T.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this library.  It shares no code with the GPU path.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define OSDN_ORACLE_BWD_STRETCH 64

static size_t bw_bthx(int64_t b, int64_t t, int64_t h, int64_t x, int64_t T, int64_t H, int64_t X) {
  return (size_t)(((b * T + t) * H + h) * X + x);
}

static size_t bw_bth(int64_t b, int64_t t, int64_t h, int64_t T, int64_t H) {
  return (size_t)((b * T + t) * H + h);
}

/*
 * Inputs as for osdn_oracle_precond_scan / osdn_oracle_delta_rule (r, alpha,
 * d1, S0 nullable).  dout [B,T,H,V] is required; dS [B,H,V,K] and dd [B,H,K]
 * may be NULL (zero).  Outputs dq, dk [B,T,H,K], dv [B,T,H,V], dbeta [B,T,H]
 * are required; dr, dalpha [B,T,H], dd1 [B,H,K], dS0 [B,H,V,K] are written
 * when not NULL.
 */
int osdn_oracle_backward(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                         const double *q, const double *k, const double *v,
                         const double *beta, const double *r, const double *alpha,
                         const double *d1, const double *S0, double eta,
                         double d_min, double d_max, int clamp, double eps,
                         int beta_aware, double q_scale, const double *dout,
                         const double *dS, const double *dd, double *dq, double *dk,
                         double *dv, double *dbeta, double *dr, double *dalpha,
                         double *dd1, double *dS0, int threads) {
  if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || !q || !k || !v || !beta || !dout ||
      !dq || !dk || !dv || !dbeta)
    return -1;
  if (threads <= 0) threads = 1;
  const int64_t nseq = B * H;
  const int64_t CH = OSDN_ORACLE_BWD_STRETCH;
  const int64_t NS = (T + CH - 1) / CH;
  const size_t VK = (size_t)V * (size_t)K;
#pragma omp parallel for num_threads(threads) schedule(dynamic, 1)
  for (int64_t bh = 0; bh < nseq; ++bh) {
    const int64_t b = bh / H, h = bh % H;
    /* ---- phase 1 forward: d_1 .. d_{T+1} */
    double *dtr = (double *)malloc(sizeof(double) * (size_t)(T + 1) * (size_t)K);
    double *s = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t i = 0; i < K; ++i) dtr[i] = d1 ? d1[bh * K + i] : 1.0;
    for (int64_t t = 0; t < T; ++t) {
      const double *kt = k + bw_bthx(b, t, h, 0, T, H, K);
      const double *d = dtr + (size_t)t * (size_t)K;
      double *dn = dtr + (size_t)(t + 1) * (size_t)K;
      const double bt = beta[bw_bth(b, t, h, T, H)];
      const double rt = r ? r[bw_bth(b, t, h, T, H)] : 1.0;
      const double bp = beta_aware ? bt : 1.0;
      double nraw = 0.0, a = 0.0;
      for (int64_t i = 0; i < K; ++i) {
        s[i] = kt[i] * kt[i];
        nraw += s[i];
        a += d[i] * s[i];
      }
      const double n = nraw > eps ? nraw : eps;
      const double c = eta * bp * (1.0 - bp * a) / n;
      for (int64_t i = 0; i < K; ++i) {
        double y = rt * d[i] + c * s[i];
        if (clamp) y = y < d_min ? d_min : (y > d_max ? d_max : y);
        dn[i] = y;
      }
    }

    /* ---- phase 2 forward: the state at the start of every stretch */
    double *ck = (double *)malloc(sizeof(double) * VK * (size_t)(NS + 1));
    double *S = (double *)malloc(sizeof(double) * VK);
    double *u = (double *)malloc(sizeof(double) * (size_t)V);
    double *wk = (double *)malloc(sizeof(double) * (size_t)K);
    for (size_t e = 0; e < VK; ++e) S[e] = S0 ? S0[(size_t)bh * VK + e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      if (t % CH == 0) memcpy(ck + (size_t)(t / CH) * VK, S, sizeof(double) * VK);
      const double *kt = k + bw_bthx(b, t, h, 0, T, H, K);
      const double *vt = v + bw_bthx(b, t, h, 0, T, H, V);
      const double *d = dtr + (size_t)t * (size_t)K;
      const double bt = beta[bw_bth(b, t, h, T, H)];
      if (alpha) {
        const double at = alpha[bw_bth(b, t, h, T, H)];
        for (size_t e = 0; e < VK; ++e) S[e] *= at;
      }
      for (int64_t j = 0; j < K; ++j) wk[j] = d[j] * kt[j];
      for (int64_t i = 0; i < V; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < K; ++j) acc += S[i * K + j] * kt[j];
        u[i] = vt[i] - acc;
      }
      for (int64_t i = 0; i < V; ++i)
        for (int64_t j = 0; j < K; ++j) S[i * K + j] += bt * u[i] * wk[j];
    }

    /* ---- phase 2 reverse, one stretch at a time (states recomputed) */
    double *Sprev = (double *)malloc(sizeof(double) * VK * (size_t)(CH + 1)); /* S_{t-1} of each token, then S_last */
    double *Sbar = (double *)malloc(sizeof(double) * VK * (size_t)CH);
    double *us = (double *)malloc(sizeof(double) * (size_t)V * (size_t)CH);
    double *G = (double *)malloc(sizeof(double) * VK);
    double *dSb = (double *)malloc(sizeof(double) * VK);
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    double *dkt = (double *)malloc(sizeof(double) * (size_t)T * (size_t)K);  /* dL/dk~_t */
    for (size_t e = 0; e < VK; ++e) G[e] = dS ? dS[(size_t)bh * VK + e] : 0.0;
    for (int64_t sidx = NS - 1; sidx >= 0; --sidx) {
      const int64_t t0 = sidx * CH, t1 = (t0 + CH < T) ? t0 + CH : T;
      /* recompute: Sprev[j] = S before token t0 + j, Sbar[j], us[j]; Sprev[t1 - t0] = S after t1 - 1 */
      memcpy(Sprev, ck + (size_t)sidx * VK, sizeof(double) * VK);
      for (int64_t t = t0; t < t1; ++t) {
        const int64_t j = t - t0;
        const double *kt = k + bw_bthx(b, t, h, 0, T, H, K);
        const double *vt = v + bw_bthx(b, t, h, 0, T, H, V);
        const double *d = dtr + (size_t)t * (size_t)K;
        const double bt = beta[bw_bth(b, t, h, T, H)];
        const double at = alpha ? alpha[bw_bth(b, t, h, T, H)] : 1.0;
        const double *Sp = Sprev + (size_t)j * VK;
        double *Sb = Sbar + (size_t)j * VK;
        double *Sn = Sprev + (size_t)(j + 1) * VK;
        double *uj = us + (size_t)j * (size_t)V;
        for (size_t e = 0; e < VK; ++e) Sb[e] = at * Sp[e];
        for (int64_t i = 0; i < V; ++i) {
          double acc = 0.0;
          for (int64_t jj = 0; jj < K; ++jj) acc += Sb[i * K + jj] * kt[jj];
          uj[i] = vt[i] - acc;
        }
        for (int64_t i = 0; i < V; ++i)
          for (int64_t jj = 0; jj < K; ++jj) Sn[i * K + jj] = Sb[i * K + jj] + bt * uj[i] * d[jj] * kt[jj];
      }
      for (int64_t t = t1 - 1; t >= t0; --t) {
        const int64_t j = t - t0;
        const double *qt = q + bw_bthx(b, t, h, 0, T, H, K);
        const double *kt = k + bw_bthx(b, t, h, 0, T, H, K);
        const double *dot = dout + bw_bthx(b, t, h, 0, T, H, V);
        const double *d = dtr + (size_t)t * (size_t)K;
        const double bt = beta[bw_bth(b, t, h, T, H)];
        const double at = alpha ? alpha[bw_bth(b, t, h, T, H)] : 1.0;
        const double *Sp = Sprev + (size_t)j * VK;       /* S_{t-1} */
        const double *St = Sprev + (size_t)(j + 1) * VK; /* S_t */
        const double *Sb = Sbar + (size_t)j * VK;
        const double *uj = us + (size_t)j * (size_t)V;
        double *dqt = dq + bw_bthx(b, t, h, 0, T, H, K);
        double *dkt_read = dk + bw_bthx(b, t, h, 0, T, H, K);
        double *dvt = dv + bw_bthx(b, t, h, 0, T, H, V);
        double *dktil = dkt + (size_t)t * (size_t)K;
        /* readout o_t = q_scale S_t q_t */
        for (int64_t i = 0; i < V; ++i)
          for (int64_t jj = 0; jj < K; ++jj) G[i * K + jj] += q_scale * dot[i] * qt[jj];
        for (int64_t jj = 0; jj < K; ++jj) {
          double acc = 0.0;
          for (int64_t i = 0; i < V; ++i) acc += St[i * K + jj] * dot[i];
          dqt[jj] = q_scale * acc;
        }
        /* write S_t = Sb + beta u k~^T */
        for (int64_t jj = 0; jj < K; ++jj) wk[jj] = d[jj] * kt[jj];
        double db = 0.0;
        for (int64_t i = 0; i < V; ++i) {
          double acc = 0.0;
          for (int64_t jj = 0; jj < K; ++jj) acc += G[i * K + jj] * wk[jj];
          w[i] = acc;
          dvt[i] = bt * acc;
          db += uj[i] * acc;
        }
        dbeta[bw_bth(b, t, h, T, H)] = db;
        for (int64_t jj = 0; jj < K; ++jj) {
          double acc = 0.0;
          for (int64_t i = 0; i < V; ++i) acc += G[i * K + jj] * uj[i];
          dktil[jj] = bt * acc;
        }
        /* residual u = v - Sb k (read with the physical key) */
        for (int64_t jj = 0; jj < K; ++jj) {
          double acc = 0.0;
          for (int64_t i = 0; i < V; ++i) acc += Sb[i * K + jj] * w[i];
          dkt_read[jj] = -bt * acc;
        }
        for (int64_t i = 0; i < V; ++i)
          for (int64_t jj = 0; jj < K; ++jj) dSb[i * K + jj] = G[i * K + jj] - bt * w[i] * kt[jj];
        /* decay Sb = alpha S_{t-1} */
        if (alpha) {
          double da = 0.0;
          for (size_t e = 0; e < VK; ++e) da += dSb[e] * Sp[e];
          if (dalpha) dalpha[bw_bth(b, t, h, T, H)] = da;
        }
        for (size_t e = 0; e < VK; ++e) G[e] = at * dSb[e];
      }
    }
    if (dS0)
      for (size_t e = 0; e < VK; ++e) dS0[(size_t)bh * VK + e] = G[e];

    /* ---- phase 1 reverse */
    double *g = (double *)malloc(sizeof(double) * (size_t)K);
    double *gy = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t i = 0; i < K; ++i) g[i] = dd ? dd[bh * K + i] : 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
      const double *kt = k + bw_bthx(b, t, h, 0, T, H, K);
      const double *d = dtr + (size_t)t * (size_t)K;
      const double *dktil = dkt + (size_t)t * (size_t)K;
      double *dkt_out = dk + bw_bthx(b, t, h, 0, T, H, K);
      const double bt = beta[bw_bth(b, t, h, T, H)];
      const double rt = r ? r[bw_bth(b, t, h, T, H)] : 1.0;
      const double bp = beta_aware ? bt : 1.0;
      double nraw = 0.0, a = 0.0;
      for (int64_t i = 0; i < K; ++i) {
        s[i] = kt[i] * kt[i];
        nraw += s[i];
        a += d[i] * s[i];
      }
      const double n = nraw > eps ? nraw : eps;
      const double c = eta * bp * (1.0 - bp * a) / n;
      double gc = 0.0, grr = 0.0;
      for (int64_t i = 0; i < K; ++i) {
        const double y = rt * d[i] + c * s[i];
        const int pass = !clamp || (y >= d_min && y <= d_max);
        gy[i] = pass ? g[i] : 0.0;
        gc += s[i] * gy[i];
        grr += d[i] * gy[i];
      }
      if (dr) dr[bw_bth(b, t, h, T, H)] = grr;
      const double dca = -eta * bp * bp / n; /* dc / da */
      const double dcn = nraw > eps ? -c / n : 0.0; /* dc / dn */
      for (int64_t i = 0; i < K; ++i) {
        const double ds = c * gy[i] + gc * dca * d[i] + gc * dcn;
        dkt_out[i] += 2.0 * kt[i] * ds + dktil[i] * d[i];
      }
      if (beta_aware) dbeta[bw_bth(b, t, h, T, H)] += gc * eta * (1.0 - 2.0 * bp * a) / n;
      for (int64_t i = 0; i < K; ++i) g[i] = dktil[i] * kt[i] + rt * gy[i] + dca * s[i] * gc;
    }
    if (dd1)
      for (int64_t i = 0; i < K; ++i) dd1[bh * K + i] = g[i];

    free(g);
    free(gy);
    free(dkt);
    free(w);
    free(dSb);
    free(G);
    free(us);
    free(Sbar);
    free(Sprev);
    free(wk);
    free(u);
    free(S);
    free(ck);
    free(s);
    free(dtr);
  }
  return 0;
}
