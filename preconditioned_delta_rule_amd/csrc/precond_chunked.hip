// Phase 1 of OSDN, chunked: the same sweep as precond_scan.hip (Section 4.2
// Eq.(4) / Algorithm 1, Section 4.4 Eq.(7), Appendix B), reorganised so that
// only a scalar per token stays on the sequential path.
//
// Per token the sweep is d <- clip(r_t d + c_t s_t) with s_t = k_t^2 and the
// step scalar c_t = a_t - b_t <d, s_t>, a_t = eta b'/max(|k_t|^2, eps),
// b_t = a_t b'.  Given every c_t, each coordinate of d follows its own
// recurrence, so the write keys can be emitted chunk-parallel.  The kernels:
//
//  prep  (one wave per (b,h,64-token chunk)): |k_t|^2, and the step scalar a
//        chunk has when every coordinate of d sits on d_min and stays there
//        (then <d, s_t> = d_min |k_t|^2); the chunk is marked when
//        r_t d_min + c_t max_i s_{t,i} <= d_min holds for all its tokens.
//  solve (one wave per (b,h), chunks in order): c_t for every token and d at
//        each chunk start.  A run of marked chunks that starts with d on
//        d_min everywhere needs no work (one step skips the whole run; its
//        chunks are re-marked so that emit starts them from d_min).
//        Otherwise, Section 4.2 notes that away
//        from the box the update is affine in d.  Suppose the coordinates on a
//        bound at the chunk start stay there and the others never reach one
//        (a fixed active set).  Then, with R_t = prod_{l<t} r_l, a free
//        coordinate is d_t = R_t (d_0 + sum_{j<t} x_j s_j), x_j = c_j/R_{j+1},
//        and x solves a unit lower-triangular system whose off-diagonal part
//        is the Gram matrix of the key squares restricted to the free
//        coordinates (the phase-1 counterpart of the chunk's UT transform; the
//        Gram on the matrix cores, the 64-step substitution in fp32).  The
//        assumption is checked afterwards, exactly for the coordinates on a
//        bound and with sum_j |x_j| s_{j,i} for the free ones; a chunk that
//        fails it is swept token by token, as the sequential kernel does.
//  emit  (one wave per (b,h,chunk)): replays d_{t+1} = clip(r_t d_t + c_t s_t)
//        from the chunk's start and writes k~_t = d_t (.) k_t (and/or the
//        bf16 residual (d_t - 1) (.) k_t).
// With vector retention (diag(r_t), Proposition A.3 of the appendix; the RV
// instantiations, K <= 128) prep marks a token with its largest retention
// (max_i r_{t,i} d_min + c_t max_i s_{t,i} <= d_min is sufficient), solve
// skips pinned runs as above and sweeps every other chunk token by token
// with the chunk's retention rows in LDS, and emit replays per coordinate.
#include "kernels.h"
#include "profile.h"
#include "scan_common.h"

namespace osdn {

namespace {

constexpr int CH = SCAN_CHUNK;  // tokens per chunk (64: one per lane)

template <typename TIn, int EPL>
__device__ __forceinline__ void lds_get(const TIn *p, float (&out)[EPL]) {
  typedef typename RowVec<TIn, EPL>::type Vt;
  const Vt v = *reinterpret_cast<const Vt *>(p);
  if constexpr (EPL == 1) {
    out[0] = to_f32(v);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = to_f32(v[e]);
  }
}

template <typename TIn, int EPL, bool FULL>
__device__ __forceinline__ void lds_put(TIn *p, const Row<TIn, EPL, FULL> &r) {
  typedef typename RowVec<TIn, EPL>::type Vt;
  Vt v;
  __builtin_memcpy(&v, r.w, sizeof(Vt));
  *reinterpret_cast<Vt *>(p) = v;
}

// ---------------------------------------------------------------- prep
template <typename TIn, int EPL, bool FULL, bool HAS_R, bool VL, bool RV = false>
__global__ __launch_bounds__(64) void scan_prep_kernel(ScanArgs a, ScanWork wk, int64_t N) {
  __shared__ float sbuf[64 * RS_PITCH];
  const int lane = threadIdx.x;
  const int64_t seq = blockIdx.x / N, n = blockIdx.x % N;
  const int64_t H = a.H, K = a.K;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t t0 = n * CH;
  if (VL && t0 >= T) return;  // past a shorter sequence's end
  const int L = (int)((T - t0) < CH ? (T - t0) : CH);
  const bool tok = lane < L;
  const TIn *kp = static_cast<const TIn *>(a.k) + ((tb + t0) * H + h) * K;
  const int64_t stride = H * K;
  const int64_t gi = (tb + t0 + (tok ? lane : 0)) * H + h;
  const float bt = a.beta[gi];
  float rt = HAS_R ? a.r[gi] : 1.0f;
  Row<TIn, EPL, FULL> rows[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) rows[u].load(kp + (u < L ? u : L - 1) * stride, lane, K);
  if constexpr (RV) {
    // the token's largest retention (a sufficient bound for the pinned test)
    const float *rp = a.r + ((tb + t0) * H + h) * K;
    float rm[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      Row<float, EPL, FULL> rr;
      rr.load(rp + (u < L ? u : L - 1) * stride, lane, K);
      float rv[EPL];
      rr.get(rv);
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) m = fmaxf(m, rv[e]);
      rm[u] = m;
    }
    rt = reduce_scatter64<true>(rm, lane, sbuf);
  }
  float sn[CH], sm[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    float k[EPL];
    rows[u].get(k);
    float pn = 0.0f, pm = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float s = k[e] * k[e];
      pn += s;
      pm = fmaxf(pm, s);
    }
    sn[u] = pn;
    sm[u] = pm;
  }
  const float nrm = reduce_scatter64<false>(sn, lane, sbuf);  // lane u: |k_{t0+u}|^2
  const float smx = reduce_scatter64<true>(sm, lane, sbuf);   // lane u: max_i k_{t0+u,i}^2
  const float dmin = a.d_min;
  const float bpr = a.beta_aware ? bt : 1.0f;
  const float ea = a.eta * bpr / fmaxf(nrm, a.eps);
  const float eb = ea * bpr;
  const float cpin = fmaf(-eb, dmin * nrm, ea);
  const bool stays = !tok || fmaf(cpin, cpin > 0.0f ? smx : 0.0f, rt * dmin) <= dmin;
  const bool pinned = a.clamp != 0 && __all(stays) != 0;
  if (tok) {
    wk.norm[gi] = nrm;
    wk.cstep[gi] = cpin;
  }
  const uint64_t stay = __ballot(stays);
  if (lane == 0) {
    wk.pin[seq * N + n] = pinned ? 1 : 0;
    wk.stay[seq * N + n] = a.clamp != 0 ? stay : 0;
  }
}

// Sum / max over each row of 16 lanes, every lane of the row receiving it
// (DPP: quad [1,0,3,2], quad [2,3,0,1], half-row mirror, row mirror).
template <int CTL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  return x + dpp_f<0x140>(x);
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  return fmaxf(x, dpp_f<0x140>(x));
}

// The same pass for K = 128, four chunks per workgroup (one per wave).  Lane
// l reads 8 consecutive coordinates (chunk l % 16) of token row 4 p + l / 16,
// so each load instruction covers four whole rows (rows of many tokens in one
// instruction cost several times more), and a token's sums need only a
// 16-lane reduction.  The per-token results pass through LDS to lane = token.
template <typename TIn, bool HAS_R, bool VL, bool RV = false>
__global__ __launch_bounds__(256) void scan_prep128_kernel(ScanArgs a, ScanWork wk, int64_t N) {
  __shared__ float sred[4][RV ? 3 : 2][CH];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ci = (int64_t)blockIdx.x * 4 + w;
  const int64_t H = a.H;
  if (ci >= a.B * H * N) return;
  const int64_t seq = ci / N, n = ci - seq * N;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t t0 = n * CH;
  if (VL && t0 >= T) return;  // past a shorter sequence's end (each wave has its own chunk and LDS)
  const int L = (int)((T - t0) < CH ? (T - t0) : CH);
  const bool tok = lane < L;
  const int64_t stride = H * 128;
  const TIn *kp = static_cast<const TIn *>(a.k) + ((tb + t0) * H + h) * 128 + 8 * (lane & 15);
  const int64_t gi = (tb + t0 + (tok ? lane : 0)) * H + h;
  const float bt = a.beta[gi];
  float rt = HAS_R ? a.r[gi] : 1.0f;
  float x[16][8];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int r = 4 * p + (lane >> 4);
    const TIn *rp = kp + (r < L ? r : L - 1) * stride;
    if constexpr (sizeof(TIn) == 2) {
      const bf16x8 v = *reinterpret_cast<const bf16x8 *>(rp);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[p][e] = to_f32(v[e]);
    } else {
      const floatx4 v0 = *reinterpret_cast<const floatx4 *>(rp);
      const floatx4 v1 = *reinterpret_cast<const floatx4 *>(rp + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[p][e] = v0[e];
        x[p][4 + e] = v1[e];
      }
    }
  }
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    float pn = 0.0f, pm = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sq = x[p][e] * x[p][e];
      pn += sq;
      pm = fmaxf(pm, sq);
    }
    // over the 16 lanes of a row: DPP quad swaps, half-row and row mirrors
    pn = row16_sum(pn);
    pm = row16_max(pm);
    if ((lane & 15) == 0) {
      sred[w][0][4 * p + (lane >> 4)] = pn;
      sred[w][1][4 * p + (lane >> 4)] = pm;
    }
  }
  if constexpr (RV) {
    // second pass, same layout: each token's largest retention
    const float *rp0 = a.r + ((tb + t0) * H + h) * 128 + 8 * (lane & 15);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int r = 4 * p + (lane >> 4);
      const float *rp = rp0 + (r < L ? r : L - 1) * stride;
      const floatx4 v0 = *reinterpret_cast<const floatx4 *>(rp);
      const floatx4 v1 = *reinterpret_cast<const floatx4 *>(rp + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[p][e] = v0[e];
        x[p][4 + e] = v1[e];
      }
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, x[p][e]);
      m = row16_max(m);
      if ((lane & 15) == 0) sred[w][RV ? 2 : 0][4 * p + (lane >> 4)] = m;
    }
    rt = sred[w][RV ? 2 : 0][lane];
  }
  const float nrm = sred[w][0][lane];  // |k_{t0+lane}|^2 (this wave's own LDS)
  const float smx = sred[w][1][lane];  // max_i k_{t0+lane,i}^2
  const float dmin = a.d_min;
  const float bpr = a.beta_aware ? bt : 1.0f;
  const float ea = a.eta * bpr / fmaxf(nrm, a.eps);
  const float eb = ea * bpr;
  const float cpin = fmaf(-eb, dmin * nrm, ea);
  const bool stays = !tok || fmaf(cpin, cpin > 0.0f ? smx : 0.0f, rt * dmin) <= dmin;
  const bool pinned = a.clamp != 0 && __all(stays) != 0;
  if (tok) {
    wk.norm[gi] = nrm;
    wk.cstep[gi] = cpin;
  }
  const uint64_t stay = __ballot(stays);
  if (lane == 0) {
    wk.pin[ci] = pinned ? 1 : 0;
    wk.stay[ci] = a.clamp != 0 ? stay : 0;
  }
}

// ---------------------------------------------------------------- factor
// The part of the closed form below that does not depend on d, for a chunk
// whose coordinates are all free.  With every coordinate free the step
// scalars solve A x = y, A = I + diag(g) tril(G, -1) unit lower triangular,
// G the Gram matrix of the chunk's key squares, g_t = b_t R_t / R_{t+1};
// only y_t = a_t / R_{t+1} - g_t <d_0, s_t> involves d_0.  This pass (one
// wave per chunk, all chunks at once) forms A^{-1} - I, so that the
// per-(b,h) pass replaces the Gram matrix and the 64-step substitution by one
// 64 x 64 matrix-vector product.  Lane c computes column c of A^{-1} by
// forward elimination in fp32 (the Gram matrix on the matrix cores, from bf16
// key squares, as in the solve pass).  When the strictly lower part N =
// diag(g) tril(G, -1) is small, ||N||_inf <= 2^-8, the Neumann series is used
// instead: A^{-1} - I = -N + N^2 - N^3 + ..., cut after N^2 (the remainder is
// below ||N||^3 / (1 - ||N||) < 6e-8 in the same norm), with N^2 on the
// matrix cores from bf16 N (relative error 2^-9 on a term below 2^-8 of N).
// The result goes out in the order the solve pass copies it into LDS:
// element (t, j) at float ((j/4) 64 + t) 4 + j%4.
// Chunks marked pinned, or outside the closed form's range (some r_t > 1, or
// R_L < 1/4), get fok = 0 and no factor.
template <typename TIn, int EPL, bool FULL, bool HAS_R, bool VL>
__global__ __launch_bounds__(64) void scan_factor_kernel(ScanArgs a, ScanWork wk, int64_t N) {
  constexpr int SP = 64 * EPL + 8;  // bf16 row pitch of the key squares
  constexpr int GP = CH + 4;        // fp32 row pitch of the Gram matrix (16-byte rows)
  // the Gram matrix overwrites the key squares once they are consumed (less
  // LDS per workgroup, more workgroups per CU)
  constexpr int NP = CH + 8;  // bf16 row pitch of N and N^T (series path)
  constexpr int SB = CH * SP * 2, GB = CH * GP * 4, NB = 2 * CH * NP * 2;
  constexpr int UB = SB > GB ? (SB > NB ? SB : NB) : (GB > NB ? GB : NB);
  __shared__ __attribute__((aligned(16))) unsigned char sbuf[UB];
  __shared__ __attribute__((aligned(16))) float sgv[CH];
  bf16 *sS = reinterpret_cast<bf16 *>(sbuf);
  float *sG = reinterpret_cast<float *>(sbuf);
  const int lane = threadIdx.x;
  const int64_t ci = blockIdx.x;
  const int64_t seq = ci / N, n = ci - seq * N;
  const int64_t H = a.H, K = a.K;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t t0 = n * CH;
  if (VL && t0 >= T) return;  // past a shorter sequence's end
  if (wk.pin[ci] == 1) {
    if (lane == 0) wk.fok[ci] = 0;
    return;
  }
  const int L = (int)((T - t0) < CH ? (T - t0) : CH);
  const bool tok = lane < L;
  const int64_t gi = (tb + t0 + (tok ? lane : 0)) * H + h;
  float bt = a.beta[gi], rt = HAS_R ? a.r[gi] : 1.0f, nrm = wk.norm[gi];
  if (!tok) {
    bt = 0.0f;
    rt = 1.0f;
    nrm = 1.0f;
  }
  const float bpr = a.beta_aware ? bt : 1.0f;
  const float ea = a.eta * bpr / fmaxf(nrm, a.eps);
  const float eb = ea * bpr;
  float g = eb;
  if constexpr (HAS_R) {
    // the same retention products and range test as the solve pass
    const float lr = logf(rt);
    float lin = lr;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(lin, off, 64);
      if (lane >= off) lin += y;
    }
    const float Rn = __expf(lin), Rt = __expf(lin - lr);
    if (!(lane_bcast(Rn, L - 1) >= 0.25f && __all(rt <= 1.0f) != 0)) {
      if (lane == 0) wk.fok[ci] = 0;
      return;
    }
    g = eb * (Rt / Rn);
  }
  sgv[lane] = g;
  // key squares of every coordinate (bf16; rows past the end are zero)
  {
    const int64_t stride = H * K;
    const TIn *rp = static_cast<const TIn *>(a.k) + ((tb + t0) * H + h) * K;
    Row<TIn, EPL, FULL> rows[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      rows[u].load(rp, lane, K);
      if (u + 1 < L) rp += stride;
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      float k[EPL];
      rows[u].get(k);
      typedef typename RowVec<bf16, EPL>::type Bv;
      Bv v;
      bf16 sq[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) sq[e] = to_bf16(u < L ? k[e] * k[e] : 0.0f);
      __builtin_memcpy(&v, sq, sizeof(Bv));
      *reinterpret_cast<Bv *>(sS + u * SP + lane * EPL) = v;
    }
  }
  wave_lds_sync();
  // the whole (symmetric) Gram matrix: lane (l16, lq) of tile (ti, tj) holds
  // G[16 ti + 4 lq + i][16 tj + l16] = G[16 tj + l16][16 ti + 4 lq + i]
  const int l16 = lane & 15, lq = lane >> 4;
  floatx4 acc[4][4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      acc[ti][tj] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < 64 * EPL; k0 += 32) {
        const bf16x8 x = *reinterpret_cast<const bf16x8 *>(&sS[(16 * ti + l16) * SP + k0 + 8 * lq]);
        const bf16x8 y = *reinterpret_cast<const bf16x8 *>(&sS[(16 * tj + l16) * SP + k0 + 8 * lq]);
        acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[ti][tj], 0, 0, 0);
      }
    }
  wave_lds_sync();  // the squares are consumed
  // ||N||_inf = max_t |g_t| sum_{j<t} |G[t][j]|
  float gt[4][4];  // g of rows 16 ti + 4 lq + i
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    const floatx4 v = *reinterpret_cast<const floatx4 *>(sgv + 16 * ti + 4 * lq);
#pragma unroll
    for (int i = 0; i < 4; ++i) gt[ti][i] = v[i];
  }
  float nmax = 0.0f;
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * ti + 4 * lq + i;
      float rs = 0.0f;
#pragma unroll
      for (int tj = 0; tj <= ti; ++tj) rs += 16 * tj + l16 < t ? fabsf(acc[ti][tj][i]) : 0.0f;
      nmax = fmaxf(nmax, fabsf(gt[ti][i]) * row16_sum(rs));
    }
  nmax = wave_max(nmax);
  float *sX = sG;  // [j][t] = (A^{-1} - I)[t][j], pitch CH + 1
  if (nmax <= 1.0f / 256.0f) {
    // ---- Neumann series: A^{-1} - I = N^2 - N (N^3 and beyond dropped)
    bf16 *sN = reinterpret_cast<bf16 *>(sbuf), *sNT = sN + CH * NP;
    float gc[4];  // g of rows 16 tj + l16
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) gc[tj] = sgv[16 * tj + l16];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        // N[t][j] (t = 16 ti + 4 lq + i, j = 16 tj + l16) into row j of N^T, and
        // by symmetry N[t'][j'] (t' = 16 tj + l16, j' = 16 ti + 4 lq + i) into row t' of N
        bf16x4 vt, vn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * ti + 4 * lq + i, j = 16 * tj + l16;
          vt[i] = to_bf16(j < t ? gt[ti][i] * acc[ti][tj][i] : 0.0f);
          vn[i] = to_bf16(t < j ? gc[tj] * acc[ti][tj][i] : 0.0f);
        }
        *reinterpret_cast<bf16x4 *>(sNT + (16 * tj + l16) * NP + 16 * ti + 4 * lq) = vt;
        *reinterpret_cast<bf16x4 *>(sN + (16 * tj + l16) * NP + 16 * ti + 4 * lq) = vn;
      }
    wave_lds_sync();
    floatx4 n2[4][4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int tj = 0; tj <= ti; ++tj) {
        n2[ti][tj] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < CH; k0 += 32) {
          const bf16x8 x = *reinterpret_cast<const bf16x8 *>(&sN[(16 * ti + l16) * NP + k0 + 8 * lq]);
          const bf16x8 y = *reinterpret_cast<const bf16x8 *>(&sNT[(16 * tj + l16) * NP + k0 + 8 * lq]);
          n2[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, n2[ti][tj], 0, 0, 0);
        }
      }
    wave_lds_sync();  // N and N^T are consumed
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int tj = 0; tj < 4; ++tj)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * ti + 4 * lq + i, j = 16 * tj + l16;
          float v = 0.0f;
          if (tj <= ti) v = j < t ? n2[ti][tj][i] - gt[ti][i] * acc[ti][tj][i] : 0.0f;
          sX[j * (CH + 1) + t] = v;
        }
  } else {
    // ---- exact: forward elimination
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int tj = 0; tj < 4; ++tj)
#pragma unroll
        for (int i = 0; i < 4; ++i) sG[(16 * ti + 4 * lq + i) * GP + 16 * tj + l16] = acc[ti][tj][i];
    wave_lds_sync();
    // M[j][t] = g_t G[j][t] = (diag(g) G)[t][j]: lane t scales column t
#pragma unroll
    for (int j = 0; j < CH; ++j) sG[j * GP + lane] *= g;
    wave_lds_sync();
    // column `lane` of A^{-1}: once z_j is final, z_t -= M[j][t] z_j for t > j
    float z[CH];
#pragma unroll
    for (int t = 0; t < CH; ++t) z[t] = t == lane ? 1.0f : 0.0f;
#pragma unroll
    for (int j = 0; j < CH - 1; ++j) {
      floatx4 mc[CH / 4];
#pragma unroll
      for (int q = (j + 1) / 4; q < CH / 4; ++q) mc[q] = *reinterpret_cast<const floatx4 *>(&sG[j * GP + 4 * q]);
      const float zj = z[j];
#pragma unroll
      for (int q = (j + 1) / 4; q < CH / 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * q + i > j) z[4 * q + i] = fmaf(-mc[q][i], zj, z[4 * q + i]);
    }
    wave_lds_sync();  // every lane is done with M
    // transpose through LDS (pitch 65: conflict-free both ways)
#pragma unroll
    for (int t = 0; t < CH; ++t) sX[lane * (CH + 1) + t] = t > lane ? z[t] : 0.0f;
  }
  wave_lds_sync();
  // one contiguous kilobyte per store instruction
  float *dst = wk.ainv + ci * (CH * CH);
#pragma unroll
  for (int q = 0; q < CH / 4; ++q) {
    floatx4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = sX[(4 * q + i) * (CH + 1) + lane];
    *reinterpret_cast<floatx4 *>(dst + (q * 64 + lane) * 4) = v;
  }
  if (lane == 0) wk.fok[ci] = 1;
}

// ---------------------------------------------------------------- solve
// Key rows reach LDS by direct copies (global_load_lds, two buffers: the
// next chunk's arrive while this one is used) when a row is a whole number of
// 16-byte pieces and both buffers fit; otherwise through registers.
template <typename TIn, int EPL, bool FULL, bool RV>
constexpr bool solve_rows_dma() {
  return FULL && !RV && 64 * EPL * sizeof(TIn) <= 512;
}

// Shared memory: the chunk's key rows (TIn [CH][64 EPL], two buffers with
// direct copies), the key squares of the free coordinates in bf16
// ([CH][64 EPL + 8]), their Gram matrix (fp32 [CH][CH+1]), per-token
// (x, c, r) (float4 [CH]), then either two chunks' A^{-1} - I from the factor
// pass (fp32 [2][CH CH], by chunk parity) or, with vector retention, the
// chunk's retention rows (fp32 [CH][64 EPL]).
template <typename TIn, int EPL, bool FULL, bool RV>
constexpr size_t solve_lds_bytes() {
  return (size_t)CH * 64 * EPL * sizeof(TIn) * (solve_rows_dma<TIn, EPL, FULL, RV>() ? 2 : 1) +
         (size_t)CH * (64 * EPL + 8) * 2 + (size_t)CH * (CH + 1) * 4 + (size_t)CH * 16 +
         (RV ? (size_t)CH * 64 * EPL * 4 : (size_t)2 * CH * CH * 4);
}

// One 16-byte global -> LDS copy per lane (global_load_lds): lane i writes
// bytes [16 i, 16 i + 16) after `lds`, which must be the same for every lane.
// The compiler does not track these copies: wait on vmcnt before reading.
__device__ __forceinline__ void dma16(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename TIn, int EPL, bool FULL, bool HAS_R, bool PF, bool VL, bool RV = false>
__global__ __launch_bounds__(64) void scan_solve_kernel(ScanArgs a, ScanWork wk, int64_t N) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int RP = 64 * EPL;      // row pitch of sR (elements)
  constexpr int SP = 64 * EPL + 8;  // row pitch of sS (bf16)
  constexpr bool DMA = solve_rows_dma<TIn, EPL, FULL, RV>();
  constexpr size_t RB = (size_t)CH * RP * sizeof(TIn) * (DMA ? 2 : 1);  // bytes of the row buffers
  TIn *sRb = reinterpret_cast<TIn *>(smem);
  bf16 *sS = reinterpret_cast<bf16 *>(smem + RB);
  float *sG = reinterpret_cast<float *>(smem + RB + (size_t)CH * SP * 2);
  floatx4 *sTok = reinterpret_cast<floatx4 *>(sG + CH * (CH + 1));
  float *sA = reinterpret_cast<float *>(sTok + CH);  // factors of chunks n, n + 1 ([2][CH CH], by n & 1)
  float *sRv = sA;                                    // RV: the chunk's retention rows [CH][RP]

  const int lane = threadIdx.x;
  const int64_t seq = blockIdx.x;
  const int64_t H = a.H, K = a.K;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t Nb = (T + CH - 1) / CH;  // this sequence's chunks (N is the row stride)
  const int64_t stride = H * K;
  const float eta = a.eta, eps = a.eps, dmin = a.d_min, dmax = a.d_max;
  const bool clamp = a.clamp != 0, aware = a.beta_aware != 0;

  float d[EPL];
  bool valid[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int64_t c = (int64_t)lane * EPL + e;
    valid[e] = c < K;
    d[e] = valid[e] ? (a.d1 ? a.d1[seq * K + c] : 1.0f) : 0.0f;
  }
  int n_pinned = 0, n_active = 0, n_seq = 0;
  uint64_t pinmask = 0, fokmask = 0;
  bool ahave = false;    // chunk n's factor copy was issued during chunk n - 1
  float pend_c = 0.0f;   // a chunk's step scalars are stored at the top of the next
  int64_t pend_gi = -1;  // pass (after its wait), so no store is in flight at that wait
  // the factor pass's A^{-1} - I of chunk m into sA (16 copies of 1 KB)
  auto dma_factor = [&](int64_t m) {
    const float *src = wk.ainv + (seq * N + m) * (CH * CH);
    float *dst = sA + (m & 1) * (CH * CH);
#pragma unroll
    for (int q = 0; q < CH / 4; ++q) dma16(src + q * 256 + lane * 4, dst + q * 256);
  };
  // chunk m's key rows into row buffer m & 1 (rows past the end repeat the
  // last one): lane l of copy i brings 16 bytes of row i RPI + l / (RB16)
  auto dma_rows = [&](int64_t m) {
    constexpr int RB16 = 64 * EPL * (int)sizeof(TIn) / 16;  // 16-byte pieces per row
    constexpr int RPI = 64 / RB16;                           // rows per copy
    const int64_t tm = m * CH;
    const int Lm = (int)((T - tm) < CH ? (T - tm) : CH);
    const TIn *src = static_cast<const TIn *>(a.k) + ((tb + tm) * H + h) * K + (lane % RB16) * (16 / sizeof(TIn));
    TIn *dst = sRb + (m & 1) * (CH * RP);
    const int lr = lane / RB16;
#pragma unroll
    for (int i = 0; i < CH / RPI; ++i) {
      const int row = i * RPI + lr;
      dma16(src + (int64_t)(row < Lm ? row : Lm - 1) * stride, dst + i * RPI * RP);
    }
  };
  Row<TIn, EPL, FULL> nrow[PF ? CH : 1];
  float nbt = 0.0f, nrt = 1.0f, nnrm = 1.0f;
  bool have = false;  // chunk n's rows already sit in (or are on their way to) LDS, its scalars in nbt/nrt/nnrm

  // every pass of the loop advances n by step >= 1 (a pinned run sets it)
  for (int64_t n = 0, step = 1; n < Nb; n += step) {
    step = 1;
    const int64_t t0 = n * CH;
    const int L = (int)((T - t0) < CH ? (T - t0) : CH);
    const bool tok = lane < L;  // lane u <-> token t0 + u
    const int64_t gi = (tb + t0 + (tok ? lane : 0)) * H + h;
    if ((n & 63) == 0) {
      const int p = n + lane < Nb ? wk.pin[seq * N + n + lane] : 0;
      pinmask = __ballot(p == 1);
      if constexpr (!RV) {
        const int f = n + lane < Nb ? wk.fok[seq * N + n + lane] : 0;
        fokmask = __ballot(f == 1);
      }
    }

    // where d sits: on d_min, on d_max, inside
    bool onlo[EPL], onhi[EPL], fr[EPL];
    bool lo = false, hi = false, free_ = false;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      onlo[e] = clamp && valid[e] && d[e] == dmin;
      onhi[e] = clamp && valid[e] && d[e] == dmax && !onlo[e];
      fr[e] = valid[e] && !onlo[e] && !onhi[e];
      lo |= onlo[e];
      hi |= onhi[e];
      free_ |= fr[e];
    }
    const bool any_lo = __any(lo) != 0, any_hi = __any(hi) != 0, any_free = __any(free_) != 0;
    if (!any_free && !any_hi) {
      // d on d_min everywhere: it stays there through the run of marked
      // chunks that starts here (c_t of those was written by the prep pass);
      // the run is marked 2 so that the emit pass starts it from d_min
      const uint64_t m = ~(pinmask >> (n & 63));
      const int run = m ? (int)__builtin_ctzll(m) : 64;
      if (run > 0) {
        if (lane < run) wk.pin[seq * N + n + lane] = 2;
        n_pinned += run;
        step = run;
        have = false;
        ahave = false;
        continue;
      }
    }
    wait_loads();  // the copies issued during the previous chunk have landed
    if (pend_gi >= 0) wk.cstep[pend_gi] = pend_c;
    pend_gi = -1;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if (valid[e]) wk.dstart[(seq * N + n) * K + lane * EPL + e] = d[e];
    // every coordinate free and the chunk has a factor: the closed form
    // needs only a matrix-vector product with it
    const bool fast = !RV && ((fokmask >> (n & 63)) & 1) != 0 && !any_lo && !any_hi && any_free;
    TIn *sR = sRb + (DMA ? (n & 1) * (CH * RP) : 0);
    {
      // copies not issued during the previous chunk: now, and wait for them
      bool issued = false;
      if (DMA && !have) {
        dma_rows(n);
        issued = true;
      }
      if (fast && !ahave) {
        dma_factor(n);
        issued = true;
      }
      if (issued) wait_loads();
    }

    // this chunk's key rows and scalars
    const TIn *kp = static_cast<const TIn *>(a.k) + ((tb + t0) * H + h) * K;
    float bt, rt, nrm;
    if ((PF || DMA) && have) {
      bt = nbt;
      rt = nrt;
      nrm = nnrm;
    } else {
      bt = a.beta[gi];
      rt = HAS_R ? a.r[gi] : 1.0f;
      nrm = wk.norm[gi];
      constexpr int GL = CH / Row<TIn, EPL, FULL>::WORDS;  // rows per load batch (<= 64 words)
      const TIn *rp = kp;  // row u0 + u, the last row repeated past the end
#pragma unroll
      for (int u0 = 0; u0 < (DMA ? 0 : CH); u0 += GL) {
        Row<TIn, EPL, FULL> tmp[GL];
#pragma unroll
        for (int u = 0; u < GL; ++u) {
          tmp[u].load(rp, lane, K);
          if (u0 + u + 1 < L) rp += stride;
        }
#pragma unroll
        for (int u = 0; u < GL; ++u) lds_put<TIn, EPL, FULL>(sR + (u0 + u) * RP + lane * EPL, tmp[u]);
      }
      if constexpr (RV) {
        const float *rp = a.r + ((tb + t0) * H + h) * K;
        constexpr int GV = CH / Row<float, EPL, FULL>::WORDS;
#pragma unroll
        for (int u0 = 0; u0 < CH; u0 += GV) {
          Row<float, EPL, FULL> tmp[GV];
#pragma unroll
          for (int u = 0; u < GV; ++u) tmp[u].load(rp + (u0 + u < L ? u0 + u : L - 1) * stride, lane, K);
#pragma unroll
          for (int u = 0; u < GV; ++u) lds_put<float, EPL, FULL>(sRv + (u0 + u) * RP + lane * EPL, tmp[u]);
        }
      }
    }
    if (!tok) {
      bt = 0.0f;
      rt = 1.0f;
      nrm = 1.0f;
    }
    // prefetch the next chunk (rows stay in registers until this one is done),
    // unless the prep pass marked it: if d ends this chunk on d_min the run
    // of marked chunks is skipped without its rows, else they are loaded then
    const bool next_marked = ((n + 1) & 63) != 0 && ((pinmask >> ((n + 1) & 63)) & 1) != 0;
    const bool pf = (PF || DMA) && n + 1 < Nb && !next_marked;
    bool ahave_next = false;
    if constexpr (PF || DMA) {
      if (pf) {
        if (!RV && ((n + 1) & 63) != 0 && ((fokmask >> ((n + 1) & 63)) & 1) != 0) {
          dma_factor(n + 1);
          ahave_next = true;
        }
        const int64_t t1 = t0 + CH;
        const int L1 = (int)((T - t1) < CH ? (T - t1) : CH);
        if constexpr (DMA) {
          dma_rows(n + 1);
        } else {
          const TIn *rp = kp + CH * stride;
#pragma unroll
          for (int u = 0; u < CH; ++u) {
            nrow[u].load(rp, lane, K);
            if (u + 1 < L1) rp += stride;
          }
        }
        const int64_t gi1 = (tb + t1 + (lane < L1 ? lane : 0)) * H + h;
        nbt = a.beta[gi1];
        nrt = HAS_R ? a.r[gi1] : 1.0f;
        nnrm = wk.norm[gi1];
      }
    }
    const float bpr = aware ? bt : 1.0f;
    const float ea = eta * bpr / fmaxf(nrm, eps);  // c_t = ea - eb <d, s_t>
    const float eb = ea * bpr;
    float cst = 0.0f;  // lane u: c for token t0 + u
    bool done = false;
    wave_lds_sync();

    // retention products R_t = prod_{l<t} r_l (log-space scan): Rn = R_{t+1},
    // Rt = R_t.  The bound on free coordinates below needs R_t non-increasing,
    // and R_L >= 1/4 keeps the 1/R_t factors from costing more than two bits;
    // otherwise a chunk with free coordinates goes token by token.
    float Rn = 1.0f, Rt = 1.0f;
    bool try_closed = !RV;  // vector retention: no closed form, token by token
    if constexpr (HAS_R) {
      if (any_free) {
        const float lr = logf(rt);
        float lin = lr;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(lin, off, 64);
          if (lane >= off) lin += y;
        }
        Rn = __expf(lin);
        Rt = __expf(lin - lr);
        try_closed = lane_bcast(Rn, L - 1) >= 0.25f && __all(rt <= 1.0f) != 0;
      }
    }

    // ---- fixed active set, closed form
    if (try_closed) {
      float pvF[CH], pvP[HAS_R ? CH : 1];
      // one pass over the rows; the branch on writing the squares is taken
      // once, outside the unrolled loop, so that the row reads can overlap
      auto sq_pass = [&](auto ws) {
        constexpr bool WS = decltype(ws)::value;
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          float k[EPL];
          lds_get<TIn, EPL>(sR + u * RP + lane * EPL, k);
          float pf_ = 0.0f, pp_ = 0.0f;
          bf16 sq[EPL];
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            const float s = u < L ? k[e] * k[e] : 0.0f;
            if (HAS_R) {
              pf_ = fmaf(fr[e] ? d[e] : 0.0f, s, pf_);
              pp_ = fmaf(fr[e] ? 0.0f : d[e], s, pp_);
            } else {
              pf_ = fmaf(d[e], s, pf_);
            }
            sq[e] = to_bf16(fr[e] ? s : 0.0f);
          }
          if constexpr (WS) {
            typedef typename RowVec<bf16, EPL>::type Bv;
            Bv v;
            __builtin_memcpy(&v, sq, sizeof(Bv));
            *reinterpret_cast<Bv *>(sS + u * SP + lane * EPL) = v;
          }
          pvF[u] = pf_;
          if (HAS_R) pvP[HAS_R ? u : 0] = pp_;
        }
      };
      if (any_free && !fast)
        sq_pass(std::true_type{});
      else
        sq_pass(std::false_type{});
      const float p0F = reduce_scatter64<false>(pvF, lane, sG);  // <d_0, s_t> over the free (all, without r) coords
      float p0P = 0.0f;
      if constexpr (HAS_R)
        if (!fast) p0P = reduce_scatter64<false>(pvP, lane, sG);  // over the coords on a bound
      wave_lds_sync();
      if (any_free && !fast) {
        // Gram matrix of the free key squares, lower 16x16 tiles
        const int l16 = lane & 15, lq = lane >> 4;
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int tj = 0; tj < 4; ++tj) {
            if (tj > ti) continue;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < 64 * EPL; k0 += 32) {
              const bf16x8 x = *reinterpret_cast<const bf16x8 *>(&sS[(16 * ti + l16) * SP + k0 + 8 * lq]);
              const bf16x8 y = *reinterpret_cast<const bf16x8 *>(&sS[(16 * tj + l16) * SP + k0 + 8 * lq]);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sG[(16 * ti + 4 * lq + i) * (CH + 1) + 16 * tj + l16] = acc[i];
          }
        wave_lds_sync();
      }
      float x = 0.0f;
      if (!any_free) {
        // every coordinate on a bound: <d, s_t> = <d_0, s_t>
        if (tok) cst = fmaf(-eb, p0P + p0F, ea);
      } else if (fast) {
        // x = y + (A^{-1} - I) y, y_t = ea_t / R_{t+1} - g_t p0F_t
        const float g = HAS_R ? eb * (Rt / Rn) : eb;
        const float y = tok ? (HAS_R ? ea / Rn - g * p0F : ea - g * p0F) : 0.0f;
        sG[lane] = y;
        wave_lds_sync();
        const float *Ai = sA + (n & 1) * (CH * CH);
        float acc = y;
#pragma unroll
        for (int q = 0; q < CH / 4; ++q) {
          const floatx4 av = *reinterpret_cast<const floatx4 *>(Ai + (q * 64 + lane) * 4);
          const floatx4 yv = *reinterpret_cast<const floatx4 *>(sG + 4 * q);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc = fmaf(av[i], yv[i], acc);
        }
        x = tok ? acc : 0.0f;
        cst = Rn * x;
      } else {
        // x_t + g_t sum_{j<t} G_jt x_j = ea_t / R_{t+1} - g_t (p0P_t / R_t + p0F_t),
        // g_t = eb_t R_t / R_{t+1}
        const float g = HAS_R ? eb * (Rt / Rn) : eb;
        float acc = 0.0f;
        if (tok) acc = HAS_R ? ea / Rn - g * (p0P / Rt + p0F) : ea - g * p0F;
        float grow[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const float gj = sG[lane * (CH + 1) + j];
          grow[j] = j < lane ? g * gj : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < CH - 1; ++j) {
          const float xj = lane_bcast(acc, j);
          acc = fmaf(-grow[j], xj, acc);  // grow[j] = 0 on lanes <= j
        }
        x = tok ? acc : 0.0f;
        cst = Rn * x;
      }
      sTok[lane] = floatx4{x, cst, rt, 0.0f};
      wave_lds_sync();
      // check the active set; d_L = R_L (d_0 + sum_j x_j s_j) on free coords
      float sum[EPL], bnd[EPL], mxl[EPL], mnh[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        sum[e] = bnd[e] = 0.0f;
        mxl[e] = dmin;
        mnh[e] = dmax;
      }
      // tokens past the sequence's end carry x = c = 0 and r = 1, which
      // leave every sum and bound below unchanged: no branch in the loop;
      // the bounds of coordinates sitting on d_min / d_max only when some do
      auto check_pass = [&](auto bounds) {
        constexpr bool BOUNDS = decltype(bounds)::value;
#pragma unroll 8
        for (int u = 0; u < CH; ++u) {
          float k[EPL];
          lds_get<TIn, EPL>(sR + u * RP + lane * EPL, k);
          const floatx4 tv = sTok[u];
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            const float s = k[e] * k[e];
            sum[e] = fmaf(tv[0], s, sum[e]);
            bnd[e] = fmaf(fabsf(tv[0]), s, bnd[e]);
            if constexpr (BOUNDS) {
              mxl[e] = fmaxf(mxl[e], fmaf(tv[1], s, tv[2] * dmin));
              mnh[e] = fminf(mnh[e], fmaf(tv[1], s, tv[2] * dmax));
            }
          }
        }
      };
      if (any_lo || any_hi)
        check_pass(std::true_type{});
      else
        check_pass(std::false_type{});
      const float RL = lane_bcast(Rn, L - 1);
      bool ok = true;
      float dn[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        dn[e] = fr[e] ? RL * (d[e] + sum[e]) : d[e];
        if (fr[e] && clamp) ok = ok && RL * (d[e] - bnd[e]) >= dmin && d[e] + bnd[e] <= dmax;
        if (onlo[e]) ok = ok && mxl[e] <= dmin;
        if (onhi[e]) ok = ok && mnh[e] >= dmax;
      }
      if (__all(ok)) {
        done = true;
        ++n_active;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d[e] = valid[e] ? dn[e] : 0.0f;
      }
    }

    int u_end = L;  // tokens whose step scalar this pass computed
    if (!done) {
      // token by token, the exact sweep.  Once every coordinate sits on d_min
      // and the prep pass found that each remaining token keeps such a d
      // there (the same test that pins a whole chunk), the rest of the chunk
      // leaves d on d_min; those tokens keep the step scalar the prep pass
      // wrote for exactly that case.
      ++n_seq;
      cst = 0.0f;
      const uint64_t stay = clamp ? wk.stay[seq * N + n] : 0;
      for (int u = 0; u < L; ++u) {
        float k[EPL], s[EPL], pa = 0.0f;
        lds_get<TIn, EPL>(sR + u * RP + lane * EPL, k);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          s[e] = k[e] * k[e];
          pa = fmaf(d[e], s[e], pa);
        }
        const float align = wave_sum(pa);
        const float c = fmaf(-lane_bcast(eb, u), align, lane_bcast(ea, u));
        float ru[EPL];
        if constexpr (RV) {
          lds_get<float, EPL>(sRv + u * RP + lane * EPL, ru);
        } else {
          const float rb = lane_bcast(rt, u);
#pragma unroll
          for (int e = 0; e < EPL; ++e) ru[e] = rb;
        }
        cst = lane == u ? c : cst;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float xx = fmaf(c, s[e], ru[e] * d[e]);
          if (clamp) xx = fminf(fmaxf(xx, dmin), dmax);
          d[e] = valid[e] ? xx : 0.0f;
        }
        if (clamp && u + 1 < L) {
          // tokens u + 1 .. L - 1 all keep d on d_min?
          const uint64_t rest = (L - u - 1 >= 64 ? ~0ull : ((1ull << (L - u - 1)) - 1)) << (u + 1);
          if ((stay & rest) == rest) {
            bool onmin = true;
#pragma unroll
            for (int e = 0; e < EPL; ++e) onmin = onmin && (!valid[e] || d[e] == dmin);
            if (__all(onmin)) {
              u_end = u + 1;
              break;
            }
          }
        }
      }
    }
    pend_c = cst;
    pend_gi = tok && lane < u_end ? gi : -1;
    wave_lds_sync();
    if constexpr (PF) {
      if (pf) {
#pragma unroll
        for (int u = 0; u < CH; ++u) lds_put<TIn, EPL, FULL>(sR + u * RP + lane * EPL, nrow[u]);
      }
    }
    have = pf;
    ahave = ahave_next;
    wave_lds_sync();
  }
  if (pend_gi >= 0) wk.cstep[pend_gi] = pend_c;
  if (a.d_out) {
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if (valid[e]) a.d_out[seq * K + lane * EPL + e] = d[e];
  }
  if (lane == 0) {
    wk.flags[3 * seq + 0] = n_pinned;
    wk.flags[3 * seq + 1] = n_active;
    wk.flags[3 * seq + 2] = n_seq;
  }
}

// ---------------------------------------------------------------- solve, K = 128
// The same pass for K = 128 with scalar (or no) retention, over four waves so
// that a chunk's closed form is spread across the CU's four SIMDs.  Wave w
// owns coordinates [32 w, 32 w + 32); lane l of it the pair 32 w + 2 (l % 16)
// + {0, 1} for tokens 16 (l / 16) .. 16 (l / 16) + 15 of the chunk, holding
// their key squares in registers.  A chunk whose coordinates are all free and
// that has a factor: <d_0, s_t> by partial sums (a reduce-scatter over the 16
// lanes of a DPP row, then over the waves through LDS); y and x = y +
// (A^{-1} - I) y in every wave (lane = token); d_L and the bound of the
// active-set check per coordinate pair (partial sums combined over the four
// token groups).  Two workgroup barriers per chunk: after the partial sums,
// and after the check (which also publishes the new d's position in the box).
// Any other chunk is swept token by token by wave 0 with d gathered in LDS.
// Key rows and factors arrive by direct copies, a quarter issued by each
// wave, each wave waiting for its own before the check's barrier.
template <typename TIn>
constexpr size_t solve4_lds_bytes() {
  // rows [2][CH][128], factors [2][CH CH], per-wave partial sums, y, x
  // ([3][4][CH]), d (128) and the per-wave flags (4)
  return (size_t)2 * CH * 128 * sizeof(TIn) + (size_t)2 * CH * CH * 4 + (size_t)3 * 4 * CH * 4 + 128 * 4 + 16;
}

// Workgroup barrier that does not wait for outstanding global loads (the
// next chunk's copies stay in flight across it); LDS accesses before it are
// complete.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Reduce-scatter over the 16 lanes of a DPP row: on entry lane j of the row
// holds v[0..15]; on return it holds the sum over the row of entry j.  Each
// level pairs lanes that differ in one bit of j (row mirror: bit 3, half-row
// mirror: bit 2, quad permutations: bits 1 and 0) and agree above it; a lane
// keeps the half of its entries whose index bit matches its own.
template <int M, int CTL>
__device__ __forceinline__ void rs16_level(float (&v)[16], int j) {
  const bool upper = (j & M) != 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    float a = v[i], b = v[i + M];
    asm("" : "+v"(a), "+v"(b));  // plain values: a register select, not an indexed access
    const float give = upper ? a : b;
    const float keep = upper ? b : a;
    v[i] = keep + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, give), CTL, 0xF,
                                                                         0xF, false));
  }
}
__device__ __forceinline__ float reduce_scatter16(float (&v)[16], int j) {
  rs16_level<8, 0x140>(v, j);
  rs16_level<4, 0x141>(v, j);
  rs16_level<2, 0x4E>(v, j);
  rs16_level<1, 0xB1>(v, j);
  return v[0];
}

template <typename TIn, bool HAS_R, bool VL>
__global__ __launch_bounds__(256) void scan_solve4_kernel(ScanArgs a, ScanWork wk, int64_t N) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int RP = 128;
  TIn *sRb = reinterpret_cast<TIn *>(smem);                                        // [2][CH][RP]
  float *sA = reinterpret_cast<float *>(smem + (size_t)2 * CH * RP * sizeof(TIn));  // [2][CH CH]
  float *sPw = sA + 2 * CH * CH;                                                    // [4][CH]
  float *sY = sPw + 4 * CH;                                                         // [4][CH]
  float *sX = sY + 4 * CH;                                                          // [4][CH]
  float *sD = sX + 4 * CH;                                                          // [128]
  int *sF = reinterpret_cast<int *>(sD + 128);                                      // [4]

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cp = l & 15, tq = l >> 4;
  const int c0 = 32 * w + 2 * cp;  // this lane's coordinates c0, c0 + 1
  const int64_t seq = blockIdx.x;
  const int64_t H = a.H;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t Nb = (T + CH - 1) / CH;
  const int64_t stride = H * RP;
  const float eta = a.eta, eps = a.eps, dmin = a.d_min, dmax = a.d_max;
  const bool clamp = a.clamp != 0, aware = a.beta_aware != 0;

  float d[2];
  d[0] = a.d1 ? a.d1[seq * RP + c0] : 1.0f;
  d[1] = a.d1 ? a.d1[seq * RP + c0 + 1] : 1.0f;

  // flags of this wave's coordinates: bit 0 some on d_min, 1 some on d_max, 2 some free
  auto wave_flags = [&]() {
    bool lo = false, hi = false, fr = false;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const bool onlo = clamp && d[e] == dmin;
      const bool onhi = clamp && d[e] == dmax && !onlo;
      lo |= onlo;
      hi |= onhi;
      fr |= !onlo && !onhi;
    }
    return (__any(lo) ? 1 : 0) | (__any(hi) ? 2 : 0) | (__any(fr) ? 4 : 0);
  };
  int gflags;  // the same flags over all coordinates
  if (l == 0) sF[w] = wave_flags();
  lds_barrier();
  gflags = sF[0] | sF[1] | sF[2] | sF[3];
  lds_barrier();  // sF is rewritten at the end of the first chunk

  // this wave's quarter of the copies of chunk m's rows and factor
  auto dma_rows = [&](int64_t m) {
    constexpr int RB16 = RP * (int)sizeof(TIn) / 16;  // 16-byte pieces per row (16 or 32)
    constexpr int RPI = 64 / RB16;                    // rows per copy (4 or 2)
    const int64_t tm = m * CH;
    const int Lm = (int)((T - tm) < CH ? (T - tm) : CH);
    const TIn *src = static_cast<const TIn *>(a.k) + ((tb + tm) * H + h) * RP + (l % RB16) * (16 / sizeof(TIn));
    TIn *dst = sRb + (m & 1) * (CH * RP);
    constexpr int NC = CH / RPI;  // copies per chunk (16 or 32), a quarter per wave
#pragma unroll
    for (int i0 = 0; i0 < NC / 4; ++i0) {
      const int i = w * (NC / 4) + i0;
      const int row = i * RPI + l / RB16;
      dma16(src + (int64_t)(row < Lm ? row : Lm - 1) * stride, dst + i * RPI * RP);
    }
  };
  auto dma_factor = [&](int64_t m) {
    const float *src = wk.ainv + (seq * N + m) * (CH * CH);
    float *dst = sA + (m & 1) * (CH * CH);
#pragma unroll
    for (int q0 = 0; q0 < 4; ++q0) {
      const int q = 4 * w + q0;
      dma16(src + q * 256 + l * 4, dst + q * 256);
    }
  };

  int n_pinned = 0, n_active = 0, n_seq = 0;
  uint64_t pinmask = 0, fokmask = 0;
  bool have = false, ahave = false;  // chunk n's rows / factor were copied during chunk n - 1
  float nbt = 0.0f, nrt = 1.0f, nnrm = 1.0f;
  float pend_c = 0.0f;  // wave 0: step scalars of the last chunk, stored after the next wait
  int64_t pend_gi = -1;

  for (int64_t n = 0, step = 1; n < Nb; n += step) {
    step = 1;
    const int64_t t0 = n * CH;
    const int L = (int)((T - t0) < CH ? (T - t0) : CH);
    const bool tok = l < L;  // lane l <-> token t0 + l in the token views
    const int64_t gi = (tb + t0 + (tok ? l : 0)) * H + h;
    if ((n & 63) == 0) {
      const int p = n + l < Nb ? wk.pin[seq * N + n + l] : 0;
      pinmask = __ballot(p == 1);
      const int f = n + l < Nb ? wk.fok[seq * N + n + l] : 0;
      fokmask = __ballot(f == 1);
    }
    const bool any_lo = (gflags & 1) != 0, any_hi = (gflags & 2) != 0, any_free = (gflags & 4) != 0;
    if (!any_free && !any_hi) {
      // d on d_min everywhere: skip the run of marked chunks (see scan_solve_kernel)
      const uint64_t m = ~(pinmask >> (n & 63));
      const int run = m ? (int)__builtin_ctzll(m) : 64;
      if (run > 0) {
        if (w == 0 && l < run) wk.pin[seq * N + n + l] = 2;
        n_pinned += run;
        step = run;
        have = false;
        ahave = false;
        continue;
      }
    }
    const bool fast = ((fokmask >> (n & 63)) & 1) != 0 && !any_lo && !any_hi;
    if (!have || (fast && !ahave)) {
      // copies not issued during the previous chunk: now, and wait for them
      if (!have) dma_rows(n);
      if (fast && !ahave) dma_factor(n);
      wait_loads();
      lds_barrier();
    }
    // per-token scalars (every wave, lane = token), used before any new
    // global access is issued so that waiting for them waits for nothing else
    float bt, rt, nrm;
    if (have) {
      bt = nbt;
      rt = nrt;
      nrm = nnrm;
    } else {
      bt = a.beta[gi];
      rt = HAS_R ? a.r[gi] : 1.0f;
      nrm = wk.norm[gi];
    }
    if (!tok) {
      bt = 0.0f;
      rt = 1.0f;
      nrm = 1.0f;
    }
    const float bpr = aware ? bt : 1.0f;
    const float ea = eta * bpr / fmaxf(nrm, eps);  // c_t = ea - eb <d, s_t>
    const float eb = ea * bpr;
    float Rn = 1.0f, Rt = 1.0f;
    if constexpr (HAS_R) {
      const float lr = logf(rt);
      float lin = lr;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(lin, off, 64);
        if (l >= off) lin += y;
      }
      Rn = __expf(lin);
      Rt = __expf(lin - lr);
    }
    asm volatile("" ::"v"(ea), "v"(eb), "v"(Rn), "v"(Rt), "v"(rt) : "memory");
    if (w == 0 && pend_gi >= 0) wk.cstep[pend_gi] = pend_c;
    pend_gi = -1;
    if (tq == 0) {
      wk.dstart[(seq * N + n) * RP + c0] = d[0];
      wk.dstart[(seq * N + n) * RP + c0 + 1] = d[1];
    }
    // the next chunk's copies and scalars, unless the prep pass marked it
    const bool next_marked = ((n + 1) & 63) != 0 && ((pinmask >> ((n + 1) & 63)) & 1) != 0;
    const bool pf = n + 1 < Nb && !next_marked;
    bool ahave_next = false;
    if (pf) {
      if (((n + 1) & 63) != 0 && ((fokmask >> ((n + 1) & 63)) & 1) != 0) {
        dma_factor(n + 1);
        ahave_next = true;
      }
      dma_rows(n + 1);
      const int64_t t1 = t0 + CH;
      const int L1 = (int)((T - t1) < CH ? (T - t1) : CH);
      const int64_t gi1 = (tb + t1 + (l < L1 ? l : 0)) * H + h;
      nbt = a.beta[gi1];
      nrt = HAS_R ? a.r[gi1] : 1.0f;
      nnrm = wk.norm[gi1];
    }
    const TIn *R = sRb + (n & 1) * (CH * RP);

    bool done = false;
    float cst = 0.0f;  // wave 0, lane = token: the step scalar
    if (fast) {
      // key squares of this lane's pair over its 16 tokens.  Rows past the
      // chunk end hold copies of its last row (finite); every use of their
      // squares is weighted by x_t = 0 or lands in a masked token's p0.
      float s0[16], s1[16], pp[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 16 * tq + i;
        float k[2];
        lds_get<TIn, 2>(R + t * RP + c0, k);
        s0[i] = k[0] * k[0];
        s1[i] = k[1] * k[1];
        pp[i] = fmaf(d[0], s0[i], d[1] * s1[i]);
      }
      sPw[w * CH + 16 * tq + cp] = reduce_scatter16(pp, cp);  // token 16 tq + cp, this wave's coordinates
      lds_barrier();  // ---- A: partial sums of every wave in LDS
      const float p0 = sPw[l] + sPw[CH + l] + sPw[2 * CH + l] + sPw[3 * CH + l];
      const float g = HAS_R ? eb * (Rt / Rn) : eb;
      const float y = tok ? (HAS_R ? ea / Rn - g * p0 : ea - g * p0) : 0.0f;
      float *sYw = sY + w * CH, *sXw = sX + w * CH;
      sYw[l] = y;
      wave_lds_sync();
      const float *Ai = sA + (n & 1) * (CH * CH);
      float xa[4] = {y, 0.0f, 0.0f, 0.0f};  // four independent chains
      // the factor's rows and y in batches of four 4-column slabs, each batch
      // requested before the previous one's products (so the LDS latency is
      // paid about once, not once per pair of slabs)
      floatx4 av[2][4], yv[2][4];
      auto fetch_ay = [&](int bt, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          av[buf][u] = *reinterpret_cast<const floatx4 *>(Ai + ((4 * bt + u) * 64 + l) * 4);
          yv[buf][u] = *reinterpret_cast<const floatx4 *>(sYw + 4 * (4 * bt + u));
        }
      };
      fetch_ay(0, 0);
#pragma unroll
      for (int bt = 0; bt < CH / 16; ++bt) {
        if (bt + 1 < CH / 16) fetch_ay(bt + 1, (bt + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) xa[i] = fmaf(av[bt & 1][u][i], yv[bt & 1][u][i], xa[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float x = tok ? (xa[0] + xa[1]) + (xa[2] + xa[3]) : 0.0f;
      sXw[l] = x;
      wave_lds_sync();
      // d_L = R_L (d_0 + sum_t x_t s_t) and the bound sum_t |x_t| s_t on this pair
      float sm[2] = {0.0f, 0.0f}, bd[2] = {0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 xv = *reinterpret_cast<const floatx4 *>(sXw + 16 * tq + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sm[0] = fmaf(xv[i], s0[4 * q + i], sm[0]);
          sm[1] = fmaf(xv[i], s1[4 * q + i], sm[1]);
          bd[0] = fmaf(fabsf(xv[i]), s0[4 * q + i], bd[0]);
          bd[1] = fmaf(fabsf(xv[i]), s1[4 * q + i], bd[1]);
        }
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        sm[e] += __shfl_xor(sm[e], 16, 64);
        sm[e] += __shfl_xor(sm[e], 32, 64);
        bd[e] += __shfl_xor(bd[e], 16, 64);
        bd[e] += __shfl_xor(bd[e], 32, 64);
      }
      const float RL = lane_bcast(Rn, L - 1);
      bool ok = true;
      float dn[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        dn[e] = RL * (d[e] + sm[e]);
        if (clamp) ok = ok && RL * (d[e] - bd[e]) >= dmin && d[e] + bd[e] <= dmax;
      }
      // publish the check and where the new d sits; the next chunk's copies
      // issued by this wave land before the barrier
      const float dsave0 = d[0], dsave1 = d[1];
      d[0] = dn[0];
      d[1] = dn[1];
      const int fl = wave_flags() | (__all(ok) ? 8 : 0);
      wait_loads();
      if (l == 0) sF[w] = fl;
      lds_barrier();  // ---- B
      const int f0 = sF[0], f1 = sF[1], f2 = sF[2], f3 = sF[3];
      if ((f0 & f1 & f2 & f3 & 8) != 0) {
        done = true;
        ++n_active;
        gflags = (f0 | f1 | f2 | f3) & 7;
        cst = Rn * x;
      } else {
        d[0] = dsave0;
        d[1] = dsave1;
      }
    }
    int u_end = L;
    if (!done) {
      // token by token in wave 0 (see scan_solve_kernel) with d gathered in LDS
      ++n_seq;
      if (tq == 0) {
        sD[c0] = d[0];
        sD[c0 + 1] = d[1];
      }
      wait_loads();
      lds_barrier();
      if (w == 0) {
        float dv[2] = {sD[2 * l], sD[2 * l + 1]};
        const uint64_t stay = clamp ? wk.stay[seq * N + n] : 0;
        for (int u = 0; u < L; ++u) {
          float k[2], sq[2];
          lds_get<TIn, 2>(R + u * RP + 2 * l, k);
          sq[0] = k[0] * k[0];
          sq[1] = k[1] * k[1];
          const float align = wave_sum(fmaf(dv[0], sq[0], dv[1] * sq[1]));
          const float c = fmaf(-lane_bcast(eb, u), align, lane_bcast(ea, u));
          const float rb = lane_bcast(rt, u);
          cst = l == u ? c : cst;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float xx = fmaf(c, sq[e], rb * dv[e]);
            if (clamp) xx = fminf(fmaxf(xx, dmin), dmax);
            dv[e] = xx;
          }
          if (clamp && u + 1 < L) {
            // tokens u + 1 .. L - 1 all keep d on d_min?
            const uint64_t rest = (L - u - 1 >= 64 ? ~0ull : ((1ull << (L - u - 1)) - 1)) << (u + 1);
            if ((stay & rest) == rest && __all(dv[0] == dmin && dv[1] == dmin)) {
              u_end = u + 1;
              break;
            }
          }
        }
        sD[2 * l] = dv[0];
        sD[2 * l + 1] = dv[1];
      }
      lds_barrier();
      d[0] = sD[c0];
      d[1] = sD[c0 + 1];
      if (l == 0) sF[w] = wave_flags();
      lds_barrier();
      gflags = sF[0] | sF[1] | sF[2] | sF[3];
      lds_barrier();  // sD, sF are rewritten by the next chunk
    }
    if (w == 0) {
      pend_c = cst;
      pend_gi = tok && l < u_end ? gi : -1;
    }
    have = pf;
    ahave = ahave_next;
  }
  if (w == 0 && pend_gi >= 0) wk.cstep[pend_gi] = pend_c;
  if (a.d_out) {
    if (tq == 0) {
      a.d_out[seq * RP + c0] = d[0];
      a.d_out[seq * RP + c0 + 1] = d[1];
    }
  }
  if (w == 0 && l == 0) {
    wk.flags[3 * seq + 0] = n_pinned;
    wk.flags[3 * seq + 1] = n_active;
    wk.flags[3 * seq + 2] = n_seq;
  }
}

// ---------------------------------------------------------------- emit
template <typename T, int EPL>
__device__ __forceinline__ typename RowVec<T, EPL>::type pack_row(const float (&x)[EPL]) {
  typename RowVec<T, EPL>::type v;
  if constexpr (EPL == 1) {
    v = from_f32<T>(x[0]);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = from_f32<T>(x[e]);
  }
  return v;
}

template <typename T, int EPL, bool FULL>
__device__ __forceinline__ void store_vec(T *p, int lane, int64_t K, const typename RowVec<T, EPL>::type &v) {
  if constexpr (FULL) {
    *reinterpret_cast<typename RowVec<T, EPL>::type *>(p + lane * EPL) = v;
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int64_t c = (int64_t)lane * EPL + e;
      if constexpr (EPL == 1) {
        if (c < K) p[c] = v;
      } else {
        if (c < K) p[c] = v[e];
      }
    }
  }
}

// Rows of one chunk: the write keys of a group of rows are computed into
// registers and then stored together, so that the stores never sit in the
// memory counter ahead of row loads that are still awaited.
template <typename TIn, int EPL, bool FULL, bool WKT, bool WRES, bool WHOLE, bool RV = false>
__device__ __forceinline__ void emit_rows(const Row<TIn, EPL, FULL> (&rows)[CH], float (&d)[EPL], float cv, float rv,
                                          float lo, float hi, int L, TIn *op, bf16 *rp, int64_t stride, int lane,
                                          int64_t K, const Row<float, EPL, FULL> *rvrows = nullptr) {
  typedef typename RowVec<TIn, EPL>::type VK;
  typedef typename RowVec<bf16, EPL>::type VR;
  constexpr int OUTW = (WKT ? (int)sizeof(VK) : 0) + (WRES ? (int)sizeof(VR) : 0);
  constexpr int G = OUTW * CH <= 512 ? CH : 16;  // rows per store group (<= 128 words held)
#pragma unroll
  for (int g = 0; g < CH; g += G) {
    VK okt[WKT ? G : 1];
    VR ores[WRES ? G : 1];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int u = g + i;
      if (WHOLE || u < L) {
        float k[EPL];
        rows[u].get(k);
        if constexpr (WKT) {
          float w[EPL];
#pragma unroll
          for (int e = 0; e < EPL; ++e) w[e] = d[e] * k[e];
          okt[i] = pack_row<TIn, EPL>(w);
        }
        if constexpr (WRES) {
          float w[EPL];
#pragma unroll
          for (int e = 0; e < EPL; ++e) w[e] = (d[e] - 1.0f) * k[e];  // d - 1 is exact on [0.5, 2]
          ores[i] = pack_row<bf16, EPL>(w);
        }
        const float c = lane_bcast(cv, u);
        float r[EPL];
        if constexpr (RV) {
          rvrows[u].get(r);
        } else {
          const float rb = lane_bcast(rv, u);
#pragma unroll
          for (int e = 0; e < EPL; ++e) r[e] = rb;
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) d[e] = fminf(fmaxf(fmaf(c, k[e] * k[e], r[e] * d[e]), lo), hi);
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int u = g + i;
      if (WHOLE || u < L) {
        if constexpr (WKT) store_vec<TIn, EPL, FULL>(op + u * stride, lane, K, okt[i]);
        if constexpr (WRES) store_vec<bf16, EPL, FULL>(rp + u * stride, lane, K, ores[i]);
      }
    }
  }
}

template <typename TIn, int EPL, bool FULL, bool HAS_R, bool WKT, bool WRES, bool VL, bool RV = false>
__global__ __launch_bounds__(64) void scan_emit_kernel(ScanArgs a, ScanWork wk, int64_t N) {
  const int lane = threadIdx.x;
  const int64_t seq = blockIdx.x / N, n = blockIdx.x % N;
  const int64_t H = a.H, K = a.K;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t t0 = n * CH;
  if (VL && t0 >= T) return;  // past a shorter sequence's end
  const int L = (int)((T - t0) < CH ? (T - t0) : CH);
  const int64_t stride = H * K;
  const int64_t row0 = ((tb + t0) * H + h) * K;
  // per-token scalars and the chunk-start d are loaded before the rows, so
  // waiting for them does not wait for the rows
  const int64_t gi = (tb + t0 + (lane < L ? lane : 0)) * H + h;
  const float cv = wk.cstep[gi];
  const float rv = HAS_R ? a.r[gi] : 1.0f;
  // a chunk the solve pass took as pinned (marked 2) starts from d_min and
  // has no stored start
  const bool pinned = wk.pin[seq * N + n] == 2;
  float d[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int64_t c = (int64_t)lane * EPL + e;
    d[e] = c < K ? wk.dstart[(seq * N + n) * K + c] : 0.0f;
  }
  const TIn *kp = static_cast<const TIn *>(a.k) + row0;
  Row<TIn, EPL, FULL> rows[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) rows[u].load(kp + (u < L ? u : L - 1) * stride, lane, K);
  Row<float, EPL, FULL> rvrows[RV ? CH : 1];
  if constexpr (RV) {
    const float *rp0 = a.r + row0;
#pragma unroll
    for (int u = 0; u < CH; ++u) rvrows[u].load(rp0 + (u < L ? u : L - 1) * stride, lane, K);
  }
  if (pinned) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) d[e] = a.d_min;
  }
  // without the box, clip to (-inf, inf) is the identity
  const float lo = a.clamp ? a.d_min : -INFINITY, hi = a.clamp ? a.d_max : INFINITY;
  TIn *op = WKT ? static_cast<TIn *>(a.k_tilde) + row0 : nullptr;
  bf16 *rp = WRES ? static_cast<bf16 *>(a.kt_res) + row0 : nullptr;
  if (L == CH)
    emit_rows<TIn, EPL, FULL, WKT, WRES, true, RV>(rows, d, cv, rv, lo, hi, L, op, rp, stride, lane, K, rvrows);
  else
    emit_rows<TIn, EPL, FULL, WKT, WRES, false, RV>(rows, d, cv, rv, lo, hi, L, op, rp, stride, lane, K, rvrows);
}

template <typename TIn, int EPL, bool FULL, bool HAS_R, bool VL, bool RV>
void launch_emit(const ScanArgs &a, const ScanWork &w, int64_t N, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.H * N)), block(64);
  if (a.k_tilde && a.kt_res)
    hipLaunchKernelGGL((scan_emit_kernel<TIn, EPL, FULL, HAS_R, true, true, VL, RV>), grid, block, 0, s, a, w, N);
  else if (a.kt_res)
    hipLaunchKernelGGL((scan_emit_kernel<TIn, EPL, FULL, HAS_R, false, true, VL, RV>), grid, block, 0, s, a, w, N);
  else
    hipLaunchKernelGGL((scan_emit_kernel<TIn, EPL, FULL, HAS_R, true, false, VL, RV>), grid, block, 0, s, a, w, N);
  prof_mark(s, "scan_emit_kernel");
}

template <typename TIn, int EPL, bool FULL, bool HAS_R, bool VL, bool RV = false>
hipError_t launch_all(const ScanArgs &a, const ScanWork &w, hipStream_t s, bool emit) {
  const int64_t N = (a.T + CH - 1) / CH;
  const int64_t nseq = a.B * a.H;
  if (N > 0) {
    if constexpr (RV) {
      if (a.K == 128)
        hipLaunchKernelGGL((scan_prep128_kernel<TIn, false, VL, true>), dim3((unsigned)((nseq * N + 3) / 4)),
                           dim3(256), 0, s, a, w, N);
      else
        hipLaunchKernelGGL((scan_prep_kernel<TIn, EPL, FULL, false, VL, true>), dim3((unsigned)(nseq * N)),
                           dim3(64), 0, s, a, w, N);
    } else if (a.K == 128) {
      hipLaunchKernelGGL((scan_prep128_kernel<TIn, HAS_R, VL>), dim3((unsigned)((nseq * N + 3) / 4)), dim3(256), 0, s,
                         a, w, N);
    } else {
      hipLaunchKernelGGL((scan_prep_kernel<TIn, EPL, FULL, HAS_R, VL>), dim3((unsigned)(nseq * N)), dim3(64), 0, s,
                         a, w, N);
    }
    prof_mark(s, "scan_prep_kernel");
    if constexpr (!RV) {
      hipLaunchKernelGGL((scan_factor_kernel<TIn, EPL, FULL, HAS_R, VL>), dim3((unsigned)(nseq * N)), dim3(64), 0, s,
                         a, w, N);
      prof_mark(s, "scan_factor_kernel");
    }
  }
  if constexpr (!RV && EPL == 2 && FULL) {
    // K = 128: four waves per (b,h)
    constexpr size_t shm = solve4_lds_bytes<TIn>();
    static_assert(shm <= 160 * 1024, "solve kernel LDS");
    auto kern = scan_solve4_kernel<TIn, HAS_R, VL>;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nseq), dim3(256), shm, s, a, w, N);
  } else {
    // register prefetch of the next chunk's rows where they do not come by direct copies
    constexpr bool PF = !RV && !solve_rows_dma<TIn, EPL, FULL, RV>() && Row<TIn, EPL, FULL>::WORDS <= 2;
    constexpr size_t shm = solve_lds_bytes<TIn, EPL, FULL, RV>();
    static_assert(shm <= 160 * 1024, "solve kernel LDS");
    auto kern = scan_solve_kernel<TIn, EPL, FULL, HAS_R, PF, VL, RV>;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nseq), dim3(64), shm, s, a, w, N);
  }
  prof_mark(s, "scan_solve_kernel");
  if (N > 0 && emit) launch_emit<TIn, EPL, FULL, HAS_R, VL, RV>(a, w, N, s);
  return hipGetLastError();
}

template <typename TIn, int EPL, bool FULL, bool VL>
hipError_t launch_r(const ScanArgs &a, const ScanWork &w, hipStream_t s, bool e) {
  if (a.r && a.r_per_key) {
    if constexpr (EPL <= 2) return launch_all<TIn, EPL, FULL, false, VL, true>(a, w, s, e);
    return hipErrorInvalidValue;  // vector retention above K = 128 takes the token-by-token kernel
  }
  return a.r ? launch_all<TIn, EPL, FULL, true, VL>(a, w, s, e) : launch_all<TIn, EPL, FULL, false, VL>(a, w, s, e);
}

template <typename TIn, bool VL>
hipError_t launch_typed(const ScanArgs &a, const ScanWork &w, hipStream_t s, bool e) {
  if (a.K <= 64) return a.K == 64 ? launch_r<TIn, 1, true, VL>(a, w, s, e) : launch_r<TIn, 1, false, VL>(a, w, s, e);
  if (a.K <= 128)
    return a.K == 128 ? launch_r<TIn, 2, true, VL>(a, w, s, e) : launch_r<TIn, 2, false, VL>(a, w, s, e);
  return a.K == 256 ? launch_r<TIn, 4, true, VL>(a, w, s, e) : launch_r<TIn, 4, false, VL>(a, w, s, e);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t scan_work_bytes(int64_t B, int64_t T, int64_t H, int64_t K) {
  const int64_t N = (T + CH - 1) / CH;
  return 2 * align256((size_t)(B * T * H) * 4) + align256((size_t)(B * H * N * K) * 4) +
         align256((size_t)(B * H * N) * 4) + align256((size_t)(B * H * N) * 8) + align256((size_t)(B * H) * 3 * 4) +
         align256((size_t)(B * H * N) * 4) + align256((size_t)(B * H * N) * CH * CH * 4);
}

ScanWork scan_work_layout(void *base, int64_t B, int64_t T, int64_t H, int64_t K) {
  const int64_t N = (T + CH - 1) / CH;
  char *p = static_cast<char *>(base);
  const size_t tok = align256((size_t)(B * T * H) * 4);
  const size_t dst = align256((size_t)(B * H * N * K) * 4);
  const size_t pin = align256((size_t)(B * H * N) * 4);
  const size_t stay = align256((size_t)(B * H * N) * 8);
  ScanWork w;
  w.norm = reinterpret_cast<float *>(p);
  w.cstep = reinterpret_cast<float *>(p + tok);
  w.dstart = reinterpret_cast<float *>(p + 2 * tok);
  w.pin = reinterpret_cast<int *>(p + 2 * tok + dst);
  w.stay = reinterpret_cast<uint64_t *>(p + 2 * tok + dst + pin);
  w.flags = reinterpret_cast<int *>(p + 2 * tok + dst + pin + stay);
  const size_t flags = align256((size_t)(B * H) * 3 * 4);
  w.fok = reinterpret_cast<int *>(p + 2 * tok + dst + pin + stay + flags);
  w.ainv = reinterpret_cast<float *>(p + 2 * tok + dst + 2 * pin + stay + flags);
  return w;
}

hipError_t launch_precond_scan_chunked(const ScanArgs &a, const ScanWork &w, bool is_bf16, hipStream_t s,
                                       bool emit) {
  if (a.B * a.H == 0) return hipSuccess;
  if (a.cu) return is_bf16 ? launch_typed<bf16, true>(a, w, s, emit) : launch_typed<float, true>(a, w, s, emit);
  return is_bf16 ? launch_typed<bf16, false>(a, w, s, emit) : launch_typed<float, false>(a, w, s, emit);
}

}  // namespace osdn
