// Phase 2 of OSDN on the matrix cores: chunkwise WY delta rule, bf16 operands,
// fp32 accumulation, K = V = 128, chunk C = 64.
//
// Paper: Section 4.3 Eq.(5)-(6) (write key K~ in the chunk Gram and in the
// intra-chunk score, physical key K in the residual), Appendix A.2
// Eqs.(8)-(11); with a decay alpha, Appendix B.1 Eqs.(13)-(15).  Per chunk,
// with boundary state S (V x K, fp32), B = diag(beta) and in-chunk log decay
// g_i = sum_{l<=i} log alpha_l (g = 0 without decay):
//   A     = strict_lower(B [e^{g_i-g_j}] . K K~^T)
//   Tm    = (I + A)^-1            (forward substitution on the 16x16 diagonal
//                                  blocks, MFMA merges of the off-diagonal ones)
//   R     = B (V - diag(e^g) K S^T)
//   Delta = Tm R                  (= U - W S^T of Eq.(11))
//   O     = q_scale (diag(e^g) Q S^T + lower([e^{g_i-g_j}] . Q K~^T) Delta)
//   S    <- e^{g_L} S + Delta^T (e^{g_L - g} . K~)
//
// Precision: every MFMA takes bf16 operands and accumulates in fp32.  Inputs
// q, k, k~, v are bf16 already.  Intermediates that are not (S, R, Delta and
// the scores) enter as a hi + lo pair of bf16 (x_hi = bf16(x), x_lo =
// bf16(x - x_hi)), i.e. about 16 significant bits, so the only 8-bit roundings
// left are Tm and the bf16 output itself.  The write keys arrive either as
// bf16 k~ (exact operands) or as the bf16 residual E = (d - 1) (.) k, in which
// case k~ = k + E is formed in fp32 and also enters as a hi + lo pair.
//
// Work split: one workgroup of 4 waves per (b,h) and tile of VT value rows,
// so a (b,h) is spread over 128/VT CUs; the tiles of one (b,h) are placed on
// the same XCD so their shared K/K~/Q reads hit that XCD's L2.  Inside the
// workgroup wave w owns tokens [16w, 16w+16) of the chunk; its K and Q rows go
// straight from global memory into registers in MFMA operand layout.
#include "kernels.h"
#include "mfma_common.h"
#include "profile.h"

namespace osdn {

namespace {

constexpr int C = 64;      // chunk length
constexpr int KD = 128;    // key dim
constexpr int VD = 128;    // value dim
constexpr int KP = KD + 8; // LDS pitch (bf16) of 128-wide rows
constexpr int CP = C + 8;  // LDS pitch (bf16) of 64-wide rows
constexpr int AP = C + 4;  // LDS pitch (f32) of the Gram
constexpr int NTHREADS = 256;

// LDS layout (bytes).  Buffers that are never live at the same time share
// the SX region: the bf16 state pair (written after the state update, read by
// the next chunk's products) and the scratch of the inverse.
template <int VT> struct Lay {
  static constexpr int KT = 0;                        // bf16 [C][KP]   write keys
  static constexpr int KTT = KT + C * KP * 2;         // bf16 [KD][CP]  write keys^T
  static constexpr int V = KTT + KD * CP * 2;         // bf16 [C][VT+8] value tile
  static constexpr int BETA = V + C * (VT + 8) * 2;   // f32 [C]
  static constexpr int G = BETA + C * 4;              // f32 [C]       cumulative log decay
  static constexpr int MH = G + C * 4;                // bf16 [C][CP]  scores, hi
  static constexpr int ML = MH + C * CP * 2;          // bf16 [C][CP]  scores, lo
  static constexpr int RTH = ML + C * CP * 2;         // bf16 [VT][CP] R^T hi
  static constexpr int RTL = RTH + VT * CP * 2;       // bf16 [VT][CP] R^T lo
  static constexpr int TR = RTL + VT * CP * 2;        // bf16 [C][CP]  (I+A)^-1 row-major
  static constexpr int SX = TR + C * CP * 2;          // union below
  static constexpr int SH = SX;                       //   bf16 [VT][KP] state hi
  static constexpr int SL = SX + VT * KP * 2;         //   bf16 [VT][KP] state lo
  static constexpr int TC = SX;                       //   bf16 [C][CP] (I+A)^-1 column-major
  static constexpr int X = SX + C * CP * 2;           //   bf16 [C][CP] merge scratch
  static constexpr int SX_BYTES = (2 * VT * KP > 2 * C * CP ? 2 * VT * KP : 2 * C * CP) * 2;
  // the gated Gram lives in the Delta^T buffers: it is written by the
  // products stage and read by the inverse, both before Delta exists
  static constexpr int A = SX + SX_BYTES;             // f32 [C][AP]
  static constexpr int DTH = SX + SX_BYTES;           // bf16 [VT][CP] Delta^T hi
  static constexpr int DTL = DTH + VT * CP * 2;       // bf16 [VT][CP] Delta^T lo
  static constexpr int DSH = DTL + VT * CP * 2;       // bf16 [VT][CP] decayed Delta^T hi
  static constexpr int DSL = DSH + VT * CP * 2;       // bf16 [VT][CP] decayed Delta^T lo
  static constexpr int DT_END = DSL + VT * CP * 2;
  static constexpr int KTL = DT_END;                  // bf16 [C][KP]  write keys, lo part
  static constexpr int KTTL = KTL + C * KP * 2;       // bf16 [KD][CP] write keys^T, lo part
  static constexpr int TOTAL = KTTL + KD * CP * 2;
};

template <int VT, bool GATED, bool KRES>
__global__ __launch_bounds__(NTHREADS) void chunk_mfma_kernel(ChunkArgs a) {
  constexpr int NT = VD / VT;   // value tiles per (b,h)
  constexpr int NCT = VT / 16;  // 16-wide column tiles per value tile
  constexpr int VV = VT / 8;    // 16-byte vectors per value-tile row
  typedef Lay<VT> L;
  static_assert(L::TOTAL <= 160 * 1024, "LDS budget");
  static_assert(L::A + C * AP * 4 <= L::DT_END, "Gram must fit in the Delta buffers");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  bf16(*sKt)[KP] = reinterpret_cast<bf16(*)[KP]>(smem + L::KT);
  bf16(*sKtT)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::KTT);
  bf16(*sKtL)[KP] = reinterpret_cast<bf16(*)[KP]>(smem + L::KTL);
  bf16(*sKtTL)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::KTTL);
  bf16(*sV)[VT + 8] = reinterpret_cast<bf16(*)[VT + 8]>(smem + L::V);
  float *sBeta = reinterpret_cast<float *>(smem + L::BETA);
  float *sG = reinterpret_cast<float *>(smem + L::G);
  float(*sA)[AP] = reinterpret_cast<float(*)[AP]>(smem + L::A);
  bf16(*sMh)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::MH);
  bf16(*sMl)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::ML);
  bf16(*sRh)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::RTH);
  bf16(*sRl)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::RTL);
  bf16(*sTr)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::TR);
  bf16(*sSh)[KP] = reinterpret_cast<bf16(*)[KP]>(smem + L::SH);
  bf16(*sSl)[KP] = reinterpret_cast<bf16(*)[KP]>(smem + L::SL);
  bf16(*sTc)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::TC);
  bf16(*sX)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::X);
  bf16(*sDh)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::DTH);
  bf16(*sDl)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::DTL);
  bf16(*sDsh)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + (GATED ? L::DSH : L::DTH));
  bf16(*sDsl)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + (GATED ? L::DSL : L::DTL));

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = l & 15, lq = l >> 4;
  // XCD-aware placement: block i runs on XCD i % 8; the NT tiles of one
  // sequence share i % 8.
  const int bid = blockIdx.x;
  const int slot = bid & 7, rest = bid >> 3;
  const int vt = rest % NT;
  const int64_t seq = (int64_t)(rest / NT) * 8 + slot;
  const int64_t H = a.H, T = a.T;
  if (seq >= a.B * H) return;
  const int64_t b = seq / H, h = seq - b * H;
  const int v0 = vt * VT;

  const bf16 *gq = static_cast<const bf16 *>(a.q);
  const bf16 *gk = static_cast<const bf16 *>(a.k);
  const bf16 *gkt = static_cast<const bf16 *>(a.kt);
  const bf16 *gv = static_cast<const bf16 *>(a.v);
  const int64_t tstride = H * KD;                 // elements between tokens (K == V == 128)
  const int64_t base = (b * T) * tstride + h * KD;  // token 0 of this (b,h)

  // ---- state tile in accumulators: wave w owns columns [32w, 32w+32) of the
  //      VT x 128 tile as NCT x 2 MFMA tiles; element i of tile (rt, ct) is
  //      S[16 rt + 4 lq + i][32 w + 16 ct + l16].
  floatx4 Sacc[NCT][2];
#pragma unroll
  for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int vr = 16 * rt + 4 * lq + i, c = 32 * w + 16 * ct + l16;
        const float s0 = a.S0 ? a.S0[(seq * VD + v0 + vr) * KD + c] : 0.0f;
        Sacc[rt][ct][i] = s0;
        const bf16 hi = to_bf16(s0);
        sSh[vr][c] = hi;
        sSl[vr][c] = to_bf16(s0 - to_f32(hi));
      }

  // ---- prefetch registers for one chunk
  //   write keys: lane l loads token l, columns [8(4w+p), 8(4w+p)+8), p < 4
  //   values:     vectors tid (+256 p) of the 64 x VT tile
  //   K, Q:       wave w's 16 tokens in MFMA A-operand layout (4 k-steps)
  bf16x8 pkt[4], pkk[4], pv[(C * VV + NTHREADS - 1) / NTHREADS], pk[4], pq[4];
  float pbeta = 0.0f, palpha = 1.0f;
  auto fetch = [&](int64_t t0) {
    {
      const int64_t t = t0 + l;
      const bool ok = t < T;
      const int64_t off = base + (ok ? t : 0) * tstride;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        bf16x8 x = ld8(gkt + off + 8 * (4 * w + p));
        pkt[p] = ok ? x : bf16x8{};
        if (KRES) {
          bf16x8 y = ld8(gk + off + 8 * (4 * w + p));
          pkk[p] = ok ? y : bf16x8{};
        }
      }
    }
#pragma unroll
    for (int p = 0; p < (C * VV + NTHREADS - 1) / NTHREADS; ++p) {
      const int vi = tid + NTHREADS * p;
      const int i = vi / VV, cv = vi % VV;
      const int64_t t = t0 + i;
      const bool ok = vi < C * VV && t < T;
      bf16x8 x = ld8(gv + base + (ok ? t : 0) * tstride + v0 + (ok ? cv * 8 : 0));
      pv[p] = ok ? x : bf16x8{};
    }
    {
      const int64_t t = t0 + 16 * w + l16;
      const bool ok = t < T;
      const int64_t off = base + (ok ? t : 0) * tstride + 8 * lq;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 x = ld8(gk + off + 32 * kk), y = ld8(gq + off + 32 * kk);
        pk[kk] = ok ? x : bf16x8{};
        pq[kk] = ok ? y : bf16x8{};
      }
    }
    if (w == 0) {
      const int64_t t = t0 + l;
      const bool ok = t < T;
      const int64_t gi = (b * T + (ok ? t : 0)) * H + h;
      const float bt = a.beta[gi];
      pbeta = ok ? bt : 0.0f;
      if (GATED) {
        const float al = a.alpha[gi];
        palpha = ok ? al : 1.0f;
      }
    }
  };

  if (T > 0) fetch(0);
  for (int64_t t0 = 0; t0 < T; t0 += C) {
    const int Lc = (int)((T - t0) < C ? (T - t0) : C);
    __syncthreads();  // previous chunk done with every LDS buffer
    // ---- stage L: registers -> LDS
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int c0 = 8 * (4 * w + p);
      if (KRES) {
        // k~ = k + residual in fp32 (exact), stored as a bf16 hi + lo pair
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = to_f32(pkk[p][e]) + to_f32(pkt[p][e]);
          hi[e] = to_bf16(x);
          lo[e] = to_bf16(x - to_f32(hi[e]));
        }
        *reinterpret_cast<bf16x8 *>(&sKt[l][c0]) = hi;
        *reinterpret_cast<bf16x8 *>(&sKtL[l][c0]) = lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sKtT[c0 + e][l] = hi[e];
          sKtTL[c0 + e][l] = lo[e];
        }
      } else {
        *reinterpret_cast<bf16x8 *>(&sKt[l][c0]) = pkt[p];
#pragma unroll
        for (int e = 0; e < 8; ++e) sKtT[c0 + e][l] = pkt[p][e];
      }
    }
#pragma unroll
    for (int p = 0; p < (C * VV + NTHREADS - 1) / NTHREADS; ++p) {
      const int vi = tid + NTHREADS * p;
      if (vi < C * VV) *reinterpret_cast<bf16x8 *>(&sV[vi / VV][(vi % VV) * 8]) = pv[p];
    }
    if (w == 0) {
      sBeta[l] = pbeta;
      if (GATED) {
        // inclusive scan of the log decays over the 64 lanes of wave 0
        float x = logf(palpha);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off, 64);
          if (l >= off) x += y;
        }
        sG[l] = x;
      }
    }
    bf16x8 kf[4], qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      kf[kk] = pk[kk];
      qf[kk] = pq[kk];
    }
    __syncthreads();
    if (t0 + C < T) fetch(t0 + C);  // overlaps with the compute below

    const int m0 = 16 * w;
    // ---- stage G: Gram A and scores M (tiles (w, tj), tj <= w), K S^T, Q S^T
    floatx4 accA[4], accM[4], accKS[NCT], accQS[NCT];
#pragma unroll
    for (int j = 0; j < 4; ++j) accA[j] = accM[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) accKS[ct] = accQS[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ko = 32 * kk + 8 * lq;
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        if (tj <= w) {
          const bf16x8 bk = ld8(&sKt[16 * tj + l16][ko]);
          accA[tj] = mfma32(kf[kk], bk, accA[tj]);
          accM[tj] = mfma32(qf[kk], bk, accM[tj]);
          if (KRES) {
            const bf16x8 bl = ld8(&sKtL[16 * tj + l16][ko]);
            accA[tj] = mfma32(kf[kk], bl, accA[tj]);
            accM[tj] = mfma32(qf[kk], bl, accM[tj]);
          }
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const bf16x8 sh = ld8(&sSh[16 * ct + l16][ko]), sl = ld8(&sSl[16 * ct + l16][ko]);
        accKS[ct] = mfma32(kf[kk], sh, accKS[ct]);
        accKS[ct] = mfma32(kf[kk], sl, accKS[ct]);
        accQS[ct] = mfma32(qf[kk], sh, accQS[ct]);
        accQS[ct] = mfma32(qf[kk], sl, accQS[ct]);
      }
    }
    // epilogue of the Gram / scores: lane holds rows m0 + 4 lq + i, column 16 tj + l16
    float gm[4], bm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gm[i] = GATED ? sG[m0 + 4 * lq + i] : 0.0f;
      bm[i] = sBeta[m0 + 4 * lq + i];
    }
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      if (tj <= w) {
        const int n = 16 * tj + l16;
        const float gn = GATED ? sG[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 4 * lq + i;
          const float ratio = GATED ? __expf(gm[i] - gn) : 1.0f;
          sA[m][n] = n < m ? bm[i] * ratio * accA[tj][i] : 0.0f;
          const float mv = n <= m ? ratio * accM[tj][i] : 0.0f;
          const bf16 mh = to_bf16(mv);
          sMh[m][n] = mh;
          sMl[m][n] = to_bf16(mv - to_f32(mh));
        }
      }
    }
    if ((w & 1) == 0) {
      // tiles (w, w+1) are read by the 32-wide k-steps of later products
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * lq + i, n = m0 + 16 + l16;
        sMh[m][n] = sMl[m][n] = sTr[m][n] = to_bf16(0.0f);
      }
    }
    floatx4 Oacc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      floatx4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * lq + i, vr = 16 * ct + l16;
        const float em = GATED ? __expf(gm[i]) : 1.0f;
        r[i] = bm[i] * (to_f32(sV[m][vr]) - em * accKS[ct][i]);
        Oacc[ct][i] = em * accQS[ct][i];
      }
      bf16x4 rh, rl;
      split4(r, rh, rl);
      *reinterpret_cast<bf16x4 *>(&sRh[16 * ct + l16][m0 + 4 * lq]) = rh;
      *reinterpret_cast<bf16x4 *>(&sRl[16 * ct + l16][m0 + 4 * lq]) = rl;
    }
    __syncthreads();

    // ---- stage T: (I + A)^-1 into sTr
    // (i) wave w inverts diagonal block w by forward substitution in fp32;
    //     lane l & 15 computes column c of the block inverse.
    {
      const int c = l16, bb = m0;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == c) ? 1.0f : 0.0f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= sA[bb + i][bb + j] * x[j];
        x[i] = acc;
      }
      if (lq == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sTr[bb + i][bb + c] = to_bf16(x[i]);
        bf16x8 lo8, hi8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lo8[i] = to_bf16(x[i]);
          hi8[i] = to_bf16(x[i + 8]);
        }
        *reinterpret_cast<bf16x8 *>(&sTc[bb + c][bb]) = lo8;
        *reinterpret_cast<bf16x8 *>(&sTc[bb + c][bb + 8]) = hi8;
      }
    }
    __syncthreads();
    // (ii) T_{q+1,q} = -T_{q+1,q+1} A_{q+1,q} T_{q,q}, q = 0 (wave 0), q = 2 (wave 1)
    if (w < 2) {
      const int q = 2 * w, p = q + 1;
      bf16x4 aop;
#pragma unroll
      for (int e = 0; e < 4; ++e) aop[e] = to_bf16(sA[16 * p + l16][16 * q + 4 * lq + e]);
      const floatx4 X = mfma16(aop, ld4(&sTc[16 * q + l16][16 * q + 4 * lq]), floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 Y = mfma16(ld4(&sTr[16 * p + l16][16 * p + 4 * lq]), pack4(X), floatx4{0.f, 0.f, 0.f, 0.f});
      bf16x4 nt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nt[i] = to_bf16(-Y[i]);
        sTr[16 * p + 4 * lq + i][16 * q + l16] = nt[i];
      }
      *reinterpret_cast<bf16x4 *>(&sTc[16 * q + l16][16 * p + 4 * lq]) = nt;
    }
    __syncthreads();
    // (iii) lower-left 32x32 block: X = A_BA T_AA, then T_BA = -T_BB X;
    //       wave w owns output block (p, q) = (2 + w/2, w%2).
    {
      const int p = 2 + (w >> 1), q = w & 1;
      floatx4 X = {0.f, 0.f, 0.f, 0.f};
      for (int kb = q; kb < 2; ++kb) {
        bf16x4 aop;
#pragma unroll
        for (int e = 0; e < 4; ++e) aop[e] = to_bf16(sA[16 * p + l16][16 * kb + 4 * lq + e]);
        X = mfma16(aop, ld4(&sTc[16 * q + l16][16 * kb + 4 * lq]), X);
      }
      *reinterpret_cast<bf16x4 *>(&sX[16 * q + l16][16 * p + 4 * lq]) = pack4(X);
      __syncthreads();
      floatx4 Y = {0.f, 0.f, 0.f, 0.f};
      for (int mb = 2; mb <= p; ++mb)
        Y = mfma16(ld4(&sTr[16 * p + l16][16 * mb + 4 * lq]), ld4(&sX[16 * q + l16][16 * mb + 4 * lq]), Y);
#pragma unroll
      for (int i = 0; i < 4; ++i) sTr[16 * p + 4 * lq + i][16 * q + l16] = to_bf16(-Y[i]);
    }
    __syncthreads();

    // ---- stage D: Delta = Tm R (rows of wave w), split and stored transposed
    const float gL = GATED ? sG[Lc - 1] : 0.0f;
    const int nks = w < 2 ? 1 : 2;  // 32-wide k-steps that reach the diagonal
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kk = 0; kk < nks; ++kk) {
        const int ko = 32 * kk + 8 * lq;
        const bf16x8 t = ld8(&sTr[m0 + l16][ko]);
        acc = mfma32(t, ld8(&sRh[16 * ct + l16][ko]), acc);
        acc = mfma32(t, ld8(&sRl[16 * ct + l16][ko]), acc);
      }
      bf16x4 dh, dl;
      split4(acc, dh, dl);
      *reinterpret_cast<bf16x4 *>(&sDh[16 * ct + l16][m0 + 4 * lq]) = dh;
      *reinterpret_cast<bf16x4 *>(&sDl[16 * ct + l16][m0 + 4 * lq]) = dl;
      if (GATED) {
        floatx4 s;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = acc[i] * __expf(gL - gm[i]);
        split4(s, dh, dl);
        *reinterpret_cast<bf16x4 *>(&sDsh[16 * ct + l16][m0 + 4 * lq]) = dh;
        *reinterpret_cast<bf16x4 *>(&sDsl[16 * ct + l16][m0 + 4 * lq]) = dl;
      }
    }
    __syncthreads();

    // ---- stage O: outputs of wave w's tokens
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      floatx4 acc = Oacc[ct];
      for (int kk = 0; kk < nks; ++kk) {
        const int ko = 32 * kk + 8 * lq;
        const bf16x8 mh = ld8(&sMh[m0 + l16][ko]), ml = ld8(&sMl[m0 + l16][ko]);
        const bf16x8 dh = ld8(&sDh[16 * ct + l16][ko]), dl = ld8(&sDl[16 * ct + l16][ko]);
        acc = mfma32(mh, dh, acc);
        acc = mfma32(mh, dl, acc);
        acc = mfma32(ml, dh, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * lq + i;
        if (m < Lc) store_out<bf16>(a.o, base + (t0 + m) * tstride + v0 + 16 * ct + l16, a.q_scale * acc[i], a.o_f32);
      }
    }
    // ---- stage S: state update, then its bf16 pair for the next chunk
    const float decay = GATED ? __expf(gL) : 1.0f;
#pragma unroll
    for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        floatx4 acc = Sacc[rt][ct];
        if (GATED) acc = acc * decay;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ko = 32 * kk + 8 * lq;
          const bf16x8 kt = ld8(&sKtT[32 * w + 16 * ct + l16][ko]);
          const bf16x8 dsh = ld8(&sDsh[16 * rt + l16][ko]);
          acc = mfma32(dsh, kt, acc);
          acc = mfma32(ld8(&sDsl[16 * rt + l16][ko]), kt, acc);
          if (KRES) acc = mfma32(dsh, ld8(&sKtTL[32 * w + 16 * ct + l16][ko]), acc);
        }
        Sacc[rt][ct] = acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int vr = 16 * rt + 4 * lq + i, c = 32 * w + 16 * ct + l16;
          const bf16 hi = to_bf16(acc[i]);
          sSh[vr][c] = hi;
          sSl[vr][c] = to_bf16(acc[i] - to_f32(hi));
        }
      }
  }

  if (a.S_out) {
#pragma unroll
    for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int vr = 16 * rt + 4 * lq + i, c = 32 * w + 16 * ct + l16;
          a.S_out[(seq * VD + v0 + vr) * KD + c] = Sacc[rt][ct][i];
        }
  }
}

template <int VT>
hipError_t launch_vt(const ChunkArgs &a, hipStream_t s) {
  constexpr int NT = VD / VT;
  const int64_t nseq = a.B * a.H;
  const int64_t groups = (nseq + 7) / 8;
  dim3 grid((unsigned)(groups * 8 * NT)), block(NTHREADS);
  if (a.alpha) {
    if (a.kt_is_res)
      hipLaunchKernelGGL((chunk_mfma_kernel<VT, true, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((chunk_mfma_kernel<VT, true, false>), grid, block, 0, s, a);
  } else {
    if (a.kt_is_res)
      hipLaunchKernelGGL((chunk_mfma_kernel<VT, false, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((chunk_mfma_kernel<VT, false, false>), grid, block, 0, s, a);
  }
  prof_mark(s, "chunk_mfma_kernel");
  return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs &a, bool is_bf16) {
  return is_bf16 && a.K == KD && a.V == VD && a.C == C;
}

hipError_t launch_chunk_mfma(const ChunkArgs &a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  return launch_vt<32>(a, s);
}

}  // namespace osdn
