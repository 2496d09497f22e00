// Phase 2 of OSDN on the matrix cores, two kernels: the state-independent UT
// transform of every chunk first, chunk-parallel, then the sweep over chunks
// that carries the state.  bf16 operands, fp32 accumulation, K = V = 128,
// chunk C = 64.
//
// Paper: Section 4.3 Eq.(5)-(6) (write key K~ in the chunk Gram and in the
// intra-chunk score, physical key K in the residual), Appendix A.2
// Eqs.(8)-(11); with a decay alpha, Appendix B.1 Eqs.(13)-(15).  Per chunk,
// with B = diag(beta) and in-chunk log decay g_i = sum_{l<=i} log alpha_l
// (g = 0 without decay):
//
//  chunk_tinv_kernel (one workgroup per chunk, all chunks at once):
//    A  = strict_lower(B [e^{g_i-g_j}] . K K~^T)
//    Tm = (I + A)^-1, written to the workspace in bf16 (row-major 64 x 64)
//
//  chunk_seq_kernel (one workgroup per (b,h) and 32 value rows, chunks in
//  order; S is the boundary state, V x K, fp32):
//    R     = B (V - diag(e^g) K S^T)
//    Delta = Tm R                                     (= U - W S^T of Eq.(11))
//    O     = q_scale (diag(e^g) Q S^T + lower([e^{g_i-g_j}] . Q K~^T) Delta)
//    S    <- e^{g_L} S + Delta^T (e^{g_L - g} . K~)
//
// Tm depends only on the chunk's keys, so the sweep carries no triangular
// solve: its per-chunk work is five small products, split over 8 waves (wave
// (rw, cw) owns token rows [16 rw, 16 rw + 16) and value columns
// [16 cw, 16 cw + 16) of the chunk), with four barriers per chunk.  Each
// input row is loaded once per workgroup and staged in LDS; the key rows
// serve both as row operands and, through transposed LDS reads, as the
// token-major operand of the state update.
//
// Precision: intermediates that are not bf16 (S, R, Delta, the scores) enter
// every product as a hi + lo pair of bf16; the write key in its residual form
// k~ = k + E enters as the pair (k, E), both exact; Tm and the output are the
// only 8-bit roundings.
#include "kernels.h"
#include "mfma_common.h"
#include "profile.h"

namespace osdn {

namespace {

constexpr int C = 64;      // chunk length
constexpr int KD = 128;    // key dim
constexpr int VD = 128;    // value dim
constexpr int VT = 32;     // value rows per sweep workgroup
constexpr int NT = VD / VT;
constexpr int KP = KD + 16; // LDS pitch (bf16) of the sweep's 128-wide rows: 288 B keeps 16-row operand reads conflict-free
constexpr int TKP = KD + 8; // the same in the UT transform, whose workgroups must fit three to a CU
constexpr int CP = C + 8;  // LDS pitch (bf16) of 64-wide rows
constexpr int AP = C + 4;  // LDS pitch (f32) of the Gram

template <int N>
struct IConst {
  static constexpr int value = N;
};

// ============================================================ UT transform
struct TinvLay {
  // the key rows are dead once the Gram is formed; the inverse reuses them
  static constexpr int KH = 0;                   // bf16 [C][TKP] write keys, or residual E
  static constexpr int KL = KH + C * TKP * 2;    // bf16 [C][TKP] keys (residual form)
  static constexpr int TR = 0;                   // bf16 [C][CP] Tm row-major
  static constexpr int TC = TR + C * CP * 2;     // bf16 [C][CP] Tm column-major
  static constexpr int X = TC + C * CP * 2;      // bf16 [C][CP] merge scratch
  static constexpr int R0 = KL + C * TKP * 2;
  static constexpr int A = R0;                   // f32 [C][AP]
  static constexpr int BETA = A + C * AP * 4;    // f32 [C]
  static constexpr int G = BETA + C * 4;         // f32 [C]
  static constexpr int SC = G + C * 4;           // f32 [C] phase-1 step scalars (EMIT)
  static constexpr int SR = SC + C * 4;          // f32 [C] retention (EMIT)
  static constexpr int TOTAL = SR + C * 4;
  static_assert(X + C * CP * 2 <= R0, "inverse scratch must fit in the key rows");
};

// EMIT (residual form only): the chunk's residual E = (d - 1) (.) k is formed
// here from the phase-1 sweep's chunk start and step scalars -- the replay
// d_{t+1} = clip(r_t d_t + c_t k_t^2), the same fp32 expressions as the
// phase-1 emit kernel -- and written for the sweep kernel, so phase 1 need
// not write it and this kernel need not read it.
template <bool GATED, bool KRES, bool EMIT, bool VL, bool RVEC = false>
__global__ __launch_bounds__(256) void chunk_tinv_kernel(ChunkArgs a, bf16 *tout, int64_t N, EmitArgs em) {
  static_assert(KRES || !EMIT, "the folded replay produces the residual form");
  typedef TinvLay L;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  bf16(*sKh)[TKP] = reinterpret_cast<bf16(*)[TKP]>(smem + L::KH);
  bf16(*sKl)[TKP] = reinterpret_cast<bf16(*)[TKP]>(smem + L::KL);
  bf16(*sTr)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::TR);
  bf16(*sTc)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::TC);
  bf16(*sX)[CP] = reinterpret_cast<bf16(*)[CP]>(smem + L::X);
  float(*sA)[AP] = reinterpret_cast<float(*)[AP]>(smem + L::A);
  float *sBeta = reinterpret_cast<float *>(smem + L::BETA);
  float *sG = reinterpret_cast<float *>(smem + L::G);
  float *sC = reinterpret_cast<float *>(smem + L::SC);
  float *sR = reinterpret_cast<float *>(smem + L::SR);

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = l & 15, lq = l >> 4;
  const int64_t H = a.H;
  const bf16 *gk = static_cast<const bf16 *>(a.k);
  const bf16 *gkt = static_cast<const bf16 *>(a.kt);
  const int64_t tstride = H * KD;
  const int64_t nch = a.B * H * N;
  // Each workgroup takes chunks blockIdx.x, blockIdx.x + gridDim.x, ...; the
  // next chunk's key rows (and write-key rows off the folded path), beta,
  // alpha and pin word are loaded into registers while this one is computed.
  bf16x8 px[4], pe[4];
  float pb = 0.0f, pa = 1.0f;
  int ppin = 0;
  auto fetch = [&](int64_t ci) {
    const int64_t seq = ci / N, n = ci - seq * N;
    const int64_t b = seq / H, h = seq - b * H;
    const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
    const int64_t t0 = n * C;
    if (VL && t0 >= T) return;  // past a shorter sequence's end: skipped below
    const int Lc = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t base = (tb + t0) * tstride + h * KD;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int vi = tid + 256 * p, i = vi >> 4, c8 = 8 * (vi & 15);
      const int64_t off = base + (i < Lc ? i : 0) * tstride + c8;
      px[p] = ld8(gk + off);
      if constexpr (!EMIT) pe[p] = ld8(gkt + off);
    }
    if (w == 0) {
      const int64_t gi = (tb + t0 + (l < Lc ? l : 0)) * H + h;
      pb = a.beta[gi];
      if constexpr (GATED) pa = a.alpha[gi];
    }
    if constexpr (EMIT) ppin = em.pin[ci];
  };
  if ((int64_t)blockIdx.x < nch) fetch(blockIdx.x);
  for (int64_t ci = blockIdx.x; ci < nch; ci += gridDim.x) {
  const int64_t seq = ci / N, n = ci - seq * N;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t t0 = n * C;
  if (VL && t0 >= T) {
    // past a shorter sequence's end (the whole workgroup alike): nothing to
    // form; the next chunk's loads still go out
    if (ci + (int64_t)gridDim.x < nch) fetch(ci + gridDim.x);
    continue;
  }
  const int Lc = (int)((T - t0) < C ? (T - t0) : C);
  const int64_t base = (tb + t0) * tstride + h * KD;  // token t0 of this (b,h)

  // ---- this chunk's rows into LDS (16-byte vectors, 16 threads per row;
  //      zero past T), beta and the cumulative log decay
  // A chunk the phase-1 sweep took as pinned (marked 2) starts from d_min,
  // and its mark guarantees that every step clips back to d_min (the mark
  // tests the replay's own fp32 expression at the largest key square), so
  // its residual is E = (d_min - 1) k, computed here in parallel and bitwise
  // equal to the token-by-token replay below.
  const bool pinned = EMIT && __builtin_amdgcn_readfirstlane(ppin) == 2;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int vi = tid + 256 * p, i = vi >> 4, c8 = 8 * (vi & 15);
    *reinterpret_cast<bf16x8 *>(&sKl[i][c8]) = i < Lc ? px[p] : bf16x8{};
    if constexpr (EMIT) {
      if (pinned) {
        const float dm1 = em.d_min - 1.0f;  // exact on [0.5, 2]
        bf16x8 e;
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = to_bf16(dm1 * to_f32(px[p][q]));
        *reinterpret_cast<bf16x8 *>(&sKh[i][c8]) = i < Lc ? e : bf16x8{};
      }
    } else {
      // write keys (with the residual form k~ = k + E both k and E are exact
      // bf16 operands, so the Gram is K E^T + K K^T; otherwise the bf16 k~
      // rows themselves)
      *reinterpret_cast<bf16x8 *>(&sKh[i][c8]) = i < Lc ? pe[p] : bf16x8{};
    }
  }
  if (w == 0) {
    const bool ok = l < Lc;
    sBeta[l] = ok ? pb : 0.0f;
    if constexpr (GATED) {
      float x = ok ? logf(pa) : 0.0f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (l >= off) x += y;
      }
      sG[l] = x;
    }
  }
  if constexpr (EMIT) {
    // step scalars and retention of the chunk's tokens, for the replay
    if (!pinned && tid < C) {
      const int64_t gi = (tb + t0 + (tid < Lc ? tid : 0)) * H + h;
      sC[tid] = em.cstep[gi];
      if constexpr (!RVEC) sR[tid] = em.r ? em.r[gi] : 1.0f;
    }
  }
  if (ci + (int64_t)gridDim.x < nch) fetch(ci + gridDim.x);
  __syncthreads();
  if constexpr (EMIT) {
    // the replay of d through the chunk (EMIT, chunks not pinned): one thread
    // per coordinate, d_{t+1} = clip(r_t d_t + c_t k_t^2), writing E
    if (!pinned) {
      if (tid < KD) {
        const int c = tid;
        float d = em.dstart[ci * KD + c];
        const float lo = em.clamp ? em.d_min : -INFINITY, hi = em.clamp ? em.d_max : INFINITY;
        auto step = [&](int u, float ru) {
          const float kv = to_f32(sKl[u][c]);
          sKh[u][c] = to_bf16((d - 1.0f) * kv);  // d - 1 is exact on [0.5, 2]
          d = fminf(fmaxf(fmaf(sC[u], kv * kv, ru * d), lo), hi);
        };
        // with per-coordinate retention (diag(r_t)) thread c reads r_{t,c}
        // from the [B,T,H,K] rows, which share the key rows' layout
        const float *rc = em.r + base + c;
        if (Lc == C) {
          // straight-line: the reads, which do not depend on d, run ahead
          if constexpr (RVEC) {
            // sixteen rows of r in flight at a time keeps the register count
            // within three workgroups per CU
            for (int u0 = 0; u0 < C; u0 += 16) {
              float rr[16];
#pragma unroll
              for (int j = 0; j < 16; ++j) rr[j] = rc[(u0 + j) * tstride];
#pragma unroll
              for (int j = 0; j < 16; ++j) step(u0 + j, rr[j]);
            }
          } else {
#pragma unroll
            for (int u = 0; u < C; ++u) step(u, sR[u]);
          }
        } else {
          for (int u = 0; u < Lc; ++u) step(u, RVEC ? rc[u * tstride] : sR[u]);
          for (int u = Lc; u < C; ++u) sKh[u][c] = to_bf16(0.0f);
        }
      }
      __syncthreads();
    }
    // the residual rows, for the sweep kernel
    bf16 *res = em.res + base;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int vi = tid + 256 * p, i = vi >> 4, c8 = 8 * (vi & 15);
      if (i < Lc) *reinterpret_cast<bf16x8 *>(res + i * tstride + c8) = ld8(&sKh[i][c8]);
    }
  }

  // Gram tiles (rt, tj), tj <= rt, three or two per wave so that every wave
  // has a similar share and its product chains interleave:
  //   slot 0: (3,0) (3,2) (2,0) (2,2)   slot 1: (3,1) (3,3) (2,1) (1,1)
  //   slot 2: (0,0) (1,0)  -      -     (waves 0 .. 3)
  {
    const int rts[3] = {w < 2 ? 3 : 2, w < 2 ? 3 : (w == 2 ? 2 : 1), w};
    const int tjs[3] = {(w & 1) * 2, w == 1 ? 3 : 1, 0};
    floatx4 acc[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto gram = [&](auto NS) {
      constexpr int ns = decltype(NS)::value;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ko = 32 * kk + 8 * lq;
        bf16x8 ka[ns], bh[ns], bl[ns];
#pragma unroll
        for (int q = 0; q < ns; ++q) {
          ka[q] = ld8(&sKl[16 * rts[q] + l16][ko]);
          bh[q] = ld8(&sKh[16 * tjs[q] + l16][ko]);
          if constexpr (KRES) bl[q] = ld8(&sKl[16 * tjs[q] + l16][ko]);
        }
#pragma unroll
        for (int q = 0; q < ns; ++q) acc[q] = mfma32(ka[q], bh[q], acc[q]);
        if constexpr (KRES) {
#pragma unroll
          for (int q = 0; q < ns; ++q) acc[q] = mfma32(ka[q], bl[q], acc[q]);
        }
      }
    };
    if (w < 2)
      gram(IConst<3>{});
    else
      gram(IConst<2>{});
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (q < 2 || w < 2) {
        const int rt = rts[q], nn = 16 * tjs[q] + l16;
        const float gn = GATED ? sG[nn] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mrow = 16 * rt + 4 * lq + i;
          const float ratio = GATED ? __expf(sG[mrow] - gn) : 1.0f;
          sA[mrow][nn] = nn < mrow ? sBeta[mrow] * ratio * acc[q][i] : 0.0f;
        }
      }
    }
  }
  __syncthreads();
  // the key rows are dead: clear Tm (its upper triangle stays zero)
  for (int i = tid; i < C * CP / 8; i += 256) reinterpret_cast<bf16x8 *>(&sTr[0][0])[i] = bf16x8{};
  __syncthreads();

  // (i) wave w inverts diagonal block w by forward substitution in fp32;
  //     lane l & 15 computes column c of the block inverse.
  {
    const int c = l16, bb = 16 * w;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == c) ? 1.0f : 0.0f;
#pragma unroll
      for (int j = 0; j < i; ++j) s -= sA[bb + i][bb + j] * x[j];
      x[i] = s;
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
  // Tm rows to the workspace: 64 x 64 bf16, two 16-byte vectors per thread
  bf16 *dst = tout + ci * (C * C);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int v = tid + 256 * p, r = v >> 3, c8 = (v & 7) * 8;
    *reinterpret_cast<bf16x8 *>(dst + r * C + c8) = ld8(&sTr[r][c8]);
  }
  __syncthreads();  // the next chunk's rows overwrite Tm's buffers
  }
}

// ============================================================ sweep
// Transposed operand read (gfx950 ds_read_b64_tr_b16).  Within each group of
// 16 lanes, with D[i][p] the p-th bf16 at lane i's address, lane j receives
// D[4 e + j / 4][j % 4] as element e.  Lane i of the group pointing at row
// r0 + i / 4, column c0 + 4 (i % 4) of a row-major bf16 matrix X therefore
// receives X[r0 + e][c0 + j], e < 4: four consecutive rows of column c0 + j,
// which is the B operand layout of the matrix cores with k running over rows.
__device__ __forceinline__ bf16x4 ld4_tr(const bf16 *p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4 *)(const_cast<bf16 *>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// B operand of a 16x16x32 product with k over the rows [r0, r0 + 32) and n
// over the columns [c0, c0 + 16) of a row-major [.][P] bf16 matrix: lane l
// (group g = l / 16) needs rows r0 + 8 g + e, e < 8, of column c0 + l % 16.
// The A operand has the same lane layout, so the same read gives an A operand
// with m over the columns from a matrix stored k-major.
template <int P>
__device__ __forceinline__ bf16x8 ld8_tr(const bf16 (*X)[P], int r0, int c0, int l) {
  const int g = l >> 4, i = l & 15;
  const bf16x4 a = ld4_tr(&X[r0 + 8 * g + (i >> 2)][c0 + 4 * (i & 3)]);
  const bf16x4 b = ld4_tr(&X[r0 + 8 * g + 4 + (i >> 2)][c0 + 4 * (i & 3)]);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// 64-wide bf16 rows without padding: the 16-byte chunk c of row r sits at
// chunk c ^ (r & 7), which keeps 16-row operand reads, transposed reads and
// 8-byte epilogue stores free of bank conflicts.  Element offset of (r, c):
__device__ __forceinline__ int sx(int r, int c) { return r * 64 + ((((c >> 3) ^ r) & 7) << 3) + (c & 7); }

// 128-wide bf16 rows without padding: chunk c of row r at chunk c ^ (r & 15)
__device__ __forceinline__ int sx128(int r, int c) { return r * 128 + ((((c >> 3) ^ r) & 15) << 3) + (c & 7); }

// ld8_tr over an sx-layout matrix (each 8-byte read stays inside one chunk)
__device__ __forceinline__ bf16x8 ld8_tr_sx(const bf16 *X, int r0, int c0, int l) {
  const int g = l >> 4, i = l & 15, c = c0 + 4 * (i & 3);
  const bf16x4 a = ld4_tr(X + sx(r0 + 8 * g + (i >> 2), c));
  const bf16x4 b = ld4_tr(X + sx(r0 + 8 * g + 4 + (i >> 2), c));
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

struct SeqLay {
  static constexpr int Q = 0;                        // bf16 [C][KP]  queries
  static constexpr int K = Q + C * KP * 2;           // bf16 [C][KP]  keys
  static constexpr int E = K + C * KP * 2;           // bf16 [C][KP]  write keys, or residual E
  static constexpr int V = E + C * KP * 2;           // bf16 [C][VT+8] value tile
  static constexpr int BETA = V + C * (VT + 8) * 2;  // f32 [C]
  static constexpr int G = BETA + C * 4;             // f32 [C] cumulative log decay
  // 64-wide rows below are unpadded, 16-byte chunks swizzled (sx)
  static constexpr int MH = G + C * 4;               // bf16 [C][C]   scores^T hi
  static constexpr int ML = MH + C * C * 2;          // bf16 [C][C]   scores^T lo
  static constexpr int RTH = ML + C * C * 2;         // bf16 [VT][C]  R^T hi
  static constexpr int RTL = RTH + VT * C * 2;       // bf16 [VT][C]  R^T lo
  static constexpr int DTH = RTL + VT * C * 2;       // bf16 [VT][C]  Delta^T hi
  static constexpr int DTL = DTH + VT * C * 2;       // bf16 [VT][C]  Delta^T lo
  static constexpr int DSH = DTL + VT * C * 2;       // bf16 [VT][C]  decayed Delta^T hi
  static constexpr int DSL = DSH + VT * C * 2;       // bf16 [VT][C]  decayed Delta^T lo
  static constexpr int SH = DSL + VT * C * 2;        // bf16 [VT][KD] state hi (sx128 layout)
  static constexpr int SL = SH + VT * KD * 2;        // bf16 [VT][KD] state lo
  static constexpr int TOTAL = SL + VT * KD * 2;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// With the residual form (KRES) the write key is k~ = k + E with k and E both
// exact bf16, so every product with k~ is the sum of a product with k and one
// with E; otherwise the E buffer holds the bf16 k~ itself.
template <bool GATED, bool KRES, bool VL>
__global__ __launch_bounds__(512) void chunk_seq_kernel(ChunkArgs a, const bf16 *tin, int64_t N) {
  typedef SeqLay L;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  bf16(*sQ)[KP] = reinterpret_cast<bf16(*)[KP]>(smem + L::Q);
  bf16(*sK)[KP] = reinterpret_cast<bf16(*)[KP]>(smem + L::K);
  bf16(*sE)[KP] = reinterpret_cast<bf16(*)[KP]>(smem + L::E);
  bf16(*sV)[VT + 8] = reinterpret_cast<bf16(*)[VT + 8]>(smem + L::V);
  float *sBeta = reinterpret_cast<float *>(smem + L::BETA);
  float *sG = reinterpret_cast<float *>(smem + L::G);
  bf16 *sMh = reinterpret_cast<bf16 *>(smem + L::MH);  // [n][m], sx layout
  bf16 *sMl = reinterpret_cast<bf16 *>(smem + L::ML);
  bf16 *sRh = reinterpret_cast<bf16 *>(smem + L::RTH);  // [v][t], sx layout
  bf16 *sRl = reinterpret_cast<bf16 *>(smem + L::RTL);
  bf16 *sDh = reinterpret_cast<bf16 *>(smem + L::DTH);
  bf16 *sDl = reinterpret_cast<bf16 *>(smem + L::DTL);
  bf16 *sDsh = reinterpret_cast<bf16 *>(smem + (GATED ? L::DSH : L::DTH));
  bf16 *sDsl = reinterpret_cast<bf16 *>(smem + (GATED ? L::DSL : L::DTL));
  bf16 *sSh = reinterpret_cast<bf16 *>(smem + L::SH);  // [v][k], sx128 layout
  bf16 *sSl = reinterpret_cast<bf16 *>(smem + L::SL);

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = l & 15, lq = l >> 4;
  const int rw = w & 3, cw = w >> 2;  // token rows [16 rw, +16), value columns [16 cw, +16)
  const int m0 = 16 * rw;
  // XCD-aware placement: block i runs on XCD i % 8; the NT tiles of one
  // sequence share i % 8, so their reads of the same keys meet in one L2.
  const int bid = blockIdx.x;
  const int slot = bid & 7, rest = bid >> 3;
  const int vt = rest % NT;
  const int64_t seq = (int64_t)(rest / NT) * 8 + slot;
  const int64_t H = a.H;
  if (seq >= a.B * H) return;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t Nb = (T + C - 1) / C;  // this sequence's chunks (N is the workspace row stride)
  const int v0 = vt * VT;

  const bf16 *gq = static_cast<const bf16 *>(a.q);
  const bf16 *gk = static_cast<const bf16 *>(a.k);
  const bf16 *gkt = static_cast<const bf16 *>(a.kt);
  const bf16 *gv = static_cast<const bf16 *>(a.v);
  bf16 *go = static_cast<bf16 *>(a.o);
  const int64_t tstride = H * KD;                   // elements between tokens (K == V == 128)
  const int64_t base = tb * tstride + h * KD;  // token 0 of this (b,h)
  const bf16 *tseq = tin + seq * N * (C * C);

  // scores: the tiles above the diagonal are never written and stay zero
  for (int i = tid; i < C * C / 8; i += 512) {
    reinterpret_cast<bf16x8 *>(sMh)[i] = bf16x8{};
    reinterpret_cast<bf16x8 *>(sMl)[i] = bf16x8{};
  }
  // Roles: waves 4-7 ("row waves") own token rows [16 rw, 16 rw + 16) of the
  // chunk for K S^T, Q S^T, R and O, over both 16-column value tiles; waves
  // 0-3 compute the score tiles, then own the state columns
  // [32 sp, 32 sp + 32) (sp = w) in accumulators, as tiles of S^T: element i
  // of tile (rt, j) is S[16 rt + l16][16 (2 sp + j) + 4 lq + i].  Wave w
  // shares a SIMD with wave w + 4; this way round measured faster than the
  // reverse.
  const bool roww = w >= 4;
  const int sp = w & 3;
  floatx4 Sacc[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int vr = 16 * rt + l16, c = 16 * (2 * sp + j) + 4 * lq;
      Sacc[rt][j] = a.S0 ? *reinterpret_cast<const floatx4 *>(a.S0 + (seq * VD + v0 + vr) * KD + c)
                         : floatx4{0.f, 0.f, 0.f, 0.f};
      if (!roww) {
        bf16x4 sh4, sl4;
        split4(Sacc[rt][j], sh4, sl4);
        *reinterpret_cast<bf16x4 *>(sSh + sx128(vr, c)) = sh4;
        *reinterpret_cast<bf16x4 *>(sSl + sx128(vr, c)) = sl4;
      }
    }

  // ---- prefetch registers for one chunk (each input element is loaded once
  //      per workgroup, in 16-byte vectors, 16 threads per token row)
  //   q, k, E rows:  vectors tid and tid + 512 of each 64 x 128 tile
  //   values:        threads < 256: token tid / 4, columns 8 (tid % 4) of the tile
  //   Tm:            rows 16 rw + l16 in MFMA A-operand layout
  // Tokens past T (last chunk only) read the chunk's first token instead and are never
  // selected here: a select would wait for the load.  Their beta is zeroed
  // at use, which makes their R and Delta rows zero; their scores fall
  // outside the causal mask and their outputs are not stored.
  // Addresses: a chunk's base pointers are wave-uniform (scalar registers);
  // each lane adds a 32-bit byte offset fixed for the whole sweep (phase 2
  // takes H <= 65536, so 64 token rows span at most 1 GiB).
  const int64_t rowb = tstride * 2;  // bytes between tokens
  const char *qb = reinterpret_cast<const char *>(gq + base);
  const char *kb = reinterpret_cast<const char *>(gk + base);
  const char *eb = reinterpret_cast<const char *>(gkt + base);
  const char *vb = reinterpret_cast<const char *>(gv + base + v0);
  char *ob = reinterpret_cast<char *>(go + base + v0);
  const char *bb = reinterpret_cast<const char *>(a.beta + tb * H + h);
  const char *ab = GATED ? reinterpret_cast<const char *>(a.alpha + tb * H + h) : nullptr;
  uint32_t roff[2], coff[2];
  int rrow[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int vi = tid + 512 * p;
    rrow[p] = vi >> 4;
    coff[p] = (uint32_t)(16 * (vi & 15));
    roff[p] = (uint32_t)(rrow[p] * rowb) + coff[p];
  }
  const int vrow = tid >> 2;
  const uint32_t vcoff = (uint32_t)(16 * (tid & 3)), voff = (uint32_t)(vrow * rowb) + vcoff;
  const uint32_t toff = (uint32_t)(((16 * rw + l16) * C + 8 * lq) * 2);
  const uint32_t boff = (uint32_t)(l * H * 4);
  const uint32_t ooff = (uint32_t)((m0 + 4 * lq) * rowb + 2 * l16);  // row waves, value tile 0

  bf16x8 pq[2], pk[2], pe[2], pv, pt[2];
  float pbeta = 0.0f, palpha = 1.0f;
  // parts: FQ = q, values, beta (and alpha); FK = k; FE = E
  constexpr int FQ = 1, FK = 2, FE = 4;
  auto fetch = [&](int64_t n, int parts) {
    const int64_t t0 = n * C;
    const int Lc = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t cb = t0 * rowb;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t o = rrow[p] < Lc ? roff[p] : coff[p];
      if (parts & FQ) pq[p] = ld8(reinterpret_cast<const bf16 *>(qb + cb + o));
      if (parts & FK) pk[p] = ld8(reinterpret_cast<const bf16 *>(kb + cb + o));
      if (parts & FE) pe[p] = ld8(reinterpret_cast<const bf16 *>(eb + cb + o));
    }
    if (!(parts & FQ)) return;
    if (tid < 256) pv = ld8(reinterpret_cast<const bf16 *>(vb + cb + (vrow < Lc ? voff : vcoff)));
    if (w == 0) {
      const int64_t sb = t0 * H * 4;
      const uint32_t o = l < Lc ? boff : 0u;
      pbeta = *reinterpret_cast<const float *>(bb + sb + o);
      if constexpr (GATED) palpha = *reinterpret_cast<const float *>(ab + sb + o);
    }
  };
  // Tm rows go straight into the registers stage D reads.  They are loaded
  // once stage D of the previous chunk is done with them, which leaves a
  // whole chunk for the load to land and needs no register copy (a copy into
  // registers with a load in flight would wait for every outstanding load).
  auto fetch_t = [&](int64_t n) {
    const char *tp = reinterpret_cast<const char *>(tseq + n * (C * C)) + toff;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) pt[kk] = ld8(reinterpret_cast<const bf16 *>(tp + 64 * kk));
  };

  if (Nb > 0) {
    fetch(0, FQ | FK | FE);
    fetch_t(0);
  }
  for (int64_t n = 0; n < Nb; ++n) {
    const int64_t t0 = n * C;
    const int Lc = (int)((T - t0) < C ? (T - t0) : C);
    __syncthreads();  // the previous chunk is done with every LDS buffer
    // ---- stage L: registers -> LDS
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int vi = tid + 512 * p, i = vi >> 4, c8 = 8 * (vi & 15);
      *reinterpret_cast<bf16x8 *>(&sQ[i][c8]) = pq[p];
      *reinterpret_cast<bf16x8 *>(&sK[i][c8]) = pk[p];
      *reinterpret_cast<bf16x8 *>(&sE[i][c8]) = pe[p];
    }
    if (tid < 256) *reinterpret_cast<bf16x8 *>(&sV[tid >> 2][8 * (tid & 3)]) = pv;
    if (w == 0) {
      const bool ok = l < Lc;
      sBeta[l] = ok ? pbeta : 0.0f;
      if constexpr (GATED) {
        float x = ok ? logf(palpha) : 0.0f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off, 64);
          if (l >= off) x += y;
        }
        sG[l] = x;
      }
    }
    __syncthreads();
    // The next chunk's rows are loaded in three parts, one per phase between
    // barriers, so that their issue overlaps with compute instead of stalling
    // one phase.  Issued on every chunk (the last one reloads its own rows,
    // valid and unused) so that the number of loads in flight does not depend
    // on the path, which lets the waits for Tm count past these loads instead
    // of draining them.
    const int64_t nn1 = n + 1 < Nb ? n + 1 : n;
    fetch(nn1, FQ);

    // ---- stage G.  Row waves: K S^T and Q S^T for their rows, both value
    //      tiles, then R (to LDS, transposed) and the Q S^T part of O (kept).
    //      Other waves: the ten score tiles on and below the diagonal, split
    //      3 / 3 / 2 / 2, each wave loading a query row block once.
    floatx4 Oacc[2];
    if (roww) {
      floatx4 accKS[2], accQS[2];
      bf16x8 kf[4], qf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ko = 32 * kk + 8 * lq;
        kf[kk] = ld8(&sK[m0 + l16][ko]);
        qf[kk] = ld8(&sQ[m0 + l16][ko]);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        bf16x8 sh[4], sl[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          sh[kk] = ld8(sSh + sx128(16 * ct + l16, 32 * kk + 8 * lq));
          sl[kk] = ld8(sSl + sx128(16 * ct + l16, 32 * kk + 8 * lq));
        }
        floatx4 ks = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          ks = mfma32(kf[kk], sh[kk], ks);
          qs = mfma32(qf[kk], sh[kk], qs);
          ks = mfma32(kf[kk], sl[kk], ks);
          qs = mfma32(qf[kk], sl[kk], qs);
        }
        accKS[ct] = ks;
        accQS[ct] = qs;
      }
      float gm[4], bm[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gm[i] = GATED ? sG[m0 + 4 * lq + i] : 0.0f;
        bm[i] = sBeta[m0 + 4 * lq + i];
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        // values V[m0 + 4 lq + i][16 ct + l16], i < 4, in one transposed read
        const bf16x4 vv = ld4_tr(&sV[m0 + 4 * lq + (l16 >> 2)][16 * ct + 4 * (l16 & 3)]);
        floatx4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float em = GATED ? __expf(gm[i]) : 1.0f;
          r[i] = bm[i] * (to_f32(vv[i]) - em * accKS[ct][i]);
          Oacc[ct][i] = em * accQS[ct][i];
        }
        bf16x4 rh, rl;
        split4(r, rh, rl);
        *reinterpret_cast<bf16x4 *>(sRh + sx(16 * ct + l16, m0 + 4 * lq)) = rh;
        *reinterpret_cast<bf16x4 *>(sRl + sx(16 * ct + l16, m0 + 4 * lq)) = rl;
      }
    } else {
      // score tiles (mr, tj), tj = tj0 .. tj0 + CNT - 1 <= mr, one query
      // block; every operand is loaded before the products, whose chains
      // interleave
      auto mrow = [&](int mr, int tj0, auto cnt) {
        constexpr int CNT = decltype(cnt)::value;
        bf16x8 qf[4], me[CNT][4], mk[CNT][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int ko = 32 * kk + 8 * lq;
          qf[kk] = ld8(&sQ[16 * mr + l16][ko]);
#pragma unroll
          for (int t = 0; t < CNT; ++t) {
            me[t][kk] = ld8(&sE[16 * (tj0 + t) + l16][ko]);
            if constexpr (KRES) mk[t][kk] = ld8(&sK[16 * (tj0 + t) + l16][ko]);
          }
        }
        floatx4 acc[CNT];
#pragma unroll
        for (int t = 0; t < CNT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int t = 0; t < CNT; ++t) {
            acc[t] = mfma32(qf[kk], me[t][kk], acc[t]);
            if constexpr (KRES) acc[t] = mfma32(qf[kk], mk[t][kk], acc[t]);
          }
        float gr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) gr[i] = GATED ? sG[16 * mr + 4 * lq + i] : 0.0f;
#pragma unroll
        for (int t = 0; t < CNT; ++t) {
          const int nn = 16 * (tj0 + t) + l16;
          const float gn = GATED ? sG[nn] : 0.0f;
          floatx4 mv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * mr + 4 * lq + i;
            const float ratio = GATED ? __expf(gr[i] - gn) : 1.0f;
            mv[i] = nn <= m ? ratio * acc[t][i] : 0.0f;
          }
          bf16x4 mh, ml;
          split4(mv, mh, ml);
          *reinterpret_cast<bf16x4 *>(sMh + sx(nn, 16 * mr + 4 * lq)) = mh;
          *reinterpret_cast<bf16x4 *>(sMl + sx(nn, 16 * mr + 4 * lq)) = ml;
        }
      };
      if (w == 0) {
        mrow(1, 0, IConst<2>{});
        mrow(0, 0, IConst<1>{});
      } else if (w == 1) {
        // two calls keep the operands of at most two tiles live
        mrow(3, 1, IConst<2>{});
        mrow(3, 3, IConst<1>{});
      } else if (w == 2) {
        mrow(2, 0, IConst<2>{});
      } else {
        mrow(2, 2, IConst<1>{});
        mrow(3, 0, IConst<1>{});
      }
    }
    __syncthreads();
    fetch(nn1, FK | FE);

    // ---- stage D: Delta tile (rw, cw) = Tm R, split and stored transposed.
    const float gL = GATED ? sG[Lc - 1] : 0.0f;
    {
      // Tm is lower triangular: rows below 32 need only the first k-step
      const int nks = rw < 2 ? 1 : 2;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk < nks) {
          const bf16x8 rh = ld8(sRh + sx(16 * cw + l16, 32 * kk + 8 * lq));
          const bf16x8 rl = ld8(sRl + sx(16 * cw + l16, 32 * kk + 8 * lq));
          acc = mfma32(pt[kk], rh, acc);
          acc = mfma32(pt[kk], rl, acc);
        }
      }
      bf16x4 dh, dl;
      split4(acc, dh, dl);
      *reinterpret_cast<bf16x4 *>(sDh + sx(16 * cw + l16, m0 + 4 * lq)) = dh;
      *reinterpret_cast<bf16x4 *>(sDl + sx(16 * cw + l16, m0 + 4 * lq)) = dl;
      if constexpr (GATED) {
        floatx4 s;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = acc[i] * __expf(gL - sG[m0 + 4 * lq + i]);
        split4(s, dh, dl);
        *reinterpret_cast<bf16x4 *>(sDsh + sx(16 * cw + l16, m0 + 4 * lq)) = dh;
        *reinterpret_cast<bf16x4 *>(sDsl + sx(16 * cw + l16, m0 + 4 * lq)) = dl;
      }
    }
    __syncthreads();
    fetch_t(nn1);

    if (roww) {
      // ---- stage O: output rows of this wave, both value tiles.  The scores
      //      of rows below 32 vanish past the first k-step.
      const int nks = rw < 2 ? 1 : 2;
      bf16x8 mh[2], ml[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk < nks) {
          mh[kk] = ld8_tr_sx(sMh, 32 * kk, m0, l);
          ml[kk] = ld8_tr_sx(sMl, 32 * kk, m0, l);
        }
      }
      bf16x8 dh[2][2], dl[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          if (kk < nks) {
            const int ko = 32 * kk + 8 * lq;
            dh[ct][kk] = ld8(sDh + sx(16 * ct + l16, ko));
            dl[ct][kk] = ld8(sDl + sx(16 * ct + l16, ko));
          }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          if (kk < nks) {
            Oacc[ct] = mfma32(mh[kk], dh[ct][kk], Oacc[ct]);
            Oacc[ct] = mfma32(mh[kk], dl[ct][kk], Oacc[ct]);
            Oacc[ct] = mfma32(ml[kk], dh[ct][kk], Oacc[ct]);
          }
      char *oc = ob + t0 * rowb + ooff;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (m0 + 4 * lq + i < Lc)
            *reinterpret_cast<bf16 *>(oc + i * rowb + 32 * ct) = to_bf16(a.q_scale * Oacc[ct][i]);
    } else {
      // ---- stage S: the wave's four tiles of S^T += K~^T Delta, then their
      //      bf16 pairs.  The write keys enter as A operands with k over
      //      tokens, read transposed from the row-major key buffers.
      const float decay = GATED ? __expf(gL) : 1.0f;
      bf16x8 dsh[2][2], dsl[2][2], be[2][2], bk[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ko = 32 * kk + 8 * lq;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          dsh[rt][kk] = ld8(sDsh + sx(16 * rt + l16, ko));
          dsl[rt][kk] = ld8(sDsl + sx(16 * rt + l16, ko));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int c0 = 16 * (2 * sp + j);
          be[j][kk] = ld8_tr(sE, 32 * kk, c0, l);
          if constexpr (KRES) bk[j][kk] = ld8_tr(sK, 32 * kk, c0, l);
        }
      }
      if constexpr (GATED) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int j = 0; j < 2; ++j) Sacc[rt][j] = Sacc[rt][j] * decay;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            Sacc[rt][j] = mfma32(be[j][kk], dsh[rt][kk], Sacc[rt][j]);
            Sacc[rt][j] = mfma32(be[j][kk], dsl[rt][kk], Sacc[rt][j]);
            if constexpr (KRES) {
              Sacc[rt][j] = mfma32(bk[j][kk], dsh[rt][kk], Sacc[rt][j]);
              Sacc[rt][j] = mfma32(bk[j][kk], dsl[rt][kk], Sacc[rt][j]);
            }
          }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bf16x4 sh4, sl4;
          split4(Sacc[rt][j], sh4, sl4);
          const int kt = 2 * sp + j;
          *reinterpret_cast<bf16x4 *>(sSh + sx128(16 * rt + l16, 16 * kt + 4 * lq)) = sh4;
          *reinterpret_cast<bf16x4 *>(sSl + sx128(16 * rt + l16, 16 * kt + 4 * lq)) = sl4;
        }
    }
  }

  if (a.S_out && !roww) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int vr = 16 * rt + l16, c = 16 * (2 * sp + j) + 4 * lq;
        *reinterpret_cast<floatx4 *>(a.S_out + (seq * VD + v0 + vr) * KD + c) = Sacc[rt][j];
      }
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <bool GATED, bool KRES, bool VL>
void launch_both(const ChunkArgs &a, bf16 *tw, int64_t N, hipStream_t s, const EmitArgs *em) {
  const int64_t nseq = a.B * a.H;
  if (N > 0) {
    // persistent UT transform: as many workgroups as fit on the device at
    // once, each taking an equal number of chunks
    const int64_t nch = nseq * N;
    const int64_t slots = (int64_t)device_cus() * ((160 * 1024) / TinvLay::TOTAL);
    const int64_t per = (nch + slots - 1) / slots;
    const dim3 grid((unsigned)((nch + per - 1) / per)), block(256);
    if constexpr (KRES) {
      if (em) {
        // per-coordinate retention has an instantiation of its own, so that
        // the scalar one keeps its register count (three workgroups per CU)
        if (em->r_vec)
          hipLaunchKernelGGL((chunk_tinv_kernel<GATED, true, true, VL, true>), grid, block, 0, s, a, tw, N, *em);
        else
          hipLaunchKernelGGL((chunk_tinv_kernel<GATED, true, true, VL>), grid, block, 0, s, a, tw, N, *em);
        prof_mark(s, "chunk_tinv_kernel");
      }
    }
    if (!em) {
      hipLaunchKernelGGL((chunk_tinv_kernel<GATED, KRES, false, VL>), grid, block, 0, s, a, tw, N, EmitArgs{});
      prof_mark(s, "chunk_tinv_kernel");
    }
  }
  const int64_t groups = (nseq + 7) / 8;
  hipLaunchKernelGGL((chunk_seq_kernel<GATED, KRES, VL>), dim3((unsigned)(groups * 8 * NT)), dim3(512), 0, s, a,
                     (const bf16 *)tw, N);
  prof_mark(s, "chunk_seq_kernel");
}

template <bool VL>
void launch_gated(const ChunkArgs &a, bf16 *tw, int64_t N, hipStream_t s, const EmitArgs *em) {
  if (a.alpha) {
    if (a.kt_is_res)
      launch_both<true, true, VL>(a, tw, N, s, em);
    else
      launch_both<true, false, VL>(a, tw, N, s, nullptr);
  } else {
    if (a.kt_is_res)
      launch_both<false, true, VL>(a, tw, N, s, em);
    else
      launch_both<false, false, VL>(a, tw, N, s, nullptr);
  }
}

}  // namespace

size_t chunk_wy_work_bytes(int64_t B, int64_t T, int64_t H) {
  const int64_t N = (T + C - 1) / C;
  return (size_t)(B * H * N) * C * C * 2;
}

hipError_t launch_chunk_wy(const ChunkArgs &a, void *work, hipStream_t s, const EmitArgs *em) {
  if (a.B * a.H == 0) return hipSuccess;
  if (em && (!a.kt_is_res || C != SCAN_CHUNK)) return hipErrorInvalidValue;
  const int64_t N = (a.T + C - 1) / C;
  bf16 *tw = static_cast<bf16 *>(work);
  if (a.cu)
    launch_gated<true>(a, tw, N, s, em);
  else
    launch_gated<false>(a, tw, N, s, em);
  return hipGetLastError();
}

}  // namespace osdn
