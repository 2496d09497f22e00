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
//  chunk_tinv_kernel (chunk-parallel, persistent workgroups):
//    A  = strict_lower(B [e^{g_i-g_j}] . K K~^T)
//    Tm = (I + A)^-1 and the scores M = lower([e^{g_i-g_j}] . Q K~^T), written
//         to the workspace in bf16 (M as hi/lo pairs) in the sweep's operand order
//
//  chunk_sweep_kernel (one workgroup per (b,h) and 32 value rows, chunks in
//  order; S is the boundary state, V x K, fp32):
//    R     = B (V - diag(e^g) K S^T)
//    Delta = Tm R                                     (= U - W S^T of Eq.(11))
//    O     = q_scale (diag(e^g) Q S^T + M Delta)
//    S    <- e^{g_L} S + Delta^T (e^{g_L - g} . K~)
//
// Tm and M depend only on the chunk's keys and queries, so the sweep carries
// no triangular solve.  It runs eight waves: two run the state-dependent
// chain (K S^T, R, Tm R, the state update), two form the outputs, four bring
// the next chunk's rows into the other LDS buffer; two barriers per chunk.
// The key rows serve both as row operands and, through transposed LDS reads,
// as the token-major operand of the state update.
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
constexpr int TKP = KD + 8; // the same in the UT transform, whose workgroups must fit three to a CU
constexpr int CP = C + 8;  // LDS pitch (bf16) of 64-wide rows
constexpr int AP = C + 4;  // LDS pitch (f32) of the Gram

// The (I + A)^-1 operands of a chunk as the sweep reads them: block j of
// (mt, s) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1) (the blocks
// below and on the diagonal), lane l = (l16, g) holding row 16 mt + l16 at
// columns 32 s + 4 g + {0..3} and 32 s + 16 + 4 g + {0..3} (tile order).
constexpr int TDUMP = 6 * 64 * 8;  // bf16 elements per chunk
// The intra-chunk scores lower([e^{g_i - g_j}] . Q K~^T) as the sweep's
// output products read them: blocks j as above, each as hi then lo bf16
// (block 2 j + 0 / 2 j + 1), lane (l16, g) holding score row 16 mt + l16 at
// key positions 32 s + 4 g + {0..3} and 32 s + 16 + 4 g + {0..3}.
constexpr int MDUMP = 12 * 64 * 8;
// Then the chunk's scalars as fp32: beta (zero past the chunk end) and, in the
// gated form, the decay factors e^{g_t} and e^{g_L - g_t} (g the cumulative
// log decay, constant past the chunk end), so that the sweep reads them as
// 256-byte pieces rather than 64 strided words, and evaluates no exponential.
constexpr int SDUMP = 3 * 64 * 2;  // in bf16 elements
constexpr int CHUNKW = TDUMP + MDUMP + SDUMP;  // workspace per chunk

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// hi / lo bf16 pairs of two result tiles, packed as tile-order operands
__device__ __forceinline__ void split8(floatx4 a, floatx4 b, bf16x8 &hi, bf16x8 &lo) {
  bf16x4 ah, al, bh, bl;
  split4(a, ah, al);
  split4(b, bh, bl);
  hi = cat8(ah, bh);
  lo = cat8(al, bl);
}

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
// The chunk's intra scores are formed here as well (state-independent), so
// that the sweep only multiplies them: wave w forms the scores of token rows
// [16 w, 16 w + 16) against every earlier key of the chunk.
// A chunk the chunked phase 1 marked as pinned on d_min (a.pin, residual form)
// has write keys d_min k: its Gram and scores are d_min times those of k.
template <bool GATED, bool KRES, bool EMIT, bool VL, bool RVEC = false>
__global__ __launch_bounds__(256, 3) void chunk_tinv_kernel(ChunkArgs a, bf16 *tout, int64_t N, EmitArgs em) {
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
  const bf16 *gq = static_cast<const bf16 *>(a.q);
  const int64_t tstride = H * KD;
  const int64_t nch = a.B * H * N;
  const int *pins = KRES ? a.pin : nullptr;
  // Each workgroup takes chunks blockIdx.x, blockIdx.x + gridDim.x, ...; the
  // next chunk's key rows (and write-key rows off the folded path), beta,
  // alpha and pin word are loaded into registers while this one is computed.
  bf16x8 px[4], pe[4], pq[4];
  float pb = 0.0f, pa = 1.0f;
  int ppin = 0;
  // EMIT: the next chunk's start d (thread = coordinate), step scalars and
  // retention (thread = token).  No vector load is issued after the
  // prefetch in a chunk, so no wait of the chunk's own work waits for it.
  float pd = 1.0f, pc = 0.0f, pr = 1.0f;
  // The loads go out in two parts (a wave's loads queue behind each other):
  // part 0 at the start of a chunk, part 1 after its scores.
  auto fetch = [&](int64_t ci, auto PART) {
    constexpr int part = decltype(PART)::value;
    const int64_t seq = ci / N, n = ci - seq * N;
    const int64_t b = seq / H, h = seq - b * H;
    const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
    const int64_t t0 = n * C;
    if (VL && t0 >= T) return;  // past a shorter sequence's end: skipped below
    const int Lc = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t base = (tb + t0) * tstride + h * KD;
    if constexpr (part == 1) {
      // queries of this wave's score rows, as B operands (lane (n, g): row
      // 16 w + n, columns 32 kk + 8 g ..)
      const int i = 16 * w + l16;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pq[kk] = ld8(gq + base + (i < Lc ? i : 0) * tstride + 32 * kk + 8 * lq);
      if (w == 0) {
        const int64_t gi = (tb + t0 + (l < Lc ? l : 0)) * H + h;
        pb = a.beta[gi];
        if constexpr (GATED) pa = a.alpha[gi];
      }
      return;
    }
    if constexpr (EMIT && !GATED) {
      // the replay's inputs first (read for pinned chunks too, which do not
      // use them: every index is in range; the gated form, short of
      // registers, reads them with the chunk)
      if (tid < KD) pd = em.dstart[ci * KD + tid];
      if (tid < C) {
        const int64_t gi = (tb + t0 + (tid < Lc ? tid : 0)) * H + h;
        pc = em.cstep[gi];
        if constexpr (!RVEC) pr = em.r ? em.r[gi] : 1.0f;
      }
    }
    // (made wave-uniform where it is used, so that it is not waited for here
    // on the folded path)
    ppin = pins ? pins[ci] : 0;
    const bool need_e = !EMIT && __builtin_amdgcn_readfirstlane(ppin) != 2;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int vi = tid + 256 * p, i = vi >> 4, c8 = 8 * (vi & 15);
      const int64_t off = base + (i < Lc ? i : 0) * tstride + c8;
      px[p] = ld8(gk + off);
      if (need_e) pe[p] = ld8(gkt + off);
    }
  };
  if ((int64_t)blockIdx.x < nch) {
    fetch(blockIdx.x, IConst<0>{});
    fetch(blockIdx.x, IConst<1>{});
  }
  for (int64_t ci = blockIdx.x; ci < nch; ci += gridDim.x) {
  const int64_t seq = ci / N, n = ci - seq * N;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t t0 = n * C;
  if (VL && t0 >= T) {
    // past a shorter sequence's end (the whole workgroup alike): nothing to
    // form; the next chunk's loads still go out
    if (ci + (int64_t)gridDim.x < nch) {
      fetch(ci + gridDim.x, IConst<0>{});
      fetch(ci + gridDim.x, IConst<1>{});
    }
    continue;
  }
  const int Lc = (int)((T - t0) < C ? (T - t0) : C);
  const int64_t base = (tb + t0) * tstride + h * KD;  // token t0 of this (b,h)

  // ---- this chunk's rows into LDS (16-byte vectors, 16 threads per row;
  //      zero past T), beta and the cumulative log decay
  // A chunk the phase-1 sweep took as pinned (marked 2) starts from d_min,
  // and its mark guarantees that every step clips back to d_min (the mark
  // tests the replay's own fp32 expression at the largest key square), so its
  // write keys are d_min k: no replay, no residual.
  const bool pinned = __builtin_amdgcn_readfirstlane(ppin) == 2;
  const float kscale = pinned ? a.d_min : 1.0f;  // write keys d_min k
  const bf16x8 qop[4] = {pq[0], pq[1], pq[2], pq[3]};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int vi = tid + 256 * p, i = vi >> 4, c8 = 8 * (vi & 15);
    *reinterpret_cast<bf16x8 *>(&sKl[i][c8]) = i < Lc ? px[p] : bf16x8{};
    // write keys (with the residual form k~ = k + E both k and E are exact
    // bf16 operands, so the Gram is K E^T + K K^T; otherwise the bf16 k~
    // rows themselves)
    if (!EMIT && !pinned) *reinterpret_cast<bf16x8 *>(&sKh[i][c8]) = i < Lc ? pe[p] : bf16x8{};
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
  float d0 = pd;  // this chunk's start d of coordinate tid (EMIT)
  if constexpr (EMIT) {
    // step scalars and retention of the chunk's tokens, for the replay
    if (!pinned && tid < C) {
      if constexpr (GATED) {
        const int64_t gi = (tb + t0 + (tid < Lc ? tid : 0)) * H + h;
        sC[tid] = em.cstep[gi];
        if constexpr (!RVEC) sR[tid] = em.r ? em.r[gi] : 1.0f;
      } else {
        sC[tid] = pc;
        if constexpr (!RVEC) sR[tid] = pr;
      }
    }
  }
  if (ci + (int64_t)gridDim.x < nch) fetch(ci + gridDim.x, IConst<0>{});
  __syncthreads();
  if constexpr (EMIT) {
    // the replay of d through the chunk (EMIT, chunks not pinned): one thread
    // per coordinate, d_{t+1} = clip(r_t d_t + c_t k_t^2), writing E
    if (!pinned) {
      if (tid < KD) {
        const int c = tid;
        float d = GATED ? em.dstart[ci * KD + c] : d0;
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
    // the residual rows, for the sweep kernel (which takes a pinned chunk's
    // write keys as d_min k and does not read them)
    if (!pinned) {
      bf16 *res = em.res + base;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int vi = tid + 256 * p, i = vi >> 4, c8 = 8 * (vi & 15);
        if (i < Lc) *reinterpret_cast<bf16x8 *>(res + i * tstride + c8) = ld8(&sKh[i][c8]);
      }
    }
  }

  // scores of token rows [16 w, 16 w + 16): tiles (jt, w) of M^T = K~ Q^T,
  // jt <= w (lane (n, g) of tile jt holds M[16 w + n][16 jt + 4 g + i], the
  // sweep's A operand in tile order), masked to the causal part, with the
  // decay ratios, as hi/lo bf16 pairs.  Without decay every wave forms all
  // four tiles (the ones above the diagonal are masked): no branch between
  // the operand reads and the products, so the reads of a slab go out
  // together.
  {
    floatx4 acc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) acc[jt] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto prod = [&](auto UK, auto UE) __attribute__((always_inline)) {
      constexpr bool uk = decltype(UK)::value, ue = decltype(UE)::value;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ko = 32 * kk + 8 * lq;
        bf16x8 ak[4], ae[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          if (uk) ak[jt] = ld8(&sKl[16 * jt + l16][ko]);
          if (ue) ae[jt] = ld8(&sKh[16 * jt + l16][ko]);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          if (uk) acc[jt] = mfma32(ak[jt], qop[kk], acc[jt]);
          if (ue) acc[jt] = mfma32(ae[jt], qop[kk], acc[jt]);
        }
      }
    };
    if constexpr (GATED) {
      // (the gated form keeps the causal tiles only: its decay ratios need
      // the registers)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ko = 32 * kk + 8 * lq;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          if (jt <= w) {
            if (KRES || pinned) acc[jt] = mfma32(ld8(&sKl[16 * jt + l16][ko]), qop[kk], acc[jt]);
            if (!pinned) acc[jt] = mfma32(ld8(&sKh[16 * jt + l16][ko]), qop[kk], acc[jt]);
          }
        }
      }
    } else if (pinned) {
      prod(IConst<1>{}, IConst<0>{});
    } else {
      prod(IConst<KRES ? 1 : 0>{}, IConst<1>{});
    }
    const int t = 16 * w + l16;
    const float gt = GATED ? sG[t] : 0.0f;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tj = 16 * jt + 4 * lq + i;
        const float ratio = GATED ? __expf(gt - sG[tj]) : 1.0f;
        acc[jt][i] = (jt <= w && tj <= t) ? kscale * ratio * acc[jt][i] : 0.0f;
      }
    bf16 *md = tout + ci * CHUNKW + TDUMP;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      if (2 * sb <= w) {
        const int j = w < 2 ? w : 2 + 2 * (w - 2) + sb;  // block (mt = w, s = sb)
        bf16x8 hi, lo;
        split8(acc[2 * sb], acc[2 * sb + 1], hi, lo);
        *reinterpret_cast<bf16x8 *>(md + ((2 * j) * 64 + l) * 8) = hi;
        *reinterpret_cast<bf16x8 *>(md + ((2 * j + 1) * 64 + l) * 8) = lo;
      }
    }
  }

  // the next chunk's queries and scalars (this chunk's are in use no longer)
  if (ci + (int64_t)gridDim.x < nch) fetch(ci + gridDim.x, IConst<1>{});

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
    // (the chunk's mark selects the form outside the loop, so that no branch
    // separates a slab's operand reads from its products)
    auto gram = [&](auto NS, auto PIN) __attribute__((always_inline)) {
      constexpr int ns = decltype(NS)::value;
      constexpr bool pin = decltype(PIN)::value;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ko = 32 * kk + 8 * lq;
        bf16x8 ka[ns], bh[ns], bl[ns];
#pragma unroll
        for (int q = 0; q < ns; ++q) {
          ka[q] = ld8(&sKl[16 * rts[q] + l16][ko]);
          if (!pin) bh[q] = ld8(&sKh[16 * tjs[q] + l16][ko]);
          if (KRES || pin) bl[q] = ld8(&sKl[16 * tjs[q] + l16][ko]);
        }
        if (!pin) {
#pragma unroll
          for (int q = 0; q < ns; ++q) acc[q] = mfma32(ka[q], bh[q], acc[q]);
        }
        if (KRES || pin) {
#pragma unroll
          for (int q = 0; q < ns; ++q) acc[q] = mfma32(ka[q], bl[q], acc[q]);
        }
      }
    };
    if (w < 2) {
      if (pinned)
        gram(IConst<3>{}, IConst<1>{});
      else
        gram(IConst<3>{}, IConst<0>{});
    } else {
      if (pinned)
        gram(IConst<2>{}, IConst<1>{});
      else
        gram(IConst<2>{}, IConst<0>{});
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (q < 2 || w < 2) {
        const int rt = rts[q], nn = 16 * tjs[q] + l16;
        const float gn = GATED ? sG[nn] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mrow = 16 * rt + 4 * lq + i;
          const float ratio = GATED ? __expf(sG[mrow] - gn) : 1.0f;
          sA[mrow][nn] = nn < mrow ? sBeta[mrow] * ratio * kscale * acc[q][i] : 0.0f;
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
  // Tm to the workspace in the sweep's operand order: block j of
  // (mt, s) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1), lane (l16, g) holding row
  // 16 mt + l16 at columns 32 s + 4 g + {0..3} and 32 s + 16 + 4 g + {0..3}
  // (the blocks above the diagonal are zero and are not stored)
  bf16 *dst = tout + ci * CHUNKW;
  for (int e = tid; e < 6 * 64; e += 256) {
    const int j = e >> 6, ln = e & 63;
    const int mt = j < 2 ? j : 2 + ((j - 2) >> 1), sb = j < 2 ? 0 : ((j - 2) & 1);
    const int row = 16 * mt + (ln & 15), c0 = 32 * sb + 4 * (ln >> 4);
    *reinterpret_cast<bf16x8 *>(dst + e * 8) = cat8(ld4(&sTr[row][c0]), ld4(&sTr[row][c0 + 16]));
  }
  // beta and the decay factors, as the sweep reads them
  {
    float *sc = reinterpret_cast<float *>(dst + TDUMP + MDUMP);
    if (tid < C) sc[tid] = sBeta[tid];
    else if (GATED && tid < 2 * C) sc[tid] = __expf(sG[tid - C]);
    else if (GATED && tid < 3 * C) sc[tid] = __expf(sG[C - 1] - sG[tid - 2 * C]);
  }
  __syncthreads();  // the next chunk's rows overwrite Tm's buffers
  }
}

// ============================================================ sweep
// Transposed operand read (gfx950 ds_read_b64_tr_b16).  Within each group of
// 16 lanes, with D[i][p] the p-th bf16 at lane i's address, lane j receives
// D[4 e + j / 4][j % 4] as element e.  Lane i of the group pointing at row
// r0 + i / 4, column c0 + 4 (i % 4) of a row-major bf16 matrix X therefore
// receives X[r0 + e][c0 + j], e < 4: four consecutive rows of column c0 + j.
__device__ __forceinline__ bf16x4 ld4_tr(const bf16 *p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4 *)(const_cast<bf16 *>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// 128-wide bf16 rows without padding: the 16-byte chunk c of row r sits at
// chunk c ^ (r & 15), so that sixteen consecutive rows read at one column
// hit sixteen different chunk positions.  Element offset of (r, c):
__device__ __forceinline__ int sx128(int r, int c) { return r * 128 + ((((c >> 3) ^ r) & 15) << 3) + (c & 7); }

// Contraction slabs in "tile order".  A 16 x 16 result tile leaves lane
// (n = l % 16, g = l / 16) holding rows 4 g .. 4 g + 3 of column n.  Two such
// tiles covering rows [32 s, 32 s + 32) of a matrix therefore give every lane
// the B operand of a 16x16x32 product over those rows with the contraction
// index kappa = 8 g + p mapped to row 32 s + 4 g + p (p < 4) or
// 32 s + 16 + 4 g + (p - 4) (p >= 4) -- no data movement.  The A operand of
// the same product must then take its columns in that order: two 8-byte
// pieces per lane instead of one 16-byte read.
__device__ __forceinline__ bf16x8 lda_tile_order(const bf16 *X, int row, int s, int g) {
  const int c0 = 32 * s + 4 * g;
  return cat8(*reinterpret_cast<const bf16x4 *>(X + sx128(row, c0)),
              *reinterpret_cast<const bf16x4 *>(X + sx128(row, c0 + 16)));
}
// A operand with m over columns [16 kt, 16 kt + 16) of a row-major key matrix
// and the contraction over its rows in tile order (slab s): transposed reads.
__device__ __forceinline__ bf16x8 lda_tr_tile_order(const bf16 *X, int kt, int s, int g, int j) {
  const int col = 16 * kt + 4 * (j & 3), r = 32 * s + 4 * g + (j >> 2);
  return cat8(ld4_tr(X + sx128(r, col)), ld4_tr(X + sx128(r + 16, col)));
}

// Workgroup barrier that does not wait for this wave's outstanding global
// loads (the next chunk's inputs stay in flight across it); LDS writes
// before it are complete.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS of one chunk's inputs (the sweep keeps two: the current chunk and the
// next one, which the loader waves fill while the current one is used).
struct SwBuf {
  static constexpr int Q = 0;               // bf16 [64][128] queries (sx128)
  static constexpr int K = Q + C * KD * 2;  // bf16 [64][128] keys (sx128)
  static constexpr int W = K + C * KD * 2;  // bf16 [64][128] write-key residual E, or k~ itself (sx128)
  static constexpr int V = W + C * KD * 2;  // bf16 [64][32] value tile
  static constexpr int BETA = V + C * 32 * 2;  // f32 [64], zero past the chunk end
  static constexpr int G = BETA + C * 4;       // f32 [64] e^{g_t} (g the cumulative log decay)
  static constexpr int GR = G + C * 4;         // f32 [64] e^{g_L - g_t}
  static constexpr int TM = GR + C * 4;        // bf16x8 [6][64] (I + A)^-1 operands (TDUMP order)
  static constexpr int BYTES = TM + 6 * 64 * 16;
};

// Phase 2 sweep over the chunks of one (b,h) and 32 value rows.  Eight waves,
// two to a SIMD:
//  waves 0, 1 ("chain" waves) own value rows v0 + 16 w .. + 16 of the state
//    with every key column, as 16 x 16 tiles of S^T in registers, and run the
//    state-dependent chain of every chunk without waiting for any other wave:
//      X = K S^T, R = B (V - diag(e^g) X), Delta = Tm R,
//      S <- e^{g_L} S + Delta^T (e^{g_L - g} . K~)
//    (S as hi + lo bf16 operands taken straight from the result tiles in
//    tile order; K~ = k + E as the two exact bf16 operands k and E, or d_min k
//    on a chunk phase 1 took as pinned on d_min);
//  waves 2, 3 ("output" waves) produce the outputs of two token-row tiles
//    each, transposed,
//      O^T = q_scale (e^g S_n Q^T + Delta^T M^T),
//    from S_n and Delta, which the chain waves leave in LDS as their operand
//    registers, and the scores M, formed chunk-parallel beside Tm;
//  waves 4 .. 7 ("loader" waves) bring the next chunk's rows, value tile,
//    (I + A)^-1 operands and scalars into the other buffer.  A wave moves
//    data from L2 at a limited rate of its own, so four waves share the
//    chunk's rows.
// Two barriers per chunk: after the chain waves have Delta (and the output
// waves Q S^T), and at the end of the chunk (next chunk's inputs in place,
// the new state written out).  A loader reaches the first one without
// waiting for its loads.
template <bool GATED, bool KRES, bool VL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void chunk_sweep_kernel(ChunkArgs a, const bf16 *tdump, int64_t N) {
  typedef SwBuf L;
  __shared__ __attribute__((aligned(16))) unsigned char lb0[L::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lb1[L::BYTES];
  // the chain waves' S operands [chain][s hi, s lo ...][lane] and Delta operands [chain][slot][lane]
  __shared__ bf16x8 sdump[2][8][64];
  __shared__ bf16x8 ddump[2][4][64];

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = l & 15, g = l >> 4;
  const int hw = w & 1;  // chain index (value rows 16 hw ..) or output-wave index
  // XCD-aware placement: block i runs on XCD i % 8; the NT value tiles of one
  // sequence share i % 8, so their reads of the same rows meet in one L2.
  const int bid = blockIdx.x;
  const int slot = bid & 7, rest = bid >> 3;
  const int vt = rest % NT;
  const int64_t seq = (int64_t)(rest / NT) * 8 + slot;
  const int64_t H = a.H;
  if (seq >= a.B * H) return;
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);
  const int64_t Nb = (T + C - 1) / C;
  const int v0 = vt * VT;

  const int64_t tstride = H * KD;
  const int64_t rowb = tstride * 2;  // bytes between tokens
  const int64_t base = tb * tstride + h * KD;
  const bf16 *tseq = tdump + seq * N * CHUNKW;
  const int *pins = KRES && a.pin ? a.pin + seq * N : nullptr;
  // a chunk's mark from the chunked phase 1 (loaded a chunk ahead)
  auto load_pin = [&](int64_t n) -> int { return pins && n < Nb ? pins[n] : 0; };
  auto chunk_len = [&](int64_t n) -> int { return (int)((T - n * C) < C ? (T - n * C) : C); };

  if (w < 2) {
    // ================================================================ chain waves
    const int vc = v0 + 16 * hw;  // first value row
    // tiles of S^T: element i of tile kt is S[vc + l16][16 kt + 4 g + i];
    // Bh / Bl: S as hi / lo operands over the key index in tile order
    floatx4 ST[8];
    bf16x8 Bh[4], Bl[4];
    bf16x8 Tm[6];  // this chunk's (I + A)^-1 operands (from LDS: the loader waves copy them)
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
      ST[kt] = a.S0 ? *reinterpret_cast<const floatx4 *>(a.S0 + (seq * VD + vc + l16) * KD + 16 * kt + 4 * g)
                    : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      split8(ST[2 * s], ST[2 * s + 1], Bh[s], Bl[s]);
      sdump[hw][2 * s][l] = Bh[s];
      sdump[hw][2 * s + 1][l] = Bl[s];
    }
    int pin_next = load_pin(0);
    lds_barrier();

    // The state update reads its operands from LDS one stage ahead of the
    // matrix-core instructions that use them (the scheduling fences keep the
    // compiler from regrouping the reads behind their uses); its first
    // operands do not depend on Delta and are requested before it is formed.
    // PIN: the chunk's write keys are d_min k.
    auto body = [&](auto PIN, int64_t n, const unsigned char *cur) __attribute__((always_inline)) {
      constexpr bool pinned = KRES && decltype(PIN)::value;
      // the state update reads one key matrix (k on a pinned chunk, k~ without
      // the residual form) or two (k and E)
      constexpr bool two = KRES && !pinned;
      constexpr int KPS = two ? 2 : 4;        // key tiles per stage
      constexpr int NST = 2 * (8 / KPS);      // stages
      const bf16 *sK = reinterpret_cast<const bf16 *>(cur + L::K);
      const bf16 *sW = reinterpret_cast<const bf16 *>(cur + L::W);
      const bf16 *sU = KRES ? sK : sW;        // k (with E as the second), or k~
      const bf16 *sV = reinterpret_cast<const bf16 *>(cur + L::V);
      const float *sBeta = reinterpret_cast<const float *>(cur + L::BETA);
      const float *sG = reinterpret_cast<const float *>(cur + L::G);
      const float *sGR = reinterpret_cast<const float *>(cur + L::GR);
      pin_next = load_pin(n + 1);

      // X = K S^T (token rows x this wave's 16 value rows).  V and beta do
      // not depend on S: their reads go out behind the key operands of the
      // second and third slabs, so that they are in place when X is done.
      floatx4 X[4];
      bf16x4 vv[4];
      floatx4 bt[4], em[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) X[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      // (the key operands of slab s + 1 are requested before the products of
      // slab s)
      bf16x8 ak[2][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) ak[0][mt] = lda_tile_order(sK, 16 * mt + l16, 0, g);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s + 1 < 4) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) ak[(s + 1) & 1][mt] = lda_tile_order(sK, 16 * mt + l16, s + 1, g);
        }
        if (s == 1) {
          // V[16 mt + 4 g + i][vc + l16] by one transposed read
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) vv[mt] = ld4_tr(sV + (16 * mt + 4 * g + (l16 >> 2)) * 32 + 16 * hw + 4 * (l16 & 3));
        } else if (s == 2) {
          // beta and e^g of tokens 16 mt + 4 g .. + 3 as one piece each
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) bt[mt] = *reinterpret_cast<const floatx4 *>(sBeta + 16 * mt + 4 * g);
        } else if (s == 3 && !GATED) {
#pragma unroll
          for (int j = 0; j < 6; ++j) Tm[j] = *reinterpret_cast<const bf16x8 *>(cur + L::TM + (j * 64 + l) * 16);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) X[mt] = mfma32(ak[s & 1][mt], Bh[s], X[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) X[mt] = mfma32(ak[s & 1][mt], Bl[s], X[mt]);
        if (s < 3) __builtin_amdgcn_sched_barrier(0);  // (R may start under the last slab's products)
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        em[mt] = GATED ? *reinterpret_cast<const floatx4 *>(sG + 16 * mt + 4 * g) : floatx4{1.f, 1.f, 1.f, 1.f};
      if (GATED) {
#pragma unroll
        for (int j = 0; j < 6; ++j) Tm[j] = *reinterpret_cast<const bf16x8 *>(cur + L::TM + (j * 64 + l) * 16);
      }
      __builtin_amdgcn_sched_barrier(0);
      // R = beta (V - e^g X)
      floatx4 R[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) R[mt][i] = bt[mt][i] * (to_f32(vv[mt][i]) - em[mt][i] * X[mt][i]);
      }
      bf16x8 Rh[2], Rl[2];
      split8(R[0], R[1], Rh[0], Rl[0]);
      split8(R[2], R[3], Rh[1], Rl[1]);
      // Delta = Tm R (Tm lower triangular: token rows below 32 need slab 0 only)
      floatx4 D[4];
      D[0] = mfma32(Tm[0], Rh[0], floatx4{0.f, 0.f, 0.f, 0.f});
      D[1] = mfma32(Tm[1], Rh[0], floatx4{0.f, 0.f, 0.f, 0.f});
      D[2] = mfma32(Tm[2], Rh[0], floatx4{0.f, 0.f, 0.f, 0.f});
      D[3] = mfma32(Tm[4], Rh[0], floatx4{0.f, 0.f, 0.f, 0.f});
      D[0] = mfma32(Tm[0], Rl[0], D[0]);
      D[1] = mfma32(Tm[1], Rl[0], D[1]);
      D[2] = mfma32(Tm[2], Rl[0], D[2]);
      D[3] = mfma32(Tm[4], Rl[0], D[3]);
      D[2] = mfma32(Tm[3], Rh[1], D[2]);
      D[3] = mfma32(Tm[5], Rh[1], D[3]);
      D[2] = mfma32(Tm[3], Rl[1], D[2]);
      D[3] = mfma32(Tm[5], Rl[1], D[3]);
      // the state update's first operands (stage 0: slab 0, key tiles 0 ..)
      bf16x8 ua[4], ub[4], una[4], unb[4];
#pragma unroll
      for (int u = 0; u < KPS; ++u) {
        ua[u] = lda_tr_tile_order(sU, u, 0, g, l16);
        if (two) ub[u] = lda_tr_tile_order(sW, u, 0, g, l16);
      }
      // Delta for the outputs (output waves), as tile-order hi/lo operands
      bf16x8 Dh[2], Dl[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        split8(D[2 * s], D[2 * s + 1], Dh[s], Dl[s]);
        ddump[hw][2 * s][l] = Dh[s];
        ddump[hw][2 * s + 1][l] = Dl[s];
      }
      // the state update's Delta, decayed to the chunk end (and scaled by
      // d_min when the write keys are d_min k); without decay the same
      // operands serve, and d_min scales the pinned chunk's product instead
      if (GATED) {
        const float dscale = pinned ? a.d_min : 1.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const floatx4 gr = *reinterpret_cast<const floatx4 *>(sGR + 16 * mt + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) D[mt][i] *= dscale * gr[i];
        }
        split8(D[0], D[1], Dh[0], Dl[0]);
        split8(D[2], D[3], Dh[1], Dl[1]);
      }
      lds_barrier();  // ---- B2: Delta is in LDS, the output waves are done with S_n
      // S <- e^{g_L} S + K~^T Delta, stage by stage
      constexpr bool apart = pinned && !GATED;  // K^T Delta formed apart, then d_min times it added
      floatx4 P[8];
      if (GATED) {
        const float decay = sG[C - 1];  // e^{g_L}
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) ST[kt] = ST[kt] * decay;
      }
      if (apart) {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) P[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      // key tiles 2 sp, 2 sp + 1 are final after stage done(sp); they are
      // split into the next chunk's operands (and left for the output waves)
      // during the following stage's products, or, in the last stage, after
      // its own products of them
      constexpr bool OVL = !GATED;
      auto done = [](int sp) { return NST / 2 + (2 * sp + 1) / KPS; };
      auto finish = [&](int sp) __attribute__((always_inline)) {
        if (apart) {
#pragma unroll
          for (int kt = 2 * sp; kt < 2 * sp + 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) ST[kt][i] = fmaf(a.d_min, P[kt][i], ST[kt][i]);
        }
        split8(ST[2 * sp], ST[2 * sp + 1], Bh[sp], Bl[sp]);
        sdump[hw][2 * sp][l] = Bh[sp];
        sdump[hw][2 * sp + 1][l] = Bl[sp];
      };
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int s = st / (NST / 2), k0 = (st % (NST / 2)) * KPS;
        if (st + 1 < NST) {
          const int s1 = (st + 1) / (NST / 2), k1 = ((st + 1) % (NST / 2)) * KPS;
#pragma unroll
          for (int u = 0; u < KPS; ++u) {
            una[u] = lda_tr_tile_order(sU, k1 + u, s1, g, l16);
            if (two) unb[u] = lda_tr_tile_order(sW, k1 + u, s1, g, l16);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < KPS; ++u) {
          if (apart) {
            P[k0 + u] = mfma32(ua[u], Dh[s], P[k0 + u]);
            P[k0 + u] = mfma32(ua[u], Dl[s], P[k0 + u]);
          } else {
            ST[k0 + u] = mfma32(ua[u], Dh[s], ST[k0 + u]);
            ST[k0 + u] = mfma32(ua[u], Dl[s], ST[k0 + u]);
            if (two) {
              ST[k0 + u] = mfma32(ub[u], Dh[s], ST[k0 + u]);
              ST[k0 + u] = mfma32(ub[u], Dl[s], ST[k0 + u]);
            }
          }
        }
#pragma unroll
        for (int sp = 0; sp < 4; ++sp)
          if (OVL && (done(sp) == st - 1 || (st == NST - 1 && done(sp) == st))) finish(sp);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < KPS; ++u) {
          ua[u] = una[u];
          if (two) ub[u] = unb[u];
        }
      }
#pragma unroll
      for (int sp = 0; sp < 4; ++sp)
        if (!OVL) finish(sp);
      lds_barrier();  // ---- B1 of the next chunk
    };
    auto run = [&](int64_t n, const unsigned char *cur) __attribute__((always_inline)) {
      if (__builtin_amdgcn_readfirstlane(pin_next) == 2)
        body(IConst<1>{}, n, cur);
      else
        body(IConst<0>{}, n, cur);
    };
    for (int64_t n = 0; n < Nb; n += 2) {
      run(n, lb0);
      if (n + 1 < Nb) run(n + 1, lb1);
    }
    if (a.S_out) {
#pragma unroll
      for (int kt = 0; kt < 8; ++kt)
        *reinterpret_cast<floatx4 *>(a.S_out + (seq * VD + vc + l16) * KD + 16 * kt + 4 * g) = ST[kt];
    }
  } else if (w < 4) {
    // ================================================================ output waves
    lds_barrier();
    auto body = [&](int64_t n, const unsigned char *cur) {
      const bf16 *sQ = reinterpret_cast<const bf16 *>(cur + L::Q);
      const float *sG = reinterpret_cast<const float *>(cur + L::G);
      const int64_t t0 = n * C;
      const int Lc = chunk_len(n);
      // this chunk's scores (formed chunk-parallel with Tm) for token-row tiles
      // mts[0] = hw (slab 0) and mts[1] = 3 - hw (slabs 0, 1), hi/lo operands;
      // needed only after the first barrier
      const int mts[2] = {hw, 3 - hw};
      const bf16 *md = tseq + n * CHUNKW + TDUMP;
      const int js[3] = {hw, 4 - 2 * hw, 5 - 2 * hw};
      bf16x8 Mh[3], Ml[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        Mh[u] = ld8(md + ((2 * js[u]) * 64 + l) * 8);
        Ml[u] = ld8(md + ((2 * js[u] + 1) * 64 + l) * 8);
      }
      // O^T = e^g S_n Q^T (value rows x token columns) for both token tiles and
      // both value tiles (S_n as the chain waves left it): an operand register
      // of a 16x16x32 product holds X[i][kappa] for lane (i, g) whether it
      // serves as the A operand of X or the B operand of X^T, so the chain's
      // S^T operands and the query operands serve with their roles swapped,
      // and each lane ends up with four consecutive values of one token.
      floatx4 O[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 aq[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) aq[s] = lda_tile_order(sQ, 16 * mts[u] + l16, s, g);
        const float eg = GATED ? sG[16 * mts[u] + l16] : 1.0f;  // e^g of token column l16
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            acc = mfma32(sdump[c][2 * s][l], aq[s], acc);
            acc = mfma32(sdump[c][2 * s + 1][l], aq[s], acc);
          }
          if (GATED) acc = acc * eg;
          O[u][c] = acc;
        }
      }
      lds_barrier();  // ---- B2: Delta is in LDS; the chain waves may rewrite S
      // O^T += Delta^T M^T (tile 0: slab 0; tile 1: slabs 0 and 1)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 d0h = ddump[c][0][l], d0l = ddump[c][1][l];
        const bf16x8 d1h = ddump[c][2][l], d1l = ddump[c][3][l];
        O[0][c] = mfma32(d0h, Mh[0], O[0][c]);
        O[1][c] = mfma32(d0h, Mh[1], O[1][c]);
        O[0][c] = mfma32(d0l, Mh[0], O[0][c]);
        O[1][c] = mfma32(d0l, Mh[1], O[1][c]);
        O[0][c] = mfma32(d0h, Ml[0], O[0][c]);
        O[1][c] = mfma32(d0h, Ml[1], O[1][c]);
        O[1][c] = mfma32(d1h, Mh[2], O[1][c]);
        O[1][c] = mfma32(d1l, Mh[2], O[1][c]);
        O[1][c] = mfma32(d1h, Ml[2], O[1][c]);
      }
      // lane (l16, g): token 16 mt + l16, value columns 16 c + 4 g .. + 3
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int m = 16 * mts[u] + l16;
        if (m < Lc) {
          const int64_t oi = base + v0 + (t0 + m) * tstride + 4 * g;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const floatx4 x = O[u][c] * a.q_scale;
            if (a.o_f32)
              *reinterpret_cast<floatx4 *>(static_cast<float *>(a.o) + oi + 16 * c) = x;
            else
              *reinterpret_cast<bf16x4 *>(static_cast<bf16 *>(a.o) + oi + 16 * c) = pack4(x);
          }
        }
      }
      lds_barrier();  // ---- B1 of the next chunk
    };
    for (int64_t n = 0; n < Nb; n += 2) {
      body(n, lb0);
      if (n + 1 < Nb) body(n + 1, lb1);
    }
  } else {
    // ================================================================ loader waves
    // Loader li brings, for a chunk: the 1 KB blocks j = 4 jj + li (jj < 4) of
    // the query, key and write-key rows (block j: rows 4 j .., lane l -> row
    // 4 j + l / 16, 16-byte piece l % 16 stored at position (l % 16) ^ (row %
    // 16), the sx128 layout), block li of the value tile (rows 16 li + l / 4,
    // piece l % 4), blocks li and li + 4 (< 6) of the (I + A)^-1 operands, and
    // (li = 0) beta, (li = 1) e^{g_t} or (li = 2) e^{g_L - g_t}, as the UT
    // transform writes them (beta zero past the chunk end, g constant past it).
    // Rows past T read the chunk's first row (their beta is zero).
    const int li = w - 4;
    const char *qb = reinterpret_cast<const char *>(static_cast<const bf16 *>(a.q) + base);
    const char *kb = reinterpret_cast<const char *>(static_cast<const bf16 *>(a.k) + base);
    const char *eb = reinterpret_cast<const char *>(static_cast<const bf16 *>(a.kt) + base);
    const char *vb = reinterpret_cast<const char *>(static_cast<const bf16 *>(a.v) + base + v0);
    const int r0 = 4 * li + (l >> 4);  // row of block jj = 0; block jj adds 16 jj
    const uint32_t rcol = (uint32_t)(16 * (((l & 15) ^ r0) & 15));  // the same for every block
    const int vrow = 16 * li + (l >> 2);
    const uint32_t vcol = (uint32_t)(16 * (l & 3)), voff = (uint32_t)(vrow * rowb) + vcol;
    // chunk n's pieces: loaded into registers, then (after the first barrier,
    // which does not wait for them) written to buffer lb; a chunk whose write
    // keys are d_min k (mark 2) has its residual neither loaded nor written
    auto fill = [&](int64_t n, unsigned char *lb, int pin, bool mid_barrier) {
      const bool skip_w = __builtin_amdgcn_readfirstlane(pin) == 2;
      const int64_t t0 = n * C;
      const int Lc = chunk_len(n);
      const char *q0 = qb + t0 * rowb, *k0 = kb + t0 * rowb, *e0 = eb + t0 * rowb, *vv = vb + t0 * rowb;
      // (held as wide vector values, not arrays, so that they stay in
      // registers across the barrier)
      typedef unsigned u32x16 __attribute__((ext_vector_type(16)));
      u32x16 rq = {}, rk = {}, rw = {};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = r0 + 16 * jj;
        const uint32_t off = r < Lc ? (uint32_t)(r * rowb) + rcol : rcol;
        const uint4 x = *reinterpret_cast<const uint4 *>(q0 + off);
        const uint4 y = *reinterpret_cast<const uint4 *>(k0 + off);
        rq[4 * jj] = x.x; rq[4 * jj + 1] = x.y; rq[4 * jj + 2] = x.z; rq[4 * jj + 3] = x.w;
        rk[4 * jj] = y.x; rk[4 * jj + 1] = y.y; rk[4 * jj + 2] = y.z; rk[4 * jj + 3] = y.w;
        if (!skip_w) {
          const uint4 z = *reinterpret_cast<const uint4 *>(e0 + off);
          rw[4 * jj] = z.x; rw[4 * jj + 1] = z.y; rw[4 * jj + 2] = z.z; rw[4 * jj + 3] = z.w;
        }
      }
      const uint4 rv = *reinterpret_cast<const uint4 *>(vv + (vrow < Lc ? voff : vcol));
      const bf16 *tm = tseq + n * CHUNKW;
      const uint4 rt0 = *reinterpret_cast<const uint4 *>(tm + (li * 64 + l) * 8);
      uint4 rt1 = {0u, 0u, 0u, 0u};
      if (li < 2) rt1 = *reinterpret_cast<const uint4 *>(tm + ((li + 4) * 64 + l) * 8);
      const float *sc = reinterpret_cast<const float *>(tm + TDUMP + MDUMP);
      float rs = 0.0f;
      if (li == 0) rs = sc[l];
      else if (GATED && li < 3) rs = sc[64 * li + l];
      if (mid_barrier) lds_barrier();  // ---- B2 (no wait for the loads)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * jj + li;
        *reinterpret_cast<uint4 *>(lb + L::Q + 1024 * j + 16 * l) =
            uint4{rq[4 * jj], rq[4 * jj + 1], rq[4 * jj + 2], rq[4 * jj + 3]};
        *reinterpret_cast<uint4 *>(lb + L::K + 1024 * j + 16 * l) =
            uint4{rk[4 * jj], rk[4 * jj + 1], rk[4 * jj + 2], rk[4 * jj + 3]};
        if (!skip_w)
          *reinterpret_cast<uint4 *>(lb + L::W + 1024 * j + 16 * l) =
              uint4{rw[4 * jj], rw[4 * jj + 1], rw[4 * jj + 2], rw[4 * jj + 3]};
      }
      *reinterpret_cast<uint4 *>(lb + L::V + 1024 * li + 16 * l) = rv;
      *reinterpret_cast<uint4 *>(lb + L::TM + (li * 64 + l) * 16) = rt0;
      if (li < 2) *reinterpret_cast<uint4 *>(lb + L::TM + ((li + 4) * 64 + l) * 16) = rt1;
      if (li == 0) reinterpret_cast<float *>(lb + L::BETA)[l] = rs;
      else if (GATED && li == 1) reinterpret_cast<float *>(lb + L::G)[l] = rs;
      else if (GATED && li == 2) reinterpret_cast<float *>(lb + L::GR)[l] = rs;
    };
    int pin_next = load_pin(1);
    if (Nb > 0) fill(0, lb0, load_pin(0), false);
    lds_barrier();
    auto body = [&](int64_t n, unsigned char *nxt) {
      const int pin = pin_next;
      pin_next = load_pin(n + 2);
      if (n + 1 < Nb)
        fill(n + 1, nxt, pin, true);
      else
        lds_barrier();  // ---- B2
      lds_barrier();    // ---- B1 of the next chunk
    };
    for (int64_t n = 0; n < Nb; n += 2) {
      body(n, lb1);
      if (n + 1 < Nb) body(n + 1, lb0);
    }
  }
}

// Compute units of the current device (queried each call: a host-side
// attribute read, no device work).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
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
  hipLaunchKernelGGL((chunk_sweep_kernel<GATED, KRES, VL>), dim3((unsigned)(groups * 8 * NT)), dim3(512), 0, s, a,
                     (const bf16 *)tw, N);
  prof_mark(s, "chunk_sweep_kernel");
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
  return (size_t)(B * H * N) * CHUNKW * 2;
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
