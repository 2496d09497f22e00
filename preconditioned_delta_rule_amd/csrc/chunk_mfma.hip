// Phase 2 of OSDN on the matrix cores: chunkwise WY delta rule, bf16 operands,
// fp32 accumulation, K = V = 128, chunk C = 64.
//
// Paper: Section 4.3 Eq.(5)-(6) (write key K~ in the chunk Gram and in the
// intra-chunk score, physical key K in the residual), Appendix A.2
// Eqs.(8)-(11); with a decay alpha, Appendix B.1 Eqs.(13)-(15).  Per chunk,
// with boundary state S (V x K, fp32), B = diag(beta) and in-chunk log decay
// g_i = sum_{l<=i} log alpha_l (g = 0 without decay):
//   A     = strict_lower(B [e^{g_i-g_j}] . K K~^T)      (MFMA)
//   Tm    = (I + A)^-1                                  (forward substitution
//                                                        on 16x16 diagonal
//                                                        blocks, MFMA merges)
//   R     = V - diag(e^g) K S^T                         (MFMA)
//   Delta = Tm B R            (= U - W S^T of Eq.(11))   (MFMA)
//   O     = q_scale (diag(e^g) Q S^T + lower([e^{g_i-g_j}] . Q K~^T) Delta)
//   S    <- e^{g_L} S + Delta^T (e^{g_L - g} . K~)       (MFMA, S stays in the
//                                                        accumulators)
// Work split: one workgroup of 4 waves per (b,h) and tile of VT value rows,
// so a (b,h) is spread over 128/VT CUs; the tiles of one (b,h) are placed on
// the same XCD so their shared K/K~/Q reads hit that XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace osdn {

namespace {

constexpr int C = 64;      // chunk length
constexpr int KD = 128;    // key dim
constexpr int VD = 128;    // value dim
constexpr int KP = KD + 8; // LDS pitch (bf16) of 128-wide rows
constexpr int CP = C + 8;  // LDS pitch (bf16) of 64-wide rows
constexpr int AP = C + 4;  // LDS pitch (f32) of the Gram
constexpr int NTHREADS = 256;

typedef short shortx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(bf16x4 a, bf16x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 16x16 tile of X Y^T over `kdim` (multiple of 32): X, Y point at the first
// row of 16-row tiles stored row-major with the given pitch (bf16 elements).
// Lane l supplies row (l & 15) and k-slice 8*(l >> 4) of each 32-wide step;
// the result holds D[4*(l>>4) + i][l & 15] in element i.
__device__ __forceinline__ floatx4 tile_nt(const bf16 *X, int ldx, const bf16 *Y, int ldy,
                                           int k0, int k1, floatx4 acc, int l) {
  const int r = l & 15, ks = (l >> 4) * 8;
  for (int k = k0; k < k1; k += 32) {
    bf16x8 x = *reinterpret_cast<const bf16x8 *>(X + r * ldx + k + ks);
    bf16x8 y = *reinterpret_cast<const bf16x8 *>(Y + r * ldy + k + ks);
    acc = mfma32(x, y, acc);
  }
  return acc;
}

__device__ __forceinline__ bf16x4 pack4(floatx4 v) {
  bf16x4 r;
  r[0] = to_bf16(v[0]);
  r[1] = to_bf16(v[1]);
  r[2] = to_bf16(v[2]);
  r[3] = to_bf16(v[3]);
  return r;
}

template <int VT> struct Smem {
  bf16 K[C][KP];      // physical keys of the chunk, row-major
  bf16 Kt[C][KP];     // write keys, row-major
  bf16 Q[C][KP];      // queries, row-major
  bf16 KtT[KD][CP];   // write keys transposed ([c][j]), operand of the state update
  bf16 V[C][VT + 8];  // value tile
  float A[C][AP];     // chunk Gram (strict lower, gated, beta-scaled), fp32
  bf16 Tr[C][CP];     // (I + A)^-1 row-major
  bf16 Tc[C][CP];     // (I + A)^-1 column-major ([j][i]), for the merges
  bf16 X[C][CP];      // merge scratch, column-major
  bf16 M[C][CP];      // local scores (lower incl. diagonal, gated)
  bf16 RT[VT][CP];    // (B R)^T
  bf16 DT[VT][CP];    // Delta^T
  bf16 DTs[VT][CP];   // Delta^T scaled by the suffix decay (gated form)
  bf16 S[VT][KP];     // bf16 copy of the state tile, row-major [v][c]
  float beta[C];
  float g[C];         // inclusive in-chunk cumulative log decay
};

template <int VT, bool GATED>
__global__ __launch_bounds__(NTHREADS) void chunk_mfma_kernel(ChunkArgs a) {
  constexpr int NT = VD / VT;          // value tiles per (b,h)
  constexpr int NCT = VT / 16;         // 16-wide column tiles per value tile
  __shared__ __attribute__((aligned(16))) Smem<VT> sm;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
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
  bf16 *go = static_cast<bf16 *>(a.o);
  const int64_t tstride = H * KD;  // elements between tokens (K == V == 128)

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
        float s0 = a.S0 ? a.S0[(seq * VD + v0 + vr) * KD + c] : 0.0f;
        Sacc[rt][ct][i] = s0;
        sm.S[vr][c] = to_bf16(s0);
      }

  // ---- global -> register prefetch of one chunk
  // K, K~, Q: 64 rows x 16 vectors of 8 bf16; thread covers vectors tid + 256 p.
  // V tile: 64 rows x VT/8 vectors.
  constexpr int VV = VT / 8;  // vectors per value-tile row
  bf16x8 pk[4], pkt[4], pq[4], pv[(C * VV + NTHREADS - 1) / NTHREADS];
  float pbeta = 0.0f, pla = 0.0f;
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int vi = tid + NTHREADS * p, i = vi >> 4, cv = vi & 15;
      const int64_t t = t0 + i;
      if (t < T) {
        const int64_t off = (b * T + t) * tstride + h * KD + cv * 8;
        pk[p] = *reinterpret_cast<const bf16x8 *>(gk + off);
        pkt[p] = *reinterpret_cast<const bf16x8 *>(gkt + off);
        pq[p] = *reinterpret_cast<const bf16x8 *>(gq + off);
      } else {
        pk[p] = bf16x8{};
        pkt[p] = bf16x8{};
        pq[p] = bf16x8{};
      }
    }
#pragma unroll
    for (int p = 0; p < (C * VV + NTHREADS - 1) / NTHREADS; ++p) {
      const int vi = tid + NTHREADS * p;
      if (vi < C * VV) {
        const int i = vi / VV, cv = vi % VV;
        const int64_t t = t0 + i;
        pv[p] = t < T ? *reinterpret_cast<const bf16x8 *>(gv + (b * T + t) * tstride + h * VD + v0 + cv * 8)
                      : bf16x8{};
      }
    }
    if (tid < C) {
      const int64_t t = t0 + tid;
      pbeta = t < T ? a.beta[(b * T + t) * H + h] : 0.0f;
      if (GATED) pla = t < T ? logf(a.alpha[(b * T + t) * H + h]) : 0.0f;
    }
  };

  if (T > 0) fetch(0);
  for (int64_t t0 = 0; t0 < T; t0 += C) {
    const int L = (int)((T - t0) < C ? (T - t0) : C);
    __syncthreads();  // previous chunk done with every LDS buffer
    // ---- stage L: registers -> LDS
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int vi = tid + NTHREADS * p, i = vi >> 4, cv = vi & 15;
      *reinterpret_cast<bf16x8 *>(&sm.K[i][cv * 8]) = pk[p];
      *reinterpret_cast<bf16x8 *>(&sm.Kt[i][cv * 8]) = pkt[p];
      *reinterpret_cast<bf16x8 *>(&sm.Q[i][cv * 8]) = pq[p];
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.KtT[cv * 8 + e][i] = pkt[p][e];
    }
#pragma unroll
    for (int p = 0; p < (C * VV + NTHREADS - 1) / NTHREADS; ++p) {
      const int vi = tid + NTHREADS * p;
      if (vi < C * VV) {
        const int i = vi / VV, cv = vi % VV;
        *reinterpret_cast<bf16x8 *>(&sm.V[i][cv * 8]) = pv[p];
      }
    }
    if (tid < C) {
      sm.beta[tid] = pbeta;
      if (GATED) {
        // inclusive scan of the log decays over the 64 lanes of wave 0
        float x = pla;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          float y = __shfl_up(x, off, 64);
          if (tid >= off) x += y;
        }
        sm.g[tid] = x;
      }
    }
    __syncthreads();
    if (t0 + C < T) fetch(t0 + C);  // overlaps with the compute below

    // ---- stage G: Gram A and scores M (lower tiles), K S^T and Q S^T
    // jobs 0..9: A tiles, 10..19: M tiles, over the 10 tiles ti >= tj.
    for (int job = w; job < 20; job += 4) {
      const int tl = job % 10;
      const int ti = tl < 1 ? 0 : tl < 3 ? 1 : tl < 6 ? 2 : 3;
      const int tj = tl - ti * (ti + 1) / 2;
      const bool isA = job < 10;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = tile_nt(isA ? &sm.K[16 * ti][0] : &sm.Q[16 * ti][0], KP, &sm.Kt[16 * tj][0], KP, 0, KD, acc, l);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * ti + 4 * lq + i, n = 16 * tj + l16;
        const float ratio = GATED ? __expf(sm.g[m] - sm.g[n]) : 1.0f;
        if (isA) {
          sm.A[m][n] = n < m ? sm.beta[m] * ratio * acc[i] : 0.0f;
        } else {
          sm.M[m][n] = to_bf16(n <= m ? ratio * acc[i] : 0.0f);
        }
      }
    }
    // zero the upper tiles that the 32-wide k-steps of later products read
    if (w < 2) {
      const int ti = 2 * w;  // tiles (0,1) and (2,3)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * ti + 4 * lq + i, n = 16 * (ti + 1) + l16;
        sm.M[m][n] = to_bf16(0.0f);
        sm.Tr[m][n] = to_bf16(0.0f);
      }
    }
    floatx4 Oacc[NCT];
    {
      const int m0 = 16 * w;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        floatx4 ks = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
        ks = tile_nt(&sm.K[m0][0], KP, &sm.S[16 * ct][0], KP, 0, KD, ks, l);
        qs = tile_nt(&sm.Q[m0][0], KP, &sm.S[16 * ct][0], KP, 0, KD, qs, l);
        bf16x4 rb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 4 * lq + i, vr = 16 * ct + l16;
          const float gm = GATED ? __expf(sm.g[m]) : 1.0f;
          rb[i] = to_bf16(sm.beta[m] * (to_f32(sm.V[m][vr]) - gm * ks[i]));
          Oacc[ct][i] = gm * qs[i];
        }
        *reinterpret_cast<bf16x4 *>(&sm.RT[16 * ct + l16][m0 + 4 * lq]) = rb;
      }
    }
    __syncthreads();

    // ---- stage T: (I + A)^-1
    // (i) wave w inverts diagonal block w by forward substitution; lane
    //     l & 15 computes column c of the block inverse in fp32.
    {
      const int c = l16, base = 16 * w;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == c) ? 1.0f : 0.0f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= sm.A[base + i][base + j] * x[j];
        x[i] = acc;
      }
      if (lq == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.Tr[base + i][base + c] = to_bf16(x[i]);
        bf16x8 lo, hi;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lo[i] = to_bf16(x[i]);
          hi[i] = to_bf16(x[i + 8]);
        }
        *reinterpret_cast<bf16x8 *>(&sm.Tc[base + c][base]) = lo;
        *reinterpret_cast<bf16x8 *>(&sm.Tc[base + c][base + 8]) = hi;
      }
    }
    __syncthreads();
    // (ii) T_{q+1,q} = -T_{q+1,q+1} A_{q+1,q} T_{q,q} for q = 0 (wave 0), 2 (wave 1)
    if (w < 2) {
      const int q = 2 * w, p = q + 1;
      bf16x4 aop, bop;
#pragma unroll
      for (int e = 0; e < 4; ++e) aop[e] = to_bf16(sm.A[16 * p + l16][16 * q + 4 * lq + e]);
      bop = *reinterpret_cast<const bf16x4 *>(&sm.Tc[16 * q + l16][16 * q + 4 * lq]);
      floatx4 X = mfma16(aop, bop, floatx4{0.f, 0.f, 0.f, 0.f});
      aop = *reinterpret_cast<const bf16x4 *>(&sm.Tr[16 * p + l16][16 * p + 4 * lq]);
      floatx4 Y = mfma16(aop, pack4(X), floatx4{0.f, 0.f, 0.f, 0.f});
      bf16x4 nt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nt[i] = to_bf16(-Y[i]);
        sm.Tr[16 * p + 4 * lq + i][16 * q + l16] = nt[i];
      }
      *reinterpret_cast<bf16x4 *>(&sm.Tc[16 * q + l16][16 * p + 4 * lq]) = nt;
    }
    __syncthreads();
    // (iii) lower-left 32x32 block: X = A_BA T_AA, then T_BA = -T_BB X,
    //       wave w owns output block (p, q) = (2 + w/2, w%2).
    {
      const int p = 2 + (w >> 1), q = w & 1;
      floatx4 X = {0.f, 0.f, 0.f, 0.f};
      for (int kb = q; kb < 2; ++kb) {
        bf16x4 aop, bop;
#pragma unroll
        for (int e = 0; e < 4; ++e) aop[e] = to_bf16(sm.A[16 * p + l16][16 * kb + 4 * lq + e]);
        bop = *reinterpret_cast<const bf16x4 *>(&sm.Tc[16 * q + l16][16 * kb + 4 * lq]);
        X = mfma16(aop, bop, X);
      }
      *reinterpret_cast<bf16x4 *>(&sm.X[16 * q + l16][16 * p + 4 * lq]) = pack4(X);
      __syncthreads();
      floatx4 Y = {0.f, 0.f, 0.f, 0.f};
      for (int mb = 2; mb <= p; ++mb) {
        bf16x4 aop = *reinterpret_cast<const bf16x4 *>(&sm.Tr[16 * p + l16][16 * mb + 4 * lq]);
        bf16x4 bop = *reinterpret_cast<const bf16x4 *>(&sm.X[16 * q + l16][16 * mb + 4 * lq]);
        Y = mfma16(aop, bop, Y);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.Tr[16 * p + 4 * lq + i][16 * q + l16] = to_bf16(-Y[i]);
    }
    __syncthreads();

    // ---- stage D: Delta = Tm (B R); wave w owns rows [16w, 16w+16)
    const float gL = GATED ? sm.g[L - 1] : 0.0f;
    {
      const int m0 = 16 * w, kend = m0 < 32 ? 32 : 64;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = tile_nt(&sm.Tr[m0][0], CP, &sm.RT[16 * ct][0], CP, 0, kend, acc, l);
        bf16x4 db, ds;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          db[i] = to_bf16(acc[i]);
          if (GATED) ds[i] = to_bf16(acc[i] * __expf(gL - sm.g[m0 + 4 * lq + i]));
        }
        *reinterpret_cast<bf16x4 *>(&sm.DT[16 * ct + l16][m0 + 4 * lq]) = db;
        if (GATED) *reinterpret_cast<bf16x4 *>(&sm.DTs[16 * ct + l16][m0 + 4 * lq]) = ds;
      }
    }
    __syncthreads();

    // ---- stage O: outputs; stage S: state update
    {
      const int m0 = 16 * w, kend = m0 < 32 ? 32 : 64;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        floatx4 acc = tile_nt(&sm.M[m0][0], CP, &sm.DT[16 * ct][0], CP, 0, kend, Oacc[ct], l);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 4 * lq + i;
          if (m < L)
            go[(b * T + t0 + m) * tstride + h * VD + v0 + 16 * ct + l16] = to_bf16(a.q_scale * acc[i]);
        }
      }
      const float decay = GATED ? __expf(gL) : 1.0f;
#pragma unroll
      for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          floatx4 acc = Sacc[rt][ct];
          if (GATED) acc = acc * decay;
          acc = tile_nt(GATED ? &sm.DTs[16 * rt][0] : &sm.DT[16 * rt][0], CP,
                        &sm.KtT[32 * w + 16 * ct][0], CP, 0, C, acc, l);
          Sacc[rt][ct] = acc;
        }
    }
    __syncthreads();  // everyone has read sm.S for this chunk
#pragma unroll
    for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.S[16 * rt + 4 * lq + i][32 * w + 16 * ct + l16] = to_bf16(Sacc[rt][ct][i]);
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
  if (a.alpha)
    hipLaunchKernelGGL((chunk_mfma_kernel<VT, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((chunk_mfma_kernel<VT, false>), grid, block, 0, s, a);
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
