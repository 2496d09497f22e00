// Phase 2 of OSDN, general shapes: the chunkwise WY delta rule in fp32
// arithmetic (any K, V <= 128, chunk C <= 64, f32 or bf16 storage).
//
// Paper: Section 4.3 Eq.(5)-(6) and Appendix A.2 Eqs.(8)-(11); with a decay
// alpha, Appendix B.1 Eqs.(13)-(15).  Per chunk of L <= C tokens with boundary
// state S (V x K), gates B = diag(beta), in-chunk log decay g_i = sum_{l<=i}
// log alpha_l (g = 0 without decay):
//   A_ij = beta_i e^{g_i - g_j} <k_i, k~_j>            (j < i)
//   R_i  = v_i - e^{g_i} S k_i
//   (I + A) Delta = B R                               (forward substitution;
//                                                       Delta = U - W S^T)
//   o_i  = e^{g_i} S (s q_i) + sum_{j<=i} e^{g_i - g_j} <s q_i, k~_j> Delta_j
//   S   <- e^{g_L} S + sum_j e^{g_L - g_j} Delta_j k~_j^T
// One workgroup of 256 threads handles one (b,h) and a tile of VT value rows;
// the chunk operands live in LDS as fp32.
#include "device_common.h"
#include "kernels.h"
#include "profile.h"

namespace osdn {

static constexpr int GEN_THREADS = 256;

struct GenLayout {
  int C, K, VT, KP;  // KP = K + 1 (LDS row pitch)
  __host__ __device__ int off_Q() const { return 0; }
  __host__ __device__ int off_K() const { return off_Q() + C * KP; }
  __host__ __device__ int off_Kt() const { return off_K() + C * KP; }
  __host__ __device__ int off_V() const { return off_Kt() + C * KP; }
  __host__ __device__ int off_A() const { return off_V() + C * VT; }
  __host__ __device__ int off_M() const { return off_A() + C * (C + 1); }
  __host__ __device__ int off_R() const { return off_M() + C * (C + 1); }
  __host__ __device__ int off_P() const { return off_R() + C * VT; }
  __host__ __device__ int off_S() const { return off_P() + C * VT; }
  __host__ __device__ int off_beta() const { return off_S() + VT * KP; }
  __host__ __device__ int off_g() const { return off_beta() + C; }
  __host__ __device__ int total() const { return off_g() + C; }
};

template <typename TIn, bool GATED, bool VL>
__global__ __launch_bounds__(GEN_THREADS) void chunk_generic_kernel(ChunkArgs a, GenLayout lay, int ntiles) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int64_t seq = blockIdx.x / ntiles;
  const int vt = blockIdx.x % ntiles;
  const int64_t H = a.H, K = a.K, V = a.V;
  const int C = lay.C, VT = lay.VT, KP = lay.KP;
  const int v0 = vt * VT;
  const int vn = (int)((V - v0) < VT ? (V - v0) : VT);  // valid rows in this tile
  const int64_t b = seq / H, h = seq - b * H;
  const int64_t T = seq_len<VL>(a, b), tb = seq_base<VL>(a, b);

  float *sQ = smem + lay.off_Q(), *sK = smem + lay.off_K(), *sKt = smem + lay.off_Kt();
  float *sV = smem + lay.off_V(), *sA = smem + lay.off_A(), *sM = smem + lay.off_M();
  float *sR = smem + lay.off_R(), *sP = smem + lay.off_P(), *sS = smem + lay.off_S();
  float *sBeta = smem + lay.off_beta(), *sG = smem + lay.off_g();
  const int CP = C + 1;

  const TIn *q = static_cast<const TIn *>(a.q);
  const TIn *k = static_cast<const TIn *>(a.k);
  const TIn *kt = static_cast<const TIn *>(a.kt);
  const TIn *v = static_cast<const TIn *>(a.v);

  for (int e = tid; e < VT * K; e += GEN_THREADS) {
    int r = e / (int)K, c = e % (int)K;
    float s0 = 0.0f;
    if (r < vn && a.S0) s0 = a.S0[(seq * V + v0 + r) * K + c];
    sS[r * KP + c] = s0;
  }

  for (int64_t t0 = 0; t0 < T; t0 += C) {
    const int L = (int)((T - t0) < C ? (T - t0) : C);
    __syncthreads();
    // ---- load the chunk (zero rows past the end of the sequence)
    for (int e = tid; e < C * K; e += GEN_THREADS) {
      int i = e / (int)K, c = e % (int)K;
      float xq = 0.0f, xk = 0.0f, xw = 0.0f;
      if (i < L) {
        int64_t g = ((tb + t0 + i) * H + h) * K + c;
        xq = to_f32(q[g]) * a.q_scale;
        xk = to_f32(k[g]);
        xw = to_f32(kt[g]) + (a.kt_is_res ? xk : 0.0f);  // k~ = k + residual
      }
      sQ[i * KP + c] = xq;
      sK[i * KP + c] = xk;
      sKt[i * KP + c] = xw;
    }
    for (int e = tid; e < C * VT; e += GEN_THREADS) {
      int i = e / VT, c = e % VT;
      float x = 0.0f;
      if (i < L && c < vn) x = to_f32(v[((tb + t0 + i) * H + h) * V + v0 + c]);
      sV[i * VT + c] = x;
    }
    if (tid < C) {
      int i = tid;
      float bt = 0.0f, la = 0.0f;
      if (i < L) {
        int64_t g = (tb + t0 + i) * H + h;
        bt = a.beta[g];
        if (GATED) la = logf(a.alpha[g]);
      }
      sBeta[i] = bt;
      sG[i] = la;
    }
    __syncthreads();
    if (GATED && tid == 0) {
      float acc = 0.0f;
      for (int i = 0; i < C; ++i) {
        acc += sG[i];
        sG[i] = acc;
      }
    }
    __syncthreads();
    // ---- chunk Gram A (strict lower), local scores M (lower incl. diagonal),
    //      residual R against the boundary state, inter-chunk readout P
    for (int e = tid; e < C * C; e += GEN_THREADS) {
      int i = e / C, j = e % C;
      float av = 0.0f, mv = 0.0f;
      if (j <= i && i < L) {
        float dk = 0.0f, dq = 0.0f;
        for (int c = 0; c < (int)K; ++c) {
          float w = sKt[j * KP + c];
          dk += sK[i * KP + c] * w;
          dq += sQ[i * KP + c] * w;
        }
        float ratio = GATED ? expf(sG[i] - sG[j]) : 1.0f;
        if (j < i) av = sBeta[i] * ratio * dk;
        mv = ratio * dq;
      }
      sA[i * CP + j] = av;
      sM[i * CP + j] = mv;
    }
    for (int e = tid; e < C * VT; e += GEN_THREADS) {
      int i = e / VT, r = e % VT;
      float ks = 0.0f, qs = 0.0f;
      for (int c = 0; c < (int)K; ++c) {
        float s = sS[r * KP + c];
        ks += sK[i * KP + c] * s;
        qs += sQ[i * KP + c] * s;
      }
      float gi = GATED ? expf(sG[i]) : 1.0f;
      sR[i * VT + r] = sBeta[i] * (sV[i * VT + r] - gi * ks);
      sP[i * VT + r] = gi * qs;
    }
    __syncthreads();
    // ---- (I + A) Delta = B R, one value column per thread
    for (int r = tid; r < VT; r += GEN_THREADS) {
      for (int i = 0; i < L; ++i) {
        float x = sR[i * VT + r];
        for (int j = 0; j < i; ++j) x -= sA[i * CP + j] * sR[j * VT + r];
        sR[i * VT + r] = x;
      }
    }
    __syncthreads();
    // ---- outputs and state update
    for (int e = tid; e < C * VT; e += GEN_THREADS) {
      int i = e / VT, r = e % VT;
      if (i < L && r < vn) {
        float acc = sP[i * VT + r];
        for (int j = 0; j <= i; ++j) acc += sM[i * CP + j] * sR[j * VT + r];
        store_out<TIn>(a.o, ((tb + t0 + i) * H + h) * V + v0 + r, acc, a.o_f32);
      }
    }
    const float gL = GATED ? sG[L - 1] : 0.0f;
    const float decay = GATED ? expf(gL) : 1.0f;
    for (int e = tid; e < VT * K; e += GEN_THREADS) {
      int r = e / (int)K, c = e % (int)K;
      float acc = decay * sS[r * KP + c];
      for (int j = 0; j < L; ++j) {
        float w = GATED ? expf(gL - sG[j]) : 1.0f;
        acc += w * sR[j * VT + r] * sKt[j * KP + c];
      }
      sS[r * KP + c] = acc;
    }
  }
  __syncthreads();
  if (a.S_out) {
    for (int e = tid; e < VT * K; e += GEN_THREADS) {
      int r = e / (int)K, c = e % (int)K;
      if (r < vn) a.S_out[(seq * V + v0 + r) * K + c] = sS[r * KP + c];
    }
  }
}

static GenLayout gen_layout(const ChunkArgs &a) {
  GenLayout lay;
  lay.C = a.C;
  lay.K = (int)a.K;
  lay.VT = (int)(a.V < 16 ? a.V : 16);
  lay.KP = (int)a.K + 1;
  return lay;
}

template <typename TIn, bool VL>
static hipError_t launch_gen(const ChunkArgs &a, hipStream_t s) {
  GenLayout lay = gen_layout(a);
  int ntiles = (int)((a.V + lay.VT - 1) / lay.VT);
  size_t shm = (size_t)lay.total() * sizeof(float);
  dim3 grid((unsigned)(a.B * a.H * ntiles)), block(GEN_THREADS);
  if (a.alpha) {
    auto kern = chunk_generic_kernel<TIn, true, VL>;
    hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    hipLaunchKernelGGL(kern, grid, block, shm, s, a, lay, ntiles);
  } else {
    auto kern = chunk_generic_kernel<TIn, false, VL>;
    hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    hipLaunchKernelGGL(kern, grid, block, shm, s, a, lay, ntiles);
  }
  prof_mark(s, "chunk_generic_kernel");
  return hipGetLastError();
}

size_t chunk_generic_lds_bytes(const ChunkArgs &a) { return (size_t)gen_layout(a).total() * sizeof(float); }

hipError_t launch_chunk_generic(const ChunkArgs &a, bool is_bf16, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  if (a.cu) return is_bf16 ? launch_gen<bf16, true>(a, s) : launch_gen<float, true>(a, s);
  return is_bf16 ? launch_gen<bf16, false>(a, s) : launch_gen<float, false>(a, s);
}

}  // namespace osdn
