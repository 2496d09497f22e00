// Internal launch interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace osdn {

// Sequences of a batch.  With cu == null, sequence b is tokens [b T, b T + T)
// of [B,T,H,.] tensors; with cu (device int64 [B+1], variable lengths), it is
// tokens [cu[b], cu[b+1]) of packed [1, cu[B], H, .] tensors and T is the
// longest length (it sizes per-chunk workspace rows).  Kernels take VL (cu
// present) as a template flag, so uniform batches compile as before.
template <bool VL, class A>
__device__ __forceinline__ int64_t seq_base(const A &a, int64_t b) {
  if constexpr (VL) return a.cu[b];
  else return b * a.T;
}
template <bool VL, class A>
__device__ __forceinline__ int64_t seq_len(const A &a, int64_t b) {
  if constexpr (VL) return a.cu[b + 1] - a.cu[b];
  else return a.T;
}

struct ScanArgs {
  const void *k;        // [B,T,H,K]
  const float *beta;    // [B,T,H]
  const float *r;       // [B,T,H], [B,T,H,K] when r_per_key, or null
  const float *d1;      // [B,H,K] or null
  void *k_tilde;        // [B,T,H,K] or null: write keys d (.) k
  void *kt_res;         // [B,T,H,K] bf16 or null: write-key residual (d - 1) (.) k
  float *d_out;         // [B,H,K] or null
  int64_t B, T, H, K;
  float eta, d_min, d_max, eps;
  int clamp, beta_aware;
  const int64_t *cu = nullptr;  // variable-length sequences (see seq_base)
  int r_per_key = 0;            // vector retention: token-by-token kernel only
};

struct ChunkArgs {
  const void *q, *k, *kt, *v;  // [B,T,H,K] / [B,T,H,V]
  bool kt_is_res;              // kt holds the residual (d - 1) (.) k, so k~ = k + kt
  const float *beta;           // [B,T,H]
  const float *alpha;          // [B,T,H] or null
  const float *S0;             // [B,H,V,K] or null
  void *o;                     // [B,T,H,V], float32 when o_f32
  float *S_out;                // [B,H,V,K] or null
  int64_t B, T, H, K, V;
  int C;
  float q_scale;
  int o_f32 = 0;               // o is float32 whatever the input type
  const int64_t *cu = nullptr;  // variable-length sequences (see seq_base)
  // residual form only: the chunked phase 1's marks ([B,H,N] per 64-token
  // chunk, 2 = every write key of the chunk is d_min k), or null
  const int *pin = nullptr;
  float d_min = 0.0f;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_precond_scan(const ScanArgs &a, bool bf16, hipStream_t s);

// Chunked phase 1 (prep / solve / emit kernels).  Workspace: per-token key
// norm and step scalar c (fp32 [B,T,H] each), d at every 64-token chunk start
// (fp32 [B,H,N,K]), one word per chunk (int [B,H,N]: 1 when the chunk keeps
// a d that sits on d_min there, rewritten to 2 when the sweep took it so, in
// which case its d start is not stored), the same per token (uint64 [B,H,N],
// bit u for token u of the chunk), and three counters per (b,h) (int
// [B,H,3]: chunks taken on the pinned, closed-form and token-by-token paths).
struct ScanWork {
  float *norm, *cstep, *dstart;
  int *pin;
  uint64_t *stay;  // [B,H,N]: bit u set when token u of the chunk keeps a d on d_min there
  int *flags;
  int *fok;     // [B,H,N]: 1 when ainv holds the chunk's factor (see precond_chunked.hip)
  float *ainv;  // [B,H,N][64*64]: strictly lower part of the chunk's inverse triangular factor
};
constexpr int SCAN_CHUNK = 64;
size_t scan_work_bytes(int64_t B, int64_t T, int64_t H, int64_t K);
ScanWork scan_work_layout(void *base, int64_t B, int64_t T, int64_t H, int64_t K);
// emit = false leaves the write keys to the caller (see EmitArgs).
hipError_t launch_precond_scan_chunked(const ScanArgs &a, const ScanWork &w, bool bf16, hipStream_t s,
                                       bool emit = true);

// The phase-1 replay of one chunk (d from the chunk start through the step
// scalars, writing the residual (d - 1) (.) k), folded into the first
// phase-2 kernel when the residual is needed only by phase 2.
struct EmitArgs {
  const float *cstep;   // [B,T,H] step scalars from the chunked sweep
  const float *dstart;  // [B,H,N,K] d at each chunk start
  const int *pin;       // [B,H,N]; 2 = the chunk starts from d_min (no stored start)
  const float *r;       // [B,T,H] retention ([B,T,H,K] when r_vec), or null
  bf16 *res;            // OUT [B,T,H,K] residual, read back by the sweep kernel
  float d_min, d_max;
  int clamp;
  int r_vec = 0;        // r is [B,T,H,K] (the chunk_wy replay only)
};
hipError_t launch_chunk_generic(const ChunkArgs &a, bool bf16, hipStream_t s);
hipError_t launch_chunk_mfma(const ChunkArgs &a, hipStream_t s);
// Two-kernel MFMA path (same shapes as launch_chunk_mfma): the per-chunk
// (I + A)^-1 of every chunk goes through a bf16 workspace [B,H,N,64,64].
size_t chunk_wy_work_bytes(int64_t B, int64_t T, int64_t H);
hipError_t launch_chunk_wy(const ChunkArgs &a, void *work, hipStream_t s, const EmitArgs *emit = nullptr);

// Decode step: up to 64 tokens per (b,h) through the recurrent form from a
// carried (d, S), one workgroup per (b,h) (K, V <= 128).
struct DecodeArgs {
  const void *q, *k, *v;      // [B,T,H,K] / [B,T,H,V]
  const float *beta;          // [B,T,H]
  const float *r, *alpha;     // [B,T,H] or null
  const float *d1, *S0;       // [B,H,K], [B,H,V,K] or null (ones, zeros)
  void *o;                    // [B,T,H,V], float32 when o_f32
  float *d_out, *S_out;       // or null; may alias d1, S0
  int o_f32 = 0;
  int64_t B, T, H, K, V;
  float eta, d_min, d_max, eps, q_scale;
  int clamp, beta_aware;
  int tb;                     // tokens staged per block (set by the launcher)
};
hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t s);

// Backward pass (three kernels, one workgroup or wave per (b,h); K, V <= 128).
struct BwdArgs {
  const void *q, *k, *v;        // [B,T,H,K] / [B,T,H,V]
  const float *beta;            // [B,T,H]
  const float *r, *alpha;       // [B,T,H] or null
  const float *d1, *S0;         // [B,H,K], [B,H,V,K] or null (ones, zeros)
  const void *dout;             // [B,T,H,V] dL/do
  const float *dS, *dd;         // [B,H,V,K] dL/dS_T, [B,H,K] dL/dd_{T+1}, or null
  void *dq, *dk, *dv;           // OUT [B,T,H,K] / [B,T,H,V]
  float *dbeta;                 // OUT [B,T,H]
  float *dr, *dalpha;           // OUT [B,T,H] or null
  float *dd1, *dS0;             // OUT [B,H,K], [B,H,V,K] or null
  // workspace regions (bwd_work_layout); NQ = ceil(V/32) value slices
  float *u;                     // [B,T,H,V] residual of every token
  float *ck;                    // [B,H,NB+1,V,K] S every 16 tokens (NB = ceil(T/16))
  float *dck;                   // [B,H,NB+1,K] d every 16 tokens
  float *dqp, *dktp, *dkrp;     // [NQ,B,T,H,K] per-slice parts of S^T dout, dL/dk~, read-key dL/dk
  float *dbp, *dap;             // [NQ,B,T,H] per-slice parts of dL/dbeta (phase 2) and dL/dalpha
  int nq;
  int64_t B, T, H, K, V;
  float eta, d_min, d_max, eps, q_scale;
  int clamp, beta_aware;
  int o_f32 = 0;                // dq, dk, dv are float32 whatever the input type
};
size_t bwd_work_bytes(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V);
void bwd_work_layout(BwdArgs &a, void *base);
hipError_t launch_bwd(const BwdArgs &a, bool bf16, hipStream_t s);

// OSKDA phase 2 (K x V state, channel-wise decay; K, V <= 128): a
// chunk-parallel kernel forms each 64-token chunk's operands, a sweep kernel
// carries the state (one workgroup per (b,h) and 32 value columns).
struct KdaArgs {
  const void *q, *k, *kt, *v;  // [B,T,H,K] / [B,T,H,V]
  bool kt_is_res;              // kt holds the bf16 residual (d - 1) (.) k, so k~ = k + kt
  const float *beta;           // [B,T,H]
  const float *alpha;          // [B,T,H,K] channel-wise decay, or null
  const float *S0;             // [B,H,K,V] or null
  void *o;                     // [B,T,H,V], float32 when o_f32
  float *S_out;                // [B,H,K,V] or null
  int64_t B, T, H, K, V;
  float q_scale;
  int o_f32 = 0;
  // workspace regions (kda_work_layout), per (b,h) and chunk n < N = ceil(T/64):
  float *kh, *qh;  // [B,H,N,64,128] Gamma . k and Gamma . q_scale q, rows permuted for MFMA
  float *kc;       // [B,H,N,128,64] ((gamma_C / Gamma) . k~)^T, rows permuted
  float *tb, *mq;  // [B,H,N,64,64] (I + A)^-1 diag(beta) and the intra-chunk scores
  float *gc;       // [B,H,N,128] gamma_C
};
size_t kda_work_bytes(int64_t B, int64_t T, int64_t H);
void kda_work_layout(KdaArgs &a, void *base);
// em (bf16, K = 128, residual form): the intra pass forms the write-key
// residual itself from the phase-1 sweep's marks and step scalars (run that
// sweep with emit = false); kt is then not read.
bool kda_can_fold(const KdaArgs &a, bool bf16);
hipError_t launch_kda(const KdaArgs &a, bool bf16, hipStream_t s, const EmitArgs *em = nullptr);

// Shape coverage of the specialised MFMA path (bf16, K = V = 128, C = 64).
bool chunk_mfma_supported(const ChunkArgs &a, bool bf16);

}  // namespace osdn
