/*
 * osdn.h -- C ABI of the OSDN (Online Scaled DeltaNet) forward hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the two-phase forward of "OSDN: Improving Delta Rule with
 * Provable Online Preconditioning in Linear Attention" (Zhou et al.,
 * arXiv:2605.13473):
 *
 *   phase 1 (osdn_precond_scan) -- the online preconditioner sweep of
 *     Section 4.2, Eq.(4) and Algorithm 1, with the retention-gated (APF) form
 *     of Section 4.4, Eq.(7), and the non-beta-aware form of Appendix B.  Per
 *     (b,h), starting from d = d1 (ones when NULL; d1 is not clamped):
 *         k~_t = d (.) k_t                    (emitted before the update)
 *         s = k_t (.) k_t,  n = max(sum s, eps),  b' = beta_t (or 1)
 *         d = clip(r_t d + eta b' (1 - b' <d, s>) / n * s, d_min, d_max)
 *
 *   phase 2 (osdn_chunk_fwd) -- the delta rule with the preconditioned write
 *     key, Section 4.3 Eq.(5), evaluated chunkwise with the WY form of
 *     Appendix A.2, Eqs.(8)-(11); with a decay alpha it is the Gated DeltaNet
 *     variant of Appendix B.1, Eqs.(13)-(15) (post-gate residual).  Per (b,h),
 *     from S = S0 (zeros when NULL), S in R^{V x K}:
 *         Sb = alpha_t S  (Sb = S without alpha)
 *         S  = Sb + beta_t (v_t - Sb k_t) k~_t^T
 *         o_t = S (q_scale q_t)
 *
 *   osdn_fwd runs both phases on one stream.
 *
 * Conventions for every entry point:
 *  - Sequence tensors are contiguous row-major [B,T,H,X] (the paper's layout
 *    before chunking, Appendix C); per-head vectors [B,H,X]; the state S is
 *    [B,H,V,K] in float32.  q, k, v, k_tilde and o share desc->dtype (o is
 *    float32 instead when desc->o_f32 is set); beta, r, alpha, d1, d_out, S0
 *    and S_out are float32.
 *  - Pointers are DEVICE pointers owned by the caller; the library allocates
 *    no memory and keeps no state between calls beyond the calling thread's
 *    last error message, its open launch profile (osdn_profile_begin /
 *    osdn_profile_end, whose HIP events live from the first launch recorded
 *    to osdn_profile_end), and, for osdn_fwd_noalloc only, its scratch array
 *    (a device array of the library, one copy per GPU) with that copy's
 *    address, looked up once per device.  stream is a hipStream_t (NULL
 *    = the default stream); work is enqueued asynchronously and outputs are
 *    valid once the stream has been synchronised.
 *  - Arguments are validated before anything is launched; on failure nothing
 *    is written and a status other than OSDN_OK is returned
 *    (osdn_last_error() then holds a message for the calling thread).  A HIP
 *    launch failure returns OSDN_EHIP.
 *  - d_out may alias d1 and S_out may alias S0 (in-place state update); no
 *    other aliasing between inputs and outputs is allowed.
 *  - Device pointers must be aligned to 16 bytes.  Device data is not checked:
 *    alpha must lie in (0, 1] and all inputs must be finite.
 */
#ifndef OSDN_H
#define OSDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { OSDN_F32 = 0, OSDN_BF16 = 1 } osdn_dtype;

typedef enum {
  OSDN_OK = 0,
  OSDN_EINVAL = 1,       /* malformed argument (sizes, NULL, alignment, box)  */
  OSDN_EUNSUPPORTED = 2, /* well formed but outside what the kernels cover   */
  OSDN_EHIP = 3          /* the HIP runtime reported an error                */
} osdn_status;

/*
 * Problem description.  Arguments follow the paper's statement of the
 * problem (Algorithm 1's inputs; the chunk interface of Appendix C).
 *   B, T, H     batch, tokens, heads; B, H >= 1, T >= 0; H <= 65536 for
 *               phase 2 (OSDN_EUNSUPPORTED above it).
 *   K, V        key / value head dims; 1 <= K <= 256 for phase 1,
 *               1 <= K, V <= 128 for phase 2.
 *   chunk       chunk length C of the WY form, 1 <= C <= 64.  The result does
 *               not depend on C beyond rounding (chunkwise equals sequential).
 *   dtype       osdn_dtype of q, k, v, k_tilde, o.
 *   eta         phase-1 step size (>= 0).
 *   d_min,d_max box of the projection; 0 < d_min <= d_max when clamp != 0.
 *   clamp       1: project onto [d_min, d_max] after every step; 0: no box.
 *   eps         floor of the squared key norm (> 0).
 *   q_scale     scale applied to q in the readout (1 = o_t = S_t q_t of the
 *               main text; K^-1/2 = the scaling used by the paper's listing).
 *   beta_aware  1: beta-aware feedback (Eq.(4)); 0: beta' = 1 in phase 1
 *               only (Appendix B); the memory write always uses beta.
 *   r_per_key   0: r is [B,T,H], one retention per token and head (Eq.(7));
 *               1: r is [B,T,H,K], the vector retention diag(r_t) of
 *               Appendix A.5, Proposition A.3 (osdn_precond_scan sweeps it
 *               chunked for K <= 128, token by token above; the forward
 *               entry points take K <= 128; osdn_decode and osdn_bwd return
 *               OSDN_EUNSUPPORTED for it).  Ignored when r is NULL.
 *   o_f32       0: the readout o has desc->dtype (rounded to nearest even
 *               from the fp32 accumulation, as the paper's listing returns
 *               o in the value dtype); 1: o is float32 whatever dtype is,
 *               i.e. the same readout before that final rounding (bf16
 *               inputs with fp32 outputs).  Taken by osdn_chunk_fwd,
 *               osdn_fwd, osdn_fwd_varlen, osdn_decode and osdn_kda_fwd;
 *               for osdn_bwd it makes dq, dk and dv float32 likewise.
 */
typedef struct osdn_desc {
  int64_t B, T, H, K, V;
  int32_t chunk;
  int32_t dtype;
  float eta, d_min, d_max;
  int32_t clamp;
  float eps;
  float q_scale;
  int32_t beta_aware;
  int32_t r_per_key;
  int32_t o_f32;
} osdn_desc;

/* Fill *desc with the given sizes and the paper's defaults: chunk 64,
 * eta 0.003, box [0.5, 2], clamp on, eps 1e-6, q_scale 1, beta-aware, bf16,
 * one retention per token and head, o in the input dtype. */
osdn_status osdn_desc_init(osdn_desc *desc, int64_t B, int64_t T, int64_t H,
                           int64_t K, int64_t V);

/* Host-only validation of a descriptor (no device work). */
osdn_status osdn_validate(const osdn_desc *desc);

/*
 * Phase 1, Algorithm 1 / Eq.(7) (Section 4.2, Section 4.4, Appendix B).
 *   k       [B,T,H,K] dtype    keys (read)
 *   beta    [B,T,H]   f32      write gates (read)
 *   r       [B,T,H]   f32      APF retention r_{t,h} ([B,T,H,K] when
 *                              desc->r_per_key), or NULL for r = 1
 *   d1      [B,H,K]   f32      initial preconditioner, or NULL for ones
 *   k_tilde [B,T,H,K] dtype    OUT: write keys d_t (.) k_t (rounded to dtype)
 *   d_out   [B,H,K]   f32      OUT: d_{T+1}, or NULL (may alias d1)
 *   workspace                  NULL: one kernel sweeps each (b,h) token by
 *                              token.  Otherwise >= osdn_precond_scan_
 *                              workspace_bytes(desc) bytes (16-byte aligned)
 *                              and the sweep runs chunked: a parallel pass for
 *                              the key norms, a parallel pass that factors
 *                              each chunk's closed form (the inverse of its
 *                              64 x 64 unit triangular system), a per-(b,h)
 *                              pass that finds the step scalar of every token
 *                              (64-token chunks whose coordinates all sit on
 *                              d_min, or all stay inside the box, are solved
 *                              in closed form; any other chunk token by
 *                              token), and a parallel pass that replays d and
 *                              writes the write keys.  Both give the same
 *                              result up to fp32 rounding.
 */
osdn_status osdn_precond_scan(const osdn_desc *desc, const void *k,
                              const float *beta, const float *r,
                              const float *d1, void *k_tilde, float *d_out,
                              void *workspace, size_t workspace_bytes,
                              void *stream);

/* Bytes of workspace for the chunked phase 1; 0 on an invalid descriptor. */
size_t osdn_precond_scan_workspace_bytes(const osdn_desc *desc);

/* Byte offset, inside a chunked phase-1 workspace, of B*H*3 int32 counters
 * left by the last sweep: per (b,h), the 64-token chunks solved with every
 * coordinate on d_min, solved with every coordinate inside the box, and swept
 * token by token.  (Diagnostics; -1 on an invalid descriptor.) */
int64_t osdn_precond_scan_counters_offset(const osdn_desc *desc);

/*
 * Phase 2, chunkwise WY delta rule with the write-key substitution of Eq.(6)
 * (Appendix A.2 Eqs.(8)-(11); Appendix B.1 Eqs.(13)-(15) when alpha != NULL).
 *   q, k, k_tilde [B,T,H,K] dtype   queries, physical keys, write keys
 *   v       [B,T,H,V] dtype          values
 *   beta    [B,T,H]   f32            write gates
 *   alpha   [B,T,H]   f32            state decay in (0,1], or NULL (OSDN)
 *   S0      [B,H,V,K] f32            initial state, or NULL for zeros
 *   o       [B,T,H,V] dtype          OUT: o_t = S_t (q_scale q_t) (f32 when
 *                                    desc->o_f32)
 *   S_out   [B,H,V,K] f32            OUT: S_T, or NULL (may alias S0)
 *   workspace                        NULL, or >= osdn_chunk_fwd_workspace_bytes
 *                                    (desc) bytes, 16-byte aligned (see below)
 */
osdn_status osdn_chunk_fwd(const osdn_desc *desc, const void *q,
                           const void *k, const void *k_tilde, const void *v,
                           const float *beta, const float *alpha,
                           const float *S0, void *o, float *S_out,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/* Bytes of the optional phase-2 workspace: nonzero only for the matrix-core
 * shapes (bf16, K = V = 128, chunk 64), where a workspace lets the (I + A)^-1
 * of every chunk be formed chunk-parallel before the sweep over chunks (a
 * bf16 64 x 64 block per chunk); without one a single kernel forms it inside
 * the sweep.  Same result up to fp32 rounding.  0 on an invalid descriptor. */
size_t osdn_chunk_fwd_workspace_bytes(const osdn_desc *desc);

/* Bytes of device workspace osdn_fwd needs (the write keys between the
 * phases, B*T*H*K elements of dtype, followed by a chunked phase-1 workspace
 * and a phase-2 workspace); 0 on an invalid descriptor. */
size_t osdn_fwd_workspace_bytes(const osdn_desc *desc);

/*
 * Both phases on one stream (the two-phase schedule of Section 4.5).
 * Arguments as above.  k_tilde_out [B,T,H,K] dtype, when not NULL, receives
 * the write keys d_t (.) k_t.  workspace (>= osdn_fwd_workspace_bytes(desc)
 * bytes, 16-byte aligned, required when T > 0) carries the write keys from
 * phase 1 to phase 2 and holds the chunked phase-1 scratch (its counters at
 * osdn_fwd_workspace_bytes(desc) - osdn_chunk_fwd_workspace_bytes(desc) -
 * osdn_precond_scan_workspace_bytes(desc) +
 * osdn_precond_scan_counters_offset(desc)) and the phase-2 scratch.  For bf16
 * the workspace holds the
 * residual (d_t - 1) (.) k_t rather
 * than k~_t, so phase 2 sees the write keys to about 16 significant bits
 * instead of bf16's 8: the result is then closer to the exact forward than
 * osdn_precond_scan followed by osdn_chunk_fwd on a bf16 k~.  That holds while
 * the box keeps d >= 1/2 (clamp on and d_min >= 1/2); otherwise d may approach
 * 0, where the residual would cancel, and the workspace holds k~_t in bf16.
 */
osdn_status osdn_fwd(const osdn_desc *desc, const void *q, const void *k,
                     const void *v, const float *beta, const float *r,
                     const float *alpha, const float *d1, const float *S0,
                     void *o, float *S_out, float *d_out, void *k_tilde_out,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * osdn_fwd over variable-length sequences packed into one token axis (the
 * packed training batches of Appendix F): sequence b is tokens
 * [cu_seqlens[b], cu_seqlens[b+1]) of the packed tensors and starts from its
 * own d1[b], S0[b] (the state is reset between sequences; nothing crosses a
 * sequence boundary).
 *   desc->B      number of sequences; desc->T  the longest sequence's length
 *                (bounds every cu_seqlens[b+1] - cu_seqlens[b]; sizes the
 *                workspace, which is osdn_fwd_workspace_bytes(desc))
 *   cu_seqlens   [B+1] int64 DEVICE pointer, 0 = c_0 <= c_1 <= ... = total
 *   q, k, k_tilde_out [1,total,H,K], v, o [1,total,H,V] dtype;
 *   beta, r, alpha [1,total,H] f32; d1, d_out [B,H,K], S0, S_out [B,H,V,K] f32.
 * Every other argument and rule is as for osdn_fwd.  cu_seqlens is device
 * data and is not checked: it must be non-decreasing from 0 with no
 * difference above desc->T.  Each sequence's result equals osdn_fwd on that
 * sequence alone, bit for bit.
 */
osdn_status osdn_fwd_varlen(const osdn_desc *desc, const int64_t *cu_seqlens,
                            const void *q, const void *k, const void *v,
                            const float *beta, const float *r,
                            const float *alpha, const float *d1,
                            const float *S0, void *o, float *S_out,
                            float *d_out, void *k_tilde_out, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * osdn_fwd without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Arguments and results are those of osdn_fwd; the
 * workspace is a scratch array of OSDN_FWD_NOALLOC_MAX_WORKSPACE bytes that
 * the library holds on every GPU it runs on, from first use until the process
 * ends.  Problems whose osdn_fwd_workspace_bytes(desc) exceeds it return
 * OSDN_EUNSUPPORTED before anything is launched.  Nothing here allocates:
 * the first call on a device looks up that device's copy of the array.  All
 * calls on one GPU share its array: calls that overlap in time on one GPU
 * (different streams or threads) race and must not be issued; consecutive
 * calls on one stream are safe (no word of the scratch is read before the
 * same call writes it).
 */
#define OSDN_FWD_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
osdn_status osdn_fwd_noalloc(const osdn_desc *desc, const void *q,
                             const void *k, const void *v, const float *beta,
                             const float *r, const float *alpha,
                             const float *d1, const float *S0, void *o,
                             float *S_out, float *d_out, void *k_tilde_out,
                             void *stream);

/*
 * Decode step: the single-token recurrence of Appendix L (one launch per
 * call), for up to OSDN_DECODE_MAX_T new tokens per (b,h) continuing from a
 * carried state.  Per (b,h) and token, in order: the write key d (.) k_t, the
 * phase-1 update of d (as in osdn_precond_scan), then the phase-2 write and
 * readout (as in osdn_chunk_fwd, token by token).  The result is that of
 * osdn_fwd on the same tokens from the same (d1, S0) up to fp32 rounding; the
 * write keys stay in fp32 here (they are never rounded to dtype).
 *   q, k    [B,T,H,K] dtype      queries, keys
 *   v       [B,T,H,V] dtype      values
 *   beta    [B,T,H]   f32        write gates
 *   r       [B,T,H]   f32        APF retention, or NULL for r = 1
 *   alpha   [B,T,H]   f32        state decay in (0,1], or NULL (OSDN)
 *   d1      [B,H,K]   f32        carried preconditioner, or NULL for ones
 *   S0      [B,H,V,K] f32        carried state, or NULL for zeros
 *   o       [B,T,H,V] dtype      OUT: readouts (f32 when desc->o_f32)
 *   S_out   [B,H,V,K] f32        OUT: state after the last token, or NULL
 *                                (may alias S0: in-place update)
 *   d_out   [B,H,K]   f32        OUT: d after the last token, or NULL (may
 *                                alias d1)
 * The descriptor is validated as for osdn_fwd (desc->chunk is not used);
 * T > OSDN_DECODE_MAX_T or B*H >= 2^31 returns OSDN_EUNSUPPORTED.  T = 0
 * copies d1 to d_out and S0 to S_out.  No workspace.
 */
#define OSDN_DECODE_MAX_T 64
osdn_status osdn_decode(const osdn_desc *desc, const void *q, const void *k,
                        const void *v, const float *beta, const float *r,
                        const float *alpha, const float *d1, const float *S0,
                        void *o, float *S_out, float *d_out, void *stream);

/*
 * Backward pass: gradients of a loss L through osdn_fwd, given dL/do and
 * optionally dL/dS_T and dL/dd_{T+1}.  Phase 2 is differentiated token by
 * token backwards (the adjoint G of the state: G += q_scale dout_t q_t^T,
 * w = G k~_t, dv_t = beta_t w, dk~_t = beta_t G^T u_t, read-key part
 * -beta_t Sb_t^T w, G = alpha_t (G - beta_t w k_t^T)); phase 1 is swept back
 * through the clamped recurrence, the gradient reaching d through
 * k~ = d (.) k as Section 4.5 describes (the clamp passes the gradient only
 * where it did not clip; the norm floor blocks the norm's derivative).
 *   q, k, v, beta, r, alpha, d1, S0   the forward's inputs, as for osdn_fwd
 *   dout    [B,T,H,V] dtype      dL/do
 *   dS      [B,H,V,K] f32        dL/dS_T, or NULL (zero)
 *   dd      [B,H,K]   f32        dL/dd_{T+1}, or NULL (zero)
 *   dq, dk  [B,T,H,K] dtype      OUT: dL/dq, dL/dk (both key roles) (f32
 *                                when desc->o_f32)
 *   dv      [B,T,H,V] dtype      OUT: dL/dv (f32 when desc->o_f32)
 *   dbeta   [B,T,H]   f32        OUT: dL/dbeta (write gate and phase-1 step)
 *   dr      [B,T,H]   f32        OUT: dL/dr, or NULL (ignored when r is NULL)
 *   dalpha  [B,T,H]   f32        OUT: dL/dalpha, or NULL (ignored when alpha is NULL)
 *   dd1     [B,H,K]   f32        OUT: dL/dd1, or NULL
 *   dS0     [B,H,V,K] f32        OUT: dL/dS0, or NULL
 *   workspace  >= osdn_bwd_workspace_bytes(desc) bytes, 16-byte aligned,
 *              required: the forward is run once more to record every
 *              token's residual (fp32 [B,T,H,V]) and the state and d every
 *              16 tokens, plus fp32 dL/dk~ and partial gradients.
 * Gradient outputs must not alias inputs or each other.  K, V <= 128;
 * B*H >= 2^31 returns OSDN_EUNSUPPORTED.  T = 0 gives dS0 = dS, dd1 = dd.
 */
size_t osdn_bwd_workspace_bytes(const osdn_desc *desc);
osdn_status osdn_bwd(const osdn_desc *desc, const void *q, const void *k,
                     const void *v, const float *beta, const float *r,
                     const float *alpha, const float *d1, const float *S0,
                     const void *dout, const float *dS, const float *dd,
                     void *dq, void *dk, void *dv, float *dbeta, float *dr,
                     float *dalpha, float *dd1, float *dS0, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * OSKDA forward: online scaling on the Kimi Delta Attention backbone
 * (Appendix B.2 and the online-scaled KDA row of Table 3).  Phase 1 is the
 * preconditioner sweep of osdn_precond_scan (Eq.(12): beta-aware or not,
 * optional retention r, clamp to the box); phase 2 keeps KDA's own K x V
 * state and gates it per key channel.  Per (b,h), from S = S0 (zeros when
 * NULL), S in R^{K x V}, for each token:
 *     Sb  = Diag(alpha_t) S            (Sb = S when alpha is NULL)
 *     u_t = v_t - Sb^T k_t             (residual read with the physical key)
 *     S   = Sb + beta_t k~_t u_t^T     (preconditioned key on the storage side)
 *     o_t = S^T (q_scale q_t)
 * evaluated in 64-token chunks with the UT-transform form of Appendix B.2
 * (desc->chunk is not used).
 *   q, k    [B,T,H,K] dtype     queries, keys
 *   v       [B,T,H,V] dtype     values
 *   beta    [B,T,H]   f32       write gates
 *   r       [B,T,H] (or [B,T,H,K] with desc->r_per_key) f32, or NULL
 *   alpha   [B,T,H,K] f32       channel-wise decay in (0,1], or NULL (none)
 *   d1      [B,H,K]   f32       initial preconditioner, or NULL for ones
 *   S0      [B,H,K,V] f32       initial state (KDA layout), or NULL for zeros
 *   o       [B,T,H,V] dtype     OUT: readouts (f32 when desc->o_f32)
 *   S_out   [B,H,K,V] f32       OUT: final state, or NULL (may alias S0)
 *   d_out   [B,H,K]   f32       OUT: d_{T+1}, or NULL (may alias d1)
 *   k_tilde_out [B,T,H,K] dtype OUT: write keys d_t (.) k_t, or NULL
 *   workspace  >= osdn_kda_fwd_workspace_bytes(desc) bytes, 16-byte aligned,
 *              required when T > 0: the write keys (for bf16 as the residual
 *              (d_t - 1) (.) k_t, as in osdn_fwd), the phase-1 scratch and
 *              about 128 KiB of fp32 chunk operands per (b,h) and 64 tokens.
 * K, V <= 128 (OSDN_EUNSUPPORTED above).  Arithmetic is fp32 throughout;
 * a channel whose decay over one chunk falls below e^-60 takes exact
 * per-entry exponentials instead of the factorised products.
 */
size_t osdn_kda_fwd_workspace_bytes(const osdn_desc *desc);
osdn_status osdn_kda_fwd(const osdn_desc *desc, const void *q, const void *k,
                         const void *v, const float *beta, const float *r,
                         const float *alpha, const float *d1, const float *S0,
                         void *o, float *S_out, float *d_out, void *k_tilde_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Launch profile (measurement aid).  osdn_profile_begin records a HIP event on
 * `stream`; until osdn_profile_end, every kernel the library launches from
 * the calling thread records another event on its stream right after the
 * launch (at most 1024 launches are recorded).  osdn_profile_end waits for the
 * last event and writes, for up to max_entries launches in order, the kernel
 * name (static string) and the device time in milliseconds from the previous
 * event to this launch's event -- the kernel's duration when the launches are
 * queued back to back on one stream.  *count receives the number of launches
 * recorded.  Ending a profile that was not begun returns OSDN_EINVAL.  The
 * events are created as launches are recorded and destroyed by
 * osdn_profile_end.
 */
osdn_status osdn_profile_begin(void *stream);
osdn_status osdn_profile_end(const char **names, float *ms, int max_entries,
                             int *count);

/* Name of a status code (static string). */
const char *osdn_status_str(int status);

/* Message describing the last failure on the calling thread ("" if none). */
const char *osdn_last_error(void);

/* Library version, (major << 16) | minor. */
int osdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OSDN_H */
