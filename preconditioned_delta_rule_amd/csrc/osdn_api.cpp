// C ABI of the OSDN forward hot path: argument validation and dispatch to the
// gfx950 kernels.  Declarations and the argument contract are in include/osdn.h.
#include "osdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.h"
#include "profile.h"

namespace {

thread_local std::string g_last_error;

// Workspace of osdn_fwd_noalloc: one copy of this array per GPU.  Host code
// never uses the name itself as a device address: the device address of each
// GPU's copy is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept in g_scratch.
__device__ __align__(256) unsigned char scratch[OSDN_FWD_NOALLOC_MAX_WORKSPACE];
constexpr int MAX_DEVICES = 64;
void *g_scratch[MAX_DEVICES] = {};
hipError_t g_scratch_err[MAX_DEVICES] = {};
std::once_flag g_scratch_once[MAX_DEVICES];

// Per-thread launch profile (osdn_profile_begin / osdn_profile_end).
constexpr int PROF_MAX = 1024;
struct Profile {
  bool open = false;
  int n = 0;
  hipEvent_t ev[PROF_MAX + 1] = {};  // created as needed, destroyed by osdn_profile_end
  const char *name[PROF_MAX] = {};
};
thread_local Profile g_prof;

osdn_status fail(osdn_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
osdn_status fail(osdn_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

osdn_status ok() {
  g_last_error.clear();
  return OSDN_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(int32_t dtype) { return dtype == OSDN_BF16 ? 2 : 4; }

osdn_status check_ptr(const void *p, const char *name, bool required) {
  if (!p) {
    if (required) return fail(OSDN_EINVAL, "%s must not be NULL", name);
    return OSDN_OK;
  }
  if (!aligned16(p)) return fail(OSDN_EINVAL, "%s is not 16-byte aligned", name);
  return OSDN_OK;
}

#define OSDN_TRY(expr)                 \
  do {                                 \
    osdn_status _st = (expr);          \
    if (_st != OSDN_OK) return _st;    \
  } while (0)

// Common descriptor checks; `phase` 1 = scan, 2 = chunk, 3 = both.
osdn_status validate(const osdn_desc *d, int phase) {
  if (!d) return fail(OSDN_EINVAL, "desc must not be NULL");
  if (d->B < 1 || d->H < 1 || d->T < 0)
    return fail(OSDN_EINVAL, "need B >= 1, H >= 1, T >= 0 (got B=%lld H=%lld T=%lld)",
                (long long)d->B, (long long)d->H, (long long)d->T);
  if (d->dtype != OSDN_F32 && d->dtype != OSDN_BF16)
    return fail(OSDN_EINVAL, "dtype must be OSDN_F32 or OSDN_BF16 (got %d)", d->dtype);
  if (d->K < 1) return fail(OSDN_EINVAL, "K must be >= 1 (got %lld)", (long long)d->K);
  if ((phase & 2) && d->V < 1) return fail(OSDN_EINVAL, "V must be >= 1 (got %lld)", (long long)d->V);
  // element counts must stay far from int64 overflow
  const double big = 4.0e18;
  if ((double)d->B * (double)d->T * (double)d->H * (double)(d->K > d->V ? d->K : d->V) > big ||
      (double)d->B * (double)d->H * (double)d->K * (double)d->V > big)
    return fail(OSDN_EINVAL, "problem size overflows 64-bit indexing");
  if (phase & 1) {
    if (!std::isfinite(d->eta) || d->eta < 0.0f) return fail(OSDN_EINVAL, "eta must be finite and >= 0");
    if (!std::isfinite(d->eps) || !(d->eps > 0.0f)) return fail(OSDN_EINVAL, "eps must be finite and > 0");
    if (d->clamp) {
      if (!std::isfinite(d->d_min) || !std::isfinite(d->d_max) || !(d->d_min > 0.0f) || d->d_min > d->d_max)
        return fail(OSDN_EINVAL, "box needs finite 0 < d_min <= d_max (got [%g, %g])", d->d_min, d->d_max);
    }
    if (d->K > 256) return fail(OSDN_EUNSUPPORTED, "phase 1 supports K <= 256 (got %lld)", (long long)d->K);
    if (d->r_per_key != 0 && d->r_per_key != 1)
      return fail(OSDN_EINVAL, "r_per_key must be 0 or 1 (got %d)", d->r_per_key);
  }
  if (phase & 2) {
    if (d->chunk < 1) return fail(OSDN_EINVAL, "chunk must be >= 1 (got %d)", d->chunk);
    if (d->chunk > 64) return fail(OSDN_EUNSUPPORTED, "chunk must be <= 64 (got %d)", d->chunk);
    // the sweep addresses 64 token rows with 32-bit byte offsets
    if (d->H > 65536) return fail(OSDN_EUNSUPPORTED, "phase 2 supports H <= 65536 (got %lld)", (long long)d->H);
    if (d->K > 128 || d->V > 128)
      return fail(OSDN_EUNSUPPORTED, "phase 2 supports K, V <= 128 (got K=%lld V=%lld)", (long long)d->K,
                  (long long)d->V);
    if (!std::isfinite(d->q_scale)) return fail(OSDN_EINVAL, "q_scale must be finite");
    if (d->o_f32 != 0 && d->o_f32 != 1) return fail(OSDN_EINVAL, "o_f32 must be 0 or 1 (got %d)", d->o_f32);
  }
  return OSDN_OK;
}

osdn_status hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(OSDN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return OSDN_OK;
}

osdn::ScanArgs scan_args(const osdn_desc *d, const void *k, const float *beta, const float *r,
                         const float *d1, void *k_tilde, float *d_out) {
  osdn::ScanArgs a;
  a.k = k;
  a.beta = beta;
  a.r = r;
  a.d1 = d1;
  a.k_tilde = k_tilde;
  a.kt_res = nullptr;
  a.d_out = d_out;
  a.B = d->B;
  a.T = d->T;
  a.H = d->H;
  a.K = d->K;
  a.eta = d->eta;
  a.d_min = d->d_min;
  a.d_max = d->d_max;
  a.eps = d->eps;
  a.clamp = d->clamp ? 1 : 0;
  a.beta_aware = d->beta_aware ? 1 : 0;
  a.r_per_key = d->r_per_key;
  return a;
}

osdn::ChunkArgs chunk_args(const osdn_desc *d, const void *q, const void *k, const void *kt, const void *v,
                           const float *beta, const float *alpha, const float *S0, void *o, float *S_out) {
  osdn::ChunkArgs a;
  a.q = q;
  a.k = k;
  a.kt = kt;
  a.kt_is_res = false;
  a.v = v;
  a.beta = beta;
  a.alpha = alpha;
  a.S0 = S0;
  a.o = o;
  a.S_out = S_out;
  a.B = d->B;
  a.T = d->T;
  a.H = d->H;
  a.K = d->K;
  a.V = d->V;
  a.C = d->chunk;
  a.q_scale = d->q_scale;
  a.o_f32 = d->o_f32;
  return a;
}

osdn_status run_scan(const osdn_desc *d, const osdn::ScanArgs &a, hipStream_t s) {
  return hip_status(osdn::launch_precond_scan(a, d->dtype == OSDN_BF16, s), "phase-1 launch");
}

// Phase-2 kernels: for bf16 with K = V = 128 and chunk 64 the matrix-core
// path (two kernels when a workspace is given, one otherwise), else the
// generic fp32-arithmetic kernel.
osdn_status run_chunk(const osdn_desc *d, const osdn::ChunkArgs &a, void *work, hipStream_t s) {
  const bool bf = d->dtype == OSDN_BF16;
  if (osdn::chunk_mfma_supported(a, bf)) {
    if (work) return hip_status(osdn::launch_chunk_wy(a, work, s), "phase-2 launch");
    return hip_status(osdn::launch_chunk_mfma(a, s), "phase-2 launch");
  }
  return hip_status(osdn::launch_chunk_generic(a, bf, s), "phase-2 launch");
}

size_t chunk_work_bytes(const osdn_desc *d) {
  osdn::ChunkArgs a;
  a.K = d->K;
  a.V = d->V;
  a.C = d->chunk;
  if (!osdn::chunk_mfma_supported(a, d->dtype == OSDN_BF16)) return 0;
  return (osdn::chunk_wy_work_bytes(d->B, d->T, d->H) + 255) & ~(size_t)255;
}

}  // namespace

namespace osdn {
void prof_mark(hipStream_t s, const char *kernel) {
  Profile &p = g_prof;
  if (!p.open || p.n >= PROF_MAX) return;
  if (!p.ev[p.n + 1] && hipEventCreate(&p.ev[p.n + 1]) != hipSuccess) return;
  if (hipEventRecord(p.ev[p.n + 1], s) != hipSuccess) return;
  p.name[p.n++] = kernel;
}
}  // namespace osdn

extern "C" {

osdn_status osdn_profile_begin(void *stream) {
  Profile &p = g_prof;
  if (!p.ev[0]) OSDN_TRY(hip_status(hipEventCreate(&p.ev[0]), "profile event"));
  OSDN_TRY(hip_status(hipEventRecord(p.ev[0], static_cast<hipStream_t>(stream)), "profile event"));
  p.open = true;
  p.n = 0;
  return ok();
}

osdn_status osdn_profile_end(const char **names, float *ms, int max_entries, int *count) {
  Profile &p = g_prof;
  if (!p.open) return fail(OSDN_EINVAL, "no profile is open on this thread");
  p.open = false;
  if (count) *count = p.n;
  osdn_status st = OSDN_OK;
  if (p.n > 0) st = hip_status(hipEventSynchronize(p.ev[p.n]), "profile event");
  for (int i = 0; st == OSDN_OK && i < p.n && i < max_entries; ++i) {
    float t = 0.0f;
    st = hip_status(hipEventElapsedTime(&t, p.ev[i], p.ev[i + 1]), "profile event");
    if (names) names[i] = p.name[i];
    if (ms) ms[i] = t;
  }
  // the events are not kept between profiles
  for (int i = 0; i <= PROF_MAX; ++i)
    if (p.ev[i]) {
      hipEventDestroy(p.ev[i]);
      p.ev[i] = nullptr;
    }
  return st == OSDN_OK ? ok() : st;
}

int osdn_version(void) { return (1 << 16) | 0; }

const char *osdn_status_str(int status) {
  switch (status) {
    case OSDN_OK: return "OSDN_OK";
    case OSDN_EINVAL: return "OSDN_EINVAL";
    case OSDN_EUNSUPPORTED: return "OSDN_EUNSUPPORTED";
    case OSDN_EHIP: return "OSDN_EHIP";
    default: return "OSDN_UNKNOWN_STATUS";
  }
}

const char *osdn_last_error(void) { return g_last_error.c_str(); }

osdn_status osdn_desc_init(osdn_desc *d, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V) {
  if (!d) return fail(OSDN_EINVAL, "desc must not be NULL");
  std::memset(d, 0, sizeof *d);
  d->B = B;
  d->T = T;
  d->H = H;
  d->K = K;
  d->V = V;
  d->chunk = 64;
  d->dtype = OSDN_BF16;
  d->eta = 0.003f;
  d->d_min = 0.5f;
  d->d_max = 2.0f;
  d->clamp = 1;
  d->eps = 1e-6f;
  d->q_scale = 1.0f;
  d->beta_aware = 1;
  return ok();
}

osdn_status osdn_validate(const osdn_desc *d) {
  OSDN_TRY(validate(d, 3));
  return ok();
}

size_t osdn_precond_scan_workspace_bytes(const osdn_desc *d) {
  if (validate(d, 1) != OSDN_OK) return 0;
  return osdn::scan_work_bytes(d->B, d->T, d->H, d->K);
}

int64_t osdn_precond_scan_counters_offset(const osdn_desc *d) {
  if (validate(d, 1) != OSDN_OK) return -1;
  osdn::ScanWork w = osdn::scan_work_layout(nullptr, d->B, d->T, d->H, d->K);
  return (int64_t)reinterpret_cast<uintptr_t>(w.flags);
}

osdn_status osdn_precond_scan(const osdn_desc *d, const void *k, const float *beta, const float *r,
                              const float *d1, void *k_tilde, float *d_out, void *workspace,
                              size_t workspace_bytes, void *stream) {
  OSDN_TRY(validate(d, 1));
  const bool need_seq = d->T > 0;
  OSDN_TRY(check_ptr(k, "k", need_seq));
  OSDN_TRY(check_ptr(beta, "beta", need_seq));
  OSDN_TRY(check_ptr(r, "r", false));
  OSDN_TRY(check_ptr(d1, "d1", false));
  OSDN_TRY(check_ptr(k_tilde, "k_tilde", need_seq));
  OSDN_TRY(check_ptr(d_out, "d_out", false));
  OSDN_TRY(check_ptr(workspace, "workspace", false));
  if (k_tilde && k_tilde == k) return fail(OSDN_EINVAL, "k_tilde must not alias k");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const osdn::ScanArgs sa = scan_args(d, k, beta, r, d1, k_tilde, d_out);
  // vector retention above K = 128 has only the token-by-token kernel
  if (!workspace || (d->r_per_key && r && d->K > 128)) {
    OSDN_TRY(run_scan(d, sa, s));
    return ok();
  }
  const size_t need = osdn::scan_work_bytes(d->B, d->T, d->H, d->K);
  if (workspace_bytes < need)
    return fail(OSDN_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  OSDN_TRY(hip_status(osdn::launch_precond_scan_chunked(
                          sa, osdn::scan_work_layout(workspace, d->B, d->T, d->H, d->K),
                          d->dtype == OSDN_BF16, s),
                      "phase-1 launch"));
  return ok();
}

size_t osdn_chunk_fwd_workspace_bytes(const osdn_desc *d) {
  if (validate(d, 2) != OSDN_OK) return 0;
  return chunk_work_bytes(d);
}

osdn_status osdn_chunk_fwd(const osdn_desc *d, const void *q, const void *k, const void *k_tilde, const void *v,
                           const float *beta, const float *alpha, const float *S0, void *o, float *S_out,
                           void *workspace, size_t workspace_bytes, void *stream) {
  OSDN_TRY(validate(d, 2));
  const bool need_seq = d->T > 0;
  OSDN_TRY(check_ptr(q, "q", need_seq));
  OSDN_TRY(check_ptr(k, "k", need_seq));
  OSDN_TRY(check_ptr(k_tilde, "k_tilde", need_seq));
  OSDN_TRY(check_ptr(v, "v", need_seq));
  OSDN_TRY(check_ptr(beta, "beta", need_seq));
  OSDN_TRY(check_ptr(alpha, "alpha", false));
  OSDN_TRY(check_ptr(S0, "S0", false));
  OSDN_TRY(check_ptr(o, "o", need_seq));
  OSDN_TRY(check_ptr(S_out, "S_out", false));
  if (o && (o == q || o == k || o == k_tilde || o == v)) return fail(OSDN_EINVAL, "o must not alias an input");
  OSDN_TRY(check_ptr(workspace, "workspace", false));
  const size_t need = chunk_work_bytes(d);
  if (workspace && workspace_bytes < need)
    return fail(OSDN_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  OSDN_TRY(run_chunk(d, chunk_args(d, q, k, k_tilde, v, beta, alpha, S0, o, S_out),
                     need ? workspace : nullptr, static_cast<hipStream_t>(stream)));
  return ok();
}

// bf16 write keys cross between the phases as the bf16 residual (d - 1) (.) k
// when the box keeps d >= 1/2: its relative error on k~ is 2^-9 |d - 1| / d,
// at most bf16's own.  Without that bound (no clamp, or d_min < 1/2) d can
// approach 0 and the residual would cancel, so k~ itself travels in bf16.
static bool keys_as_residual(const osdn_desc *d) {
  return d->dtype == OSDN_BF16 && d->clamp && d->d_min >= 0.5f;
}

static size_t fwd_keys_bytes(const osdn_desc *d) {
  const size_t n = (size_t)d->B * (size_t)d->T * (size_t)d->H * (size_t)d->K * elem_bytes(d->dtype);
  return (n + 255) & ~(size_t)255;
}

size_t osdn_fwd_workspace_bytes(const osdn_desc *d) {
  if (validate(d, 3) != OSDN_OK) return 0;
  return fwd_keys_bytes(d) + osdn::scan_work_bytes(d->B, d->T, d->H, d->K) + chunk_work_bytes(d);
}

static osdn_status fwd_impl(const osdn_desc *d, const int64_t *cu, const void *q, const void *k, const void *v,
                            const float *beta, const float *r, const float *alpha, const float *d1,
                            const float *S0, void *o, float *S_out, float *d_out, void *k_tilde_out,
                            void *workspace, size_t workspace_bytes, void *stream) {
  OSDN_TRY(validate(d, 3));
  const bool need_seq = d->T > 0;
  OSDN_TRY(check_ptr(q, "q", need_seq));
  OSDN_TRY(check_ptr(k, "k", need_seq));
  OSDN_TRY(check_ptr(v, "v", need_seq));
  OSDN_TRY(check_ptr(beta, "beta", need_seq));
  OSDN_TRY(check_ptr(r, "r", false));
  OSDN_TRY(check_ptr(alpha, "alpha", false));
  OSDN_TRY(check_ptr(d1, "d1", false));
  OSDN_TRY(check_ptr(S0, "S0", false));
  OSDN_TRY(check_ptr(o, "o", need_seq));
  OSDN_TRY(check_ptr(S_out, "S_out", false));
  OSDN_TRY(check_ptr(d_out, "d_out", false));
  OSDN_TRY(check_ptr(k_tilde_out, "k_tilde_out", false));
  // (phase 2 takes K <= 128, so vector retention always has the chunked phase 1 here)
  const bool rvec = d->r_per_key && r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  osdn::ScanArgs sa = scan_args(d, k, beta, r, d1, k_tilde_out, d_out);
  osdn::ChunkArgs ca = chunk_args(d, q, k, k_tilde_out, v, beta, alpha, S0, o, S_out);
  sa.cu = ca.cu = need_seq ? cu : nullptr;
  if (!need_seq) {
    // nothing to sweep: d_out = d1 and S_out = S0 (the kernels do the copy)
    OSDN_TRY(run_scan(d, sa, s));
    OSDN_TRY(run_chunk(d, ca, nullptr, s));
    return ok();
  }
  OSDN_TRY(check_ptr(workspace, "workspace", true));
  const size_t need = osdn_fwd_workspace_bytes(d);
  if (workspace_bytes < need)
    return fail(OSDN_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  char *ws = static_cast<char *>(workspace);
  const bool res = keys_as_residual(d);
  if (res) {
    // bf16: the write keys travel between the phases as the bf16 residual
    // (d - 1) (.) k, which with k gives k~ to ~16 bits
    sa.kt_res = ws;
    ca.kt = ws;
    ca.kt_is_res = true;
  } else if (!k_tilde_out) {
    sa.k_tilde = ws;
    ca.kt = ws;
  }
  const size_t scan_bytes = osdn::scan_work_bytes(d->B, d->T, d->H, d->K);
  const osdn::ScanWork sw = osdn::scan_work_layout(ws + fwd_keys_bytes(d), d->B, d->T, d->H, d->K);
  void *cw = chunk_work_bytes(d) ? ws + fwd_keys_bytes(d) + scan_bytes : nullptr;
  // bf16 on the matrix cores without k_tilde_out: the residual is formed by
  // the first phase-2 kernel, which replays d itself (one pass over k fewer)
  const bool fold = res && cw && !k_tilde_out;
  if (res) {
    // a chunk the chunked phase 1 marks as pinned keeps d = d_min at every
    // token: phase 2 takes its write keys as d_min k (exact operands)
    ca.pin = sw.pin;
    ca.d_min = d->d_min;
  }
  OSDN_TRY(hip_status(osdn::launch_precond_scan_chunked(sa, sw, d->dtype == OSDN_BF16, s, !fold),
                      "phase-1 launch"));
  if (fold) {
    osdn::EmitArgs em;
    em.cstep = sw.cstep;
    em.dstart = sw.dstart;
    em.pin = sw.pin;
    em.r = r;
    em.res = static_cast<osdn::bf16 *>(workspace);
    em.d_min = d->d_min;
    em.d_max = d->d_max;
    em.clamp = d->clamp ? 1 : 0;
    em.r_vec = rvec ? 1 : 0;
    OSDN_TRY(hip_status(osdn::launch_chunk_wy(ca, cw, s, &em), "phase-2 launch"));
  } else {
    OSDN_TRY(run_chunk(d, ca, cw, s));
  }
  return ok();
}

osdn_status osdn_fwd(const osdn_desc *d, const void *q, const void *k, const void *v, const float *beta,
                     const float *r, const float *alpha, const float *d1, const float *S0, void *o, float *S_out,
                     float *d_out, void *k_tilde_out, void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl(d, nullptr, q, k, v, beta, r, alpha, d1, S0, o, S_out, d_out, k_tilde_out, workspace,
                  workspace_bytes, stream);
}

osdn_status osdn_fwd_varlen(const osdn_desc *d, const int64_t *cu_seqlens, const void *q, const void *k,
                            const void *v, const float *beta, const float *r, const float *alpha, const float *d1,
                            const float *S0, void *o, float *S_out, float *d_out, void *k_tilde_out,
                            void *workspace, size_t workspace_bytes, void *stream) {
  OSDN_TRY(validate(d, 3));
  OSDN_TRY(check_ptr(cu_seqlens, "cu_seqlens", true));
  return fwd_impl(d, cu_seqlens, q, k, v, beta, r, alpha, d1, S0, o, S_out, d_out, k_tilde_out, workspace,
                  workspace_bytes, stream);
}

osdn_status osdn_fwd_noalloc(const osdn_desc *d, const void *q, const void *k, const void *v, const float *beta,
                             const float *r, const float *alpha, const float *d1, const float *S0, void *o,
                             float *S_out, float *d_out, void *k_tilde_out, void *stream) {
  OSDN_TRY(validate(d, 3));
  const size_t need = osdn_fwd_workspace_bytes(d);
  if (need > OSDN_FWD_NOALLOC_MAX_WORKSPACE)
    return fail(OSDN_EUNSUPPORTED, "osdn_fwd_noalloc: this problem needs %zu bytes of workspace, the built-in "
                "scratch holds %zu (call osdn_fwd with a workspace)", need, (size_t)OSDN_FWD_NOALLOC_MAX_WORKSPACE);
  int dev = -1;
  OSDN_TRY(hip_status(hipGetDevice(&dev), "osdn_fwd_noalloc: current device"));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(OSDN_EUNSUPPORTED, "osdn_fwd_noalloc: device %d out of range", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g_scratch_err[dev] == hipSuccess) g_scratch[dev] = p;
  });
  OSDN_TRY(hip_status(g_scratch_err[dev], "osdn_fwd_noalloc: scratch address"));
  if (!g_scratch[dev]) return fail(OSDN_EHIP, "osdn_fwd_noalloc: no scratch address on device %d", dev);
  return fwd_impl(d, nullptr, q, k, v, beta, r, alpha, d1, S0, o, S_out, d_out, k_tilde_out, g_scratch[dev],
                  OSDN_FWD_NOALLOC_MAX_WORKSPACE, stream);
}

osdn_status osdn_decode(const osdn_desc *d, const void *q, const void *k, const void *v, const float *beta,
                        const float *r, const float *alpha, const float *d1, const float *S0, void *o,
                        float *S_out, float *d_out, void *stream) {
  OSDN_TRY(validate(d, 3));
  if (d->r_per_key && r) return fail(OSDN_EUNSUPPORTED, "osdn_decode takes one retention per token and head");
  if (d->T > OSDN_DECODE_MAX_T)
    return fail(OSDN_EUNSUPPORTED, "osdn_decode takes at most %d tokens (got T=%lld)", OSDN_DECODE_MAX_T,
                (long long)d->T);
  if ((double)d->B * (double)d->H > 2147483647.0)
    return fail(OSDN_EUNSUPPORTED, "osdn_decode supports B*H < 2^31 (got %lld)", (long long)(d->B * d->H));
  const bool need_seq = d->T > 0;
  OSDN_TRY(check_ptr(q, "q", need_seq));
  OSDN_TRY(check_ptr(k, "k", need_seq));
  OSDN_TRY(check_ptr(v, "v", need_seq));
  OSDN_TRY(check_ptr(beta, "beta", need_seq));
  OSDN_TRY(check_ptr(r, "r", false));
  OSDN_TRY(check_ptr(alpha, "alpha", false));
  OSDN_TRY(check_ptr(d1, "d1", false));
  OSDN_TRY(check_ptr(S0, "S0", false));
  OSDN_TRY(check_ptr(o, "o", need_seq));
  OSDN_TRY(check_ptr(S_out, "S_out", false));
  OSDN_TRY(check_ptr(d_out, "d_out", false));
  if (o && (o == q || o == k || o == v)) return fail(OSDN_EINVAL, "o must not alias an input");
  if (S_out && (S_out == d1 || static_cast<const void *>(S_out) == o))
    return fail(OSDN_EINVAL, "S_out may alias S0 only");
  if (d_out && (d_out == S0 || static_cast<const void *>(d_out) == o))
    return fail(OSDN_EINVAL, "d_out may alias d1 only");
  osdn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.r = r;
  a.alpha = alpha;
  a.d1 = d1;
  a.S0 = S0;
  a.o = o;
  a.d_out = d_out;
  a.S_out = S_out;
  a.B = d->B;
  a.T = d->T;
  a.H = d->H;
  a.K = d->K;
  a.V = d->V;
  a.eta = d->eta;
  a.d_min = d->d_min;
  a.d_max = d->d_max;
  a.eps = d->eps;
  a.q_scale = d->q_scale;
  a.o_f32 = d->o_f32;
  a.clamp = d->clamp ? 1 : 0;
  a.beta_aware = d->beta_aware ? 1 : 0;
  OSDN_TRY(hip_status(osdn::launch_decode(a, d->dtype == OSDN_BF16, static_cast<hipStream_t>(stream)),
                      "decode launch"));
  return ok();
}

size_t osdn_bwd_workspace_bytes(const osdn_desc *d) {
  if (validate(d, 3) != OSDN_OK) return 0;
  return osdn::bwd_work_bytes(d->B, d->T, d->H, d->K, d->V);
}

osdn_status osdn_bwd(const osdn_desc *d, const void *q, const void *k, const void *v, const float *beta,
                     const float *r, const float *alpha, const float *d1, const float *S0, const void *dout,
                     const float *dS, const float *dd, void *dq, void *dk, void *dv, float *dbeta, float *dr,
                     float *dalpha, float *dd1, float *dS0, void *workspace, size_t workspace_bytes,
                     void *stream) {
  OSDN_TRY(validate(d, 3));
  if (d->r_per_key && r) return fail(OSDN_EUNSUPPORTED, "osdn_bwd takes one retention per token and head");
  if ((double)d->B * (double)d->H > 2147483647.0)
    return fail(OSDN_EUNSUPPORTED, "osdn_bwd supports B*H < 2^31 (got %lld)", (long long)(d->B * d->H));
  const bool need_seq = d->T > 0;
  OSDN_TRY(check_ptr(q, "q", need_seq));
  OSDN_TRY(check_ptr(k, "k", need_seq));
  OSDN_TRY(check_ptr(v, "v", need_seq));
  OSDN_TRY(check_ptr(beta, "beta", need_seq));
  OSDN_TRY(check_ptr(r, "r", false));
  OSDN_TRY(check_ptr(alpha, "alpha", false));
  OSDN_TRY(check_ptr(d1, "d1", false));
  OSDN_TRY(check_ptr(S0, "S0", false));
  OSDN_TRY(check_ptr(dout, "dout", need_seq));
  OSDN_TRY(check_ptr(dS, "dS", false));
  OSDN_TRY(check_ptr(dd, "dd", false));
  OSDN_TRY(check_ptr(dq, "dq", need_seq));
  OSDN_TRY(check_ptr(dk, "dk", need_seq));
  OSDN_TRY(check_ptr(dv, "dv", need_seq));
  OSDN_TRY(check_ptr(dbeta, "dbeta", need_seq));
  OSDN_TRY(check_ptr(dr, "dr", false));
  OSDN_TRY(check_ptr(dalpha, "dalpha", false));
  OSDN_TRY(check_ptr(dd1, "dd1", false));
  OSDN_TRY(check_ptr(dS0, "dS0", false));
  OSDN_TRY(check_ptr(workspace, "workspace", true));
  const void *ins[] = {q, k, v, beta, r, alpha, d1, S0, dout, dS, dd};
  const void *outs[] = {dq, dk, dv, dbeta, dr, dalpha, dd1, dS0};
  const int nout = (int)(sizeof outs / sizeof outs[0]);
  for (int x = 0; x < nout; ++x) {
    if (!outs[x]) continue;
    for (const void *i : ins)
      if (outs[x] == i) return fail(OSDN_EINVAL, "gradient outputs must not alias inputs");
    for (int y = x + 1; y < nout; ++y)
      if (outs[y] == outs[x]) return fail(OSDN_EINVAL, "gradient outputs must be distinct");
  }
  const size_t need = osdn::bwd_work_bytes(d->B, d->T, d->H, d->K, d->V);
  if (workspace_bytes < need)
    return fail(OSDN_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  osdn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.r = r;
  a.alpha = alpha;
  a.d1 = d1;
  a.S0 = S0;
  a.dout = dout;
  a.dS = dS;
  a.dd = dd;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dbeta = dbeta;
  a.dr = r ? dr : nullptr;
  a.dalpha = alpha ? dalpha : nullptr;
  a.dd1 = dd1;
  a.dS0 = dS0;
  a.B = d->B;
  a.T = d->T;
  a.H = d->H;
  a.K = d->K;
  a.V = d->V;
  a.eta = d->eta;
  a.d_min = d->d_min;
  a.d_max = d->d_max;
  a.eps = d->eps;
  a.q_scale = d->q_scale;
  a.clamp = d->clamp ? 1 : 0;
  a.beta_aware = d->beta_aware ? 1 : 0;
  a.o_f32 = d->o_f32;
  osdn::bwd_work_layout(a, workspace);
  OSDN_TRY(hip_status(osdn::launch_bwd(a, d->dtype == OSDN_BF16, static_cast<hipStream_t>(stream)),
                      "backward launch"));
  return ok();
}

size_t osdn_kda_fwd_workspace_bytes(const osdn_desc *d) {
  if (validate(d, 3) != OSDN_OK) return 0;
  return fwd_keys_bytes(d) + osdn::scan_work_bytes(d->B, d->T, d->H, d->K) +
         osdn::kda_work_bytes(d->B, d->T, d->H);
}

osdn_status osdn_kda_fwd(const osdn_desc *d, const void *q, const void *k, const void *v, const float *beta,
                         const float *r, const float *alpha, const float *d1, const float *S0, void *o,
                         float *S_out, float *d_out, void *k_tilde_out, void *workspace, size_t workspace_bytes,
                         void *stream) {
  OSDN_TRY(validate(d, 3));
  const bool need_seq = d->T > 0;
  OSDN_TRY(check_ptr(q, "q", need_seq));
  OSDN_TRY(check_ptr(k, "k", need_seq));
  OSDN_TRY(check_ptr(v, "v", need_seq));
  OSDN_TRY(check_ptr(beta, "beta", need_seq));
  OSDN_TRY(check_ptr(r, "r", false));
  OSDN_TRY(check_ptr(alpha, "alpha", false));
  OSDN_TRY(check_ptr(d1, "d1", false));
  OSDN_TRY(check_ptr(S0, "S0", false));
  OSDN_TRY(check_ptr(o, "o", need_seq));
  OSDN_TRY(check_ptr(S_out, "S_out", false));
  OSDN_TRY(check_ptr(d_out, "d_out", false));
  OSDN_TRY(check_ptr(k_tilde_out, "k_tilde_out", false));
  if (o && (o == q || o == k || o == v || o == k_tilde_out)) return fail(OSDN_EINVAL, "o must not alias an input");
  if (k_tilde_out && (k_tilde_out == q || k_tilde_out == k || k_tilde_out == v))
    return fail(OSDN_EINVAL, "k_tilde_out must not alias an input");
  if (S_out && (S_out == d1 || static_cast<const void *>(S_out) == o))
    return fail(OSDN_EINVAL, "S_out may alias S0 only");
  if (d_out && (d_out == S0 || static_cast<const void *>(d_out) == o))
    return fail(OSDN_EINVAL, "d_out may alias d1 only");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = d->dtype == OSDN_BF16;
  osdn::ScanArgs sa = scan_args(d, k, beta, r, d1, k_tilde_out, d_out);
  osdn::KdaArgs ka;
  ka.q = q;
  ka.k = k;
  ka.kt = k_tilde_out;
  ka.kt_is_res = false;
  ka.v = v;
  ka.beta = beta;
  ka.alpha = alpha;
  ka.S0 = S0;
  ka.o = o;
  ka.S_out = S_out;
  ka.B = d->B;
  ka.T = d->T;
  ka.H = d->H;
  ka.K = d->K;
  ka.V = d->V;
  ka.q_scale = d->q_scale;
  ka.o_f32 = d->o_f32;
  if (!need_seq) {
    // nothing to sweep: d_out = d1 and S_out = S0 (the kernels do the copy)
    OSDN_TRY(run_scan(d, sa, s));
    OSDN_TRY(hip_status(osdn::launch_kda(ka, bf, s), "phase-2 launch"));
    return ok();
  }
  OSDN_TRY(check_ptr(workspace, "workspace", true));
  const size_t need = osdn_kda_fwd_workspace_bytes(d);
  if (workspace_bytes < need)
    return fail(OSDN_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  char *ws = static_cast<char *>(workspace);
  if (keys_as_residual(d)) {
    // bf16: the write keys reach phase 2 as the bf16 residual (d - 1) (.) k
    sa.kt_res = ws;
    ka.kt = ws;
    ka.kt_is_res = true;
  } else if (!k_tilde_out) {
    sa.k_tilde = ws;
    ka.kt = ws;
  }
  const size_t scan_bytes = osdn::scan_work_bytes(d->B, d->T, d->H, d->K);
  const osdn::ScanWork sw = osdn::scan_work_layout(ws + fwd_keys_bytes(d), d->B, d->T, d->H, d->K);
  // bf16, K = 128, residual form, one retention per token: the intra pass
  // forms the residual from the chunked sweep's marks and step scalars
  const bool fold = osdn::kda_can_fold(ka, bf) && !(d->r_per_key && r) && !k_tilde_out;
  OSDN_TRY(hip_status(osdn::launch_precond_scan_chunked(sa, sw, bf, s, !fold), "phase-1 launch"));
  osdn::kda_work_layout(ka, ws + fwd_keys_bytes(d) + scan_bytes);
  if (fold) {
    osdn::EmitArgs em;
    em.cstep = sw.cstep;
    em.dstart = sw.dstart;
    em.pin = sw.pin;
    em.r = r;
    em.res = nullptr;
    em.d_min = d->d_min;
    em.d_max = d->d_max;
    em.clamp = d->clamp ? 1 : 0;
    OSDN_TRY(hip_status(osdn::launch_kda(ka, bf, s, &em), "phase-2 launch"));
  } else {
    OSDN_TRY(hip_status(osdn::launch_kda(ka, bf, s), "phase-2 launch"));
  }
  return ok();
}

}  // extern "C"
