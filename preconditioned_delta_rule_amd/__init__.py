"""OSDN forward hot path on MI355X: thin Python binding of libosdn.so.

The three calls mirror the C ABI of include/osdn.h (same names, same argument
order); this module only checks tensor metadata, allocates outputs through
PyTorch and passes device pointers plus the current HIP stream.  Every step of
the computation runs in the library's gfx950 kernels.  There is no fallback:
if libosdn.so is missing or cannot be loaded every call raises.

Paper: "OSDN: Improving Delta Rule with Provable Online Preconditioning in
Linear Attention" (arXiv:2605.13473) -- phase 1 is Algorithm 1 / Eq.(4) with
the APF retention of Eq.(7); phase 2 is the chunkwise delta rule with the
write key substituted in the chunk Gram and the local score (Eq.(6),
Appendix A.2), optionally gated (Appendix B.1).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["precond_scan", "precond_scan_workspace_bytes", "scan_counters", "chunk_fwd",
           "chunk_fwd_workspace_bytes", "fwd", "fwd_varlen", "fwd_noalloc", "FWD_NOALLOC_MAX_WORKSPACE", "kda_fwd", "kda_fwd_workspace_bytes", "decode", "DECODE_MAX_T", "bwd",
           "bwd_workspace_bytes", "kernel_times", "fwd_workspace_bytes", "fwd_scan_counters", "Desc", "OsdnError",
           "library_path", "load", "F32", "BF16"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libosdn.so")
_lib = None

F32, BF16 = 0, 1
OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
DECODE_MAX_T = 64  # OSDN_DECODE_MAX_T

SYMBOLS = ("osdn_desc_init", "osdn_validate", "osdn_precond_scan",
           "osdn_precond_scan_workspace_bytes", "osdn_precond_scan_counters_offset",
           "osdn_chunk_fwd", "osdn_chunk_fwd_workspace_bytes", "osdn_fwd_workspace_bytes",
           "osdn_fwd", "osdn_fwd_varlen", "osdn_fwd_noalloc", "osdn_decode", "osdn_bwd_workspace_bytes", "osdn_bwd",
           "osdn_kda_fwd_workspace_bytes", "osdn_kda_fwd", "osdn_profile_begin", "osdn_profile_end",
           "osdn_status_str", "osdn_last_error", "osdn_version")


class OsdnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (status_name(status), message))
        self.status = status


class Desc(ctypes.Structure):
    """Mirror of struct osdn_desc."""
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("K", ctypes.c_int64), ("V", ctypes.c_int64), ("chunk", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("eta", ctypes.c_float), ("d_min", ctypes.c_float),
                ("d_max", ctypes.c_float), ("clamp", ctypes.c_int32), ("eps", ctypes.c_float),
                ("q_scale", ctypes.c_float), ("beta_aware", ctypes.c_int32),
                ("r_per_key", ctypes.c_int32), ("o_f32", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libosdn.so (raises if it is missing) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libosdn.so not found at %s; build it with "
                           "`python -m preconditioned_delta_rule_amd.build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, fp, i64, ci = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    dp = ctypes.POINTER(Desc)
    lib.osdn_desc_init.argtypes = [dp, i64, i64, i64, i64, i64]
    lib.osdn_validate.argtypes = [dp]
    lib.osdn_precond_scan.argtypes = [dp, vp, fp, fp, fp, vp, fp, vp, ctypes.c_size_t, vp]
    lib.osdn_precond_scan_workspace_bytes.argtypes = [dp]
    lib.osdn_precond_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.osdn_precond_scan_counters_offset.argtypes = [dp]
    lib.osdn_precond_scan_counters_offset.restype = ctypes.c_int64
    lib.osdn_chunk_fwd.argtypes = [dp, vp, vp, vp, vp, fp, fp, fp, vp, fp, vp, ctypes.c_size_t, vp]
    lib.osdn_chunk_fwd_workspace_bytes.argtypes = [dp]
    lib.osdn_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.osdn_fwd_workspace_bytes.argtypes = [dp]
    lib.osdn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.osdn_fwd.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, vp, vp,
                             ctypes.c_size_t, vp]
    lib.osdn_decode.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, vp]
    lib.osdn_fwd_noalloc.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, vp, vp]
    lib.osdn_fwd_varlen.argtypes = [dp, vp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, vp, vp,
                                    ctypes.c_size_t, vp]
    lib.osdn_bwd_workspace_bytes.argtypes = [dp]
    lib.osdn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.osdn_bwd.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, vp, vp, vp, fp, fp, fp,
                             fp, fp, vp, ctypes.c_size_t, vp]
    lib.osdn_kda_fwd_workspace_bytes.argtypes = [dp]
    lib.osdn_kda_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.osdn_kda_fwd.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, vp, vp,
                                 ctypes.c_size_t, vp]
    lib.osdn_profile_begin.argtypes = [vp]
    lib.osdn_profile_end.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float),
                                     ci, ctypes.POINTER(ci)]
    lib.osdn_status_str.argtypes = [ci]
    lib.osdn_status_str.restype = ctypes.c_char_p
    lib.osdn_last_error.argtypes = []
    lib.osdn_last_error.restype = ctypes.c_char_p
    for name in ("osdn_desc_init", "osdn_validate", "osdn_precond_scan", "osdn_chunk_fwd",
                 "osdn_fwd", "osdn_fwd_varlen", "osdn_fwd_noalloc", "osdn_decode", "osdn_bwd", "osdn_kda_fwd",
                 "osdn_profile_begin",
                 "osdn_profile_end",
                 "osdn_version"):
        getattr(lib, name).restype = ci
    _lib = lib
    return lib


def status_name(status) -> str:
    try:
        return load().osdn_status_str(int(status)).decode()
    except Exception:
        return "status %d" % status


def _check(status):
    if status != OK:
        raise OsdnError(status, load().osdn_last_error().decode())


def make_desc(B, T, H, K, V, *, dtype=BF16, chunk=64, eta=0.003, d_min=0.5, d_max=2.0,
              clamp=True, eps=1e-6, q_scale=1.0, beta_aware=True, r_per_key=False,
              o_f32=False) -> Desc:
    d = Desc()
    _check(load().osdn_desc_init(ctypes.byref(d), B, T, H, K, V))
    d.dtype, d.chunk = int(dtype), int(chunk)
    d.eta, d.d_min, d.d_max = float(eta), float(d_min), float(d_max)
    d.clamp, d.eps, d.q_scale = int(bool(clamp)), float(eps), float(q_scale)
    d.beta_aware = int(bool(beta_aware))
    d.r_per_key = int(bool(r_per_key))
    d.o_f32 = int(bool(o_f32))
    return d


def _need_r(r, B, T, H, K, dev):
    """r is [B,T,H] (one retention per token and head) or [B,T,H,K] (vector
    retention); returns whether it is the vector form."""
    if r is not None and isinstance(r, torch.Tensor) and r.dim() == 4:
        _need(r, "r", (B, T, H, K), torch.float32, dev)
        return True
    _need(r, "r", (B, T, H), torch.float32, dev)
    return False


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(workspace, need, dev):
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if not isinstance(workspace, torch.Tensor) or workspace.device != dev \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % dev)
    return workspace


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def precond_scan_workspace_bytes(B, T, H, K, dtype=BF16) -> int:
    desc = make_desc(B, T, H, K, K, dtype=dtype)
    return int(load().osdn_precond_scan_workspace_bytes(ctypes.byref(desc)))


def scan_counters(workspace, B, T, H, K, dtype=BF16, offset=0):
    """Per-(b,h) chunk counters a chunked phase-1 sweep left in `workspace`
    (starting `offset` bytes in): int32 [B,H,3] = chunks taken with d pinned on
    d_min, in closed form with a fixed active set, and token by token."""
    desc = make_desc(B, T, H, K, K, dtype=dtype)
    off = offset + int(load().osdn_precond_scan_counters_offset(ctypes.byref(desc)))
    raw = workspace.view(torch.uint8).reshape(-1)[off:off + B * H * 3 * 4]
    return raw.cpu().view(torch.int32).reshape(B, H, 3)


def precond_scan(k, beta, r=None, d1=None, *, eta=0.003, d_min=0.5, d_max=2.0,
                 clamp=True, eps=1e-6, beta_aware=True, k_tilde=None, d_out=None,
                 chunked=True, workspace=None):
    """Phase 1.  k [B,T,H,K] (bf16/f32), beta [B,T,H] f32, r [B,T,H] or (vector
    retention) [B,T,H,K] f32, d1 [B,H,K] f32.  chunked=True runs the chunked
    kernels in `workspace` (allocated when None), chunked=False the
    token-by-token kernel (which vector retention always takes).
    Returns (k_tilde [B,T,H,K] in k's dtype, d_out [B,H,K] f32)."""
    B, T, H, K = k.shape
    dev, f32 = k.device, torch.float32
    _need(k, "k", (B, T, H, K), k.dtype, dev)
    _need(beta, "beta", (B, T, H), f32, dev)
    rvec = _need_r(r, B, T, H, K, dev)
    _need(d1, "d1", (B, H, K), f32, dev)
    if k_tilde is None:
        k_tilde = torch.empty_like(k)
    if d_out is None:
        d_out = torch.empty((B, H, K), dtype=f32, device=dev)
    _need(k_tilde, "k_tilde", (B, T, H, K), k.dtype, dev)
    _need(d_out, "d_out", (B, H, K), f32, dev)
    desc = make_desc(B, T, H, K, K, dtype=_dtype_code(k), eta=eta, d_min=d_min,
                     d_max=d_max, clamp=clamp, eps=eps, beta_aware=beta_aware, r_per_key=rvec)
    if chunked:
        need = int(load().osdn_precond_scan_workspace_bytes(ctypes.byref(desc)))
        workspace = _workspace(workspace, need, dev)
    else:
        workspace = None
    _check(load().osdn_precond_scan(ctypes.byref(desc), _ptr(k), _ptr(beta), _ptr(r),
                                    _ptr(d1), _ptr(k_tilde), _ptr(d_out), _ptr(workspace),
                                    ctypes.c_size_t(_nbytes(workspace)), _stream(dev)))
    return k_tilde, d_out


def chunk_fwd_workspace_bytes(B, T, H, K, V, dtype=BF16, chunk=64) -> int:
    desc = make_desc(B, T, H, K, V, dtype=dtype, chunk=chunk)
    return int(load().osdn_chunk_fwd_workspace_bytes(ctypes.byref(desc)))


def chunk_fwd(q, k, k_tilde, v, beta, alpha=None, S0=None, *, chunk=64, q_scale=1.0,
              o=None, S_out=None, two_pass=True, workspace=None, o_f32=False):
    """Phase 2.  q, k, k_tilde [B,T,H,K], v [B,T,H,V] (one dtype), beta and
    alpha [B,T,H] f32, S0 [B,H,V,K] f32.  two_pass=True hands the library a
    workspace (allocated when None) so that the matrix-core shapes form every
    chunk's (I + A)^-1 chunk-parallel first; two_pass=False passes none.
    o_f32=True returns o in float32 (the readout before rounding to q's dtype).
    Returns (o [B,T,H,V], S_out [B,H,V,K])."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev, dt, f32 = q.device, q.dtype, torch.float32
    for name, t in (("q", q), ("k", k), ("k_tilde", k_tilde)):
        _need(t, name, (B, T, H, K), dt, dev)
    _need(v, "v", (B, T, H, V), dt, dev)
    _need(beta, "beta", (B, T, H), f32, dev)
    _need(alpha, "alpha", (B, T, H), f32, dev)
    _need(S0, "S0", (B, H, V, K), f32, dev)
    odt = f32 if o_f32 else dt
    if o is None:
        o = torch.empty((B, T, H, V), dtype=odt, device=dev)
    if S_out is None:
        S_out = torch.empty((B, H, V, K), dtype=f32, device=dev)
    _need(o, "o", (B, T, H, V), odt, dev)
    _need(S_out, "S_out", (B, H, V, K), f32, dev)
    desc = make_desc(B, T, H, K, V, dtype=_dtype_code(q), chunk=chunk, q_scale=q_scale, o_f32=o_f32)
    need = int(load().osdn_chunk_fwd_workspace_bytes(ctypes.byref(desc))) if two_pass else 0
    workspace = _workspace(workspace, need, dev) if need else None
    _check(load().osdn_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(k_tilde), _ptr(v),
                                 _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(o), _ptr(S_out),
                                 _ptr(workspace), ctypes.c_size_t(_nbytes(workspace)),
                                 _stream(dev)))
    return o, S_out


def fwd_workspace_bytes(B, T, H, K, V, dtype=BF16, chunk=64) -> int:
    desc = make_desc(B, T, H, K, V, dtype=dtype, chunk=chunk)
    return int(load().osdn_fwd_workspace_bytes(ctypes.byref(desc)))


def fwd_scan_counters(workspace, B, T, H, K, V, dtype=BF16, chunk=64):
    """The phase-1 chunk counters (see scan_counters) inside an osdn_fwd workspace."""
    off = (fwd_workspace_bytes(B, T, H, K, V, dtype, chunk)
           - chunk_fwd_workspace_bytes(B, T, H, K, V, dtype, chunk)
           - precond_scan_workspace_bytes(B, T, H, K, dtype))
    return scan_counters(workspace, B, T, H, K, dtype, offset=off)


def fwd(q, k, v, beta, r=None, alpha=None, d1=None, S0=None, *, chunk=64, eta=0.003,
        d_min=0.5, d_max=2.0, clamp=True, eps=1e-6, q_scale=1.0, beta_aware=True,
        o=None, S_out=None, d_out=None, k_tilde_out=None, workspace=None, o_f32=False):
    """Both phases on the current stream.  o_f32=True returns o in float32 (the
    readout before rounding to q's dtype).  Returns (o, S_out, d_out)."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev, dt, f32 = q.device, q.dtype, torch.float32
    _need(k, "k", (B, T, H, K), dt, dev)
    _need(v, "v", (B, T, H, V), dt, dev)
    _need(beta, "beta", (B, T, H), f32, dev)
    rvec = _need_r(r, B, T, H, K, dev)
    _need(alpha, "alpha", (B, T, H), f32, dev)
    _need(d1, "d1", (B, H, K), f32, dev)
    _need(S0, "S0", (B, H, V, K), f32, dev)
    odt = f32 if o_f32 else dt
    if o is None:
        o = torch.empty((B, T, H, V), dtype=odt, device=dev)
    if S_out is None:
        S_out = torch.empty((B, H, V, K), dtype=f32, device=dev)
    if d_out is None:
        d_out = torch.empty((B, H, K), dtype=f32, device=dev)
    _need(o, "o", (B, T, H, V), odt, dev)
    _need(k_tilde_out, "k_tilde_out", (B, T, H, K), dt, dev)
    desc = make_desc(B, T, H, K, V, dtype=_dtype_code(q), chunk=chunk, eta=eta, d_min=d_min,
                     d_max=d_max, clamp=clamp, eps=eps, q_scale=q_scale, beta_aware=beta_aware,
                     r_per_key=rvec, o_f32=o_f32)
    need = int(load().osdn_fwd_workspace_bytes(ctypes.byref(desc)))
    workspace = _workspace(workspace, need, dev)
    _check(load().osdn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r),
                           _ptr(alpha), _ptr(d1), _ptr(S0), _ptr(o), _ptr(S_out), _ptr(d_out),
                           _ptr(k_tilde_out), _ptr(workspace),
                           ctypes.c_size_t(_nbytes(workspace)), _stream(dev)))
    return o, S_out, d_out


FWD_NOALLOC_MAX_WORKSPACE = 64 << 20  # OSDN_FWD_NOALLOC_MAX_WORKSPACE


def fwd_noalloc(q, k, v, beta, r=None, alpha=None, d1=None, S0=None, *, o, S_out, d_out, chunk=64,
                eta=0.003, d_min=0.5, d_max=2.0, clamp=True, eps=1e-6, q_scale=1.0, beta_aware=True,
                k_tilde_out=None, o_f32=False):
    """fwd with the library's built-in scratch as workspace (osdn_fwd_noalloc):
    the outputs o, S_out, d_out are the caller's and nothing is allocated.
    Returns (o, S_out, d_out)."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev, dt, f32 = q.device, q.dtype, torch.float32
    _need(k, "k", (B, T, H, K), dt, dev)
    _need(v, "v", (B, T, H, V), dt, dev)
    _need(beta, "beta", (B, T, H), f32, dev)
    rvec = _need_r(r, B, T, H, K, dev)
    _need(alpha, "alpha", (B, T, H), f32, dev)
    _need(d1, "d1", (B, H, K), f32, dev)
    _need(S0, "S0", (B, H, V, K), f32, dev)
    _need(o, "o", (B, T, H, V), f32 if o_f32 else dt, dev)
    _need(S_out, "S_out", (B, H, V, K), f32, dev)
    _need(d_out, "d_out", (B, H, K), f32, dev)
    _need(k_tilde_out, "k_tilde_out", (B, T, H, K), dt, dev)
    desc = make_desc(B, T, H, K, V, dtype=_dtype_code(q), chunk=chunk, eta=eta, d_min=d_min,
                     d_max=d_max, clamp=clamp, eps=eps, q_scale=q_scale, beta_aware=beta_aware,
                     r_per_key=rvec, o_f32=o_f32)
    _check(load().osdn_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r),
                                   _ptr(alpha), _ptr(d1), _ptr(S0), _ptr(o), _ptr(S_out), _ptr(d_out),
                                   _ptr(k_tilde_out), _stream(dev)))
    return o, S_out, d_out


def kda_fwd(q, k, v, beta, r=None, alpha=None, d1=None, S0=None, *, eta=0.003, d_min=0.5,
            d_max=2.0, clamp=True, eps=1e-6, q_scale=1.0, beta_aware=True, o=None, S_out=None,
            d_out=None, k_tilde_out=None, workspace=None, o_f32=False):
    """OSKDA forward on the current stream: q, k [B,T,H,K], v [B,T,H,V], beta
    [B,T,H], r [B,T,H] or [B,T,H,K], alpha [B,T,H,K] (channel-wise decay), d1
    [B,H,K], S0 [B,H,K,V].  Returns (o [B,T,H,V], S_out [B,H,K,V], d_out)."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev, dt, f32 = q.device, q.dtype, torch.float32
    _need(k, "k", (B, T, H, K), dt, dev)
    _need(v, "v", (B, T, H, V), dt, dev)
    _need(beta, "beta", (B, T, H), f32, dev)
    rvec = _need_r(r, B, T, H, K, dev)
    _need(alpha, "alpha", (B, T, H, K), f32, dev)
    _need(d1, "d1", (B, H, K), f32, dev)
    _need(S0, "S0", (B, H, K, V), f32, dev)
    odt = f32 if o_f32 else dt
    if o is None:
        o = torch.empty((B, T, H, V), dtype=odt, device=dev)
    if S_out is None:
        S_out = torch.empty((B, H, K, V), dtype=f32, device=dev)
    if d_out is None:
        d_out = torch.empty((B, H, K), dtype=f32, device=dev)
    _need(o, "o", (B, T, H, V), odt, dev)
    _need(k_tilde_out, "k_tilde_out", (B, T, H, K), dt, dev)
    desc = make_desc(B, T, H, K, V, dtype=_dtype_code(q), eta=eta, d_min=d_min, d_max=d_max,
                     clamp=clamp, eps=eps, q_scale=q_scale, beta_aware=beta_aware, r_per_key=rvec,
                     o_f32=o_f32)
    need = int(load().osdn_kda_fwd_workspace_bytes(ctypes.byref(desc)))
    workspace = _workspace(workspace, need, dev)
    _check(load().osdn_kda_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r),
                               _ptr(alpha), _ptr(d1), _ptr(S0), _ptr(o), _ptr(S_out), _ptr(d_out),
                               _ptr(k_tilde_out), _ptr(workspace),
                               ctypes.c_size_t(_nbytes(workspace)), _stream(dev)))
    return o, S_out, d_out


def kda_fwd_workspace_bytes(B, T, H, K, V, dtype=BF16) -> int:
    desc = make_desc(B, T, H, K, V, dtype=dtype)
    return int(load().osdn_kda_fwd_workspace_bytes(ctypes.byref(desc)))


def fwd_varlen(q, k, v, beta, r=None, alpha=None, d1=None, S0=None, *, cu_seqlens,
               max_seqlen=None, chunk=64, eta=0.003, d_min=0.5, d_max=2.0, clamp=True, eps=1e-6,
               q_scale=1.0, beta_aware=True, o=None, S_out=None, d_out=None, k_tilde_out=None,
               workspace=None, o_f32=False):
    """fwd over sequences packed on one token axis: q, k [1,total,H,K], v
    [1,total,H,V], beta/r/alpha [1,total,H]; cu_seqlens int64 [S+1] on the
    device (sequence b = tokens [cu[b], cu[b+1])); d1 [S,H,K], S0 [S,H,V,K].
    max_seqlen (the longest length) is read from cu_seqlens when None.
    Returns (o [1,total,H,V], S_out [S,H,V,K], d_out [S,H,K])."""
    _, total, H, K = q.shape
    V = v.shape[-1]
    dev, dt, f32 = q.device, q.dtype, torch.float32
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int64 \
            or cu_seqlens.device != dev or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int64 vector on %s" % dev)
    S = cu_seqlens.numel() - 1
    if max_seqlen is None:
        max_seqlen = int(torch.diff(cu_seqlens).max().item()) if S > 0 else 0
    _need(k, "k", (1, total, H, K), dt, dev)
    _need(v, "v", (1, total, H, V), dt, dev)
    _need(beta, "beta", (1, total, H), f32, dev)
    rvec = _need_r(r, 1, total, H, K, dev)
    _need(alpha, "alpha", (1, total, H), f32, dev)
    _need(d1, "d1", (S, H, K), f32, dev)
    _need(S0, "S0", (S, H, V, K), f32, dev)
    odt = f32 if o_f32 else dt
    if o is None:
        o = torch.empty((1, total, H, V), dtype=odt, device=dev)
    if S_out is None:
        S_out = torch.empty((S, H, V, K), dtype=f32, device=dev)
    if d_out is None:
        d_out = torch.empty((S, H, K), dtype=f32, device=dev)
    _need(o, "o", (1, total, H, V), odt, dev)
    _need(k_tilde_out, "k_tilde_out", (1, total, H, K), dt, dev)
    desc = make_desc(S, max_seqlen, H, K, V, dtype=_dtype_code(q), chunk=chunk, eta=eta,
                     d_min=d_min, d_max=d_max, clamp=clamp, eps=eps, q_scale=q_scale,
                     beta_aware=beta_aware, r_per_key=rvec, o_f32=o_f32)
    need = int(load().osdn_fwd_workspace_bytes(ctypes.byref(desc)))
    workspace = _workspace(workspace, need, dev)
    _check(load().osdn_fwd_varlen(ctypes.byref(desc), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(beta), _ptr(r), _ptr(alpha), _ptr(d1), _ptr(S0), _ptr(o),
                                  _ptr(S_out), _ptr(d_out), _ptr(k_tilde_out), _ptr(workspace),
                                  ctypes.c_size_t(_nbytes(workspace)), _stream(dev)))
    return o, S_out, d_out


def decode(q, k, v, beta, r=None, alpha=None, d1=None, S0=None, *, eta=0.003, d_min=0.5,
           d_max=2.0, clamp=True, eps=1e-6, q_scale=1.0, beta_aware=True, o=None, S_out=None,
           d_out=None, o_f32=False):
    """Decode step (the single-token recurrence, one launch): T <= DECODE_MAX_T
    new tokens per (b,h) from the carried (d1, S0).  Shapes as in fwd.  Pass
    S_out=S0 and d_out=d1 to update the state in place.
    Returns (o, S_out, d_out)."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev, dt, f32 = q.device, q.dtype, torch.float32
    _need(k, "k", (B, T, H, K), dt, dev)
    _need(v, "v", (B, T, H, V), dt, dev)
    _need(beta, "beta", (B, T, H), f32, dev)
    rvec = _need_r(r, B, T, H, K, dev)
    _need(alpha, "alpha", (B, T, H), f32, dev)
    _need(d1, "d1", (B, H, K), f32, dev)
    _need(S0, "S0", (B, H, V, K), f32, dev)
    odt = f32 if o_f32 else dt
    if o is None:
        o = torch.empty((B, T, H, V), dtype=odt, device=dev)
    if S_out is None:
        S_out = torch.empty((B, H, V, K), dtype=f32, device=dev)
    if d_out is None:
        d_out = torch.empty((B, H, K), dtype=f32, device=dev)
    _need(o, "o", (B, T, H, V), odt, dev)
    _need(S_out, "S_out", (B, H, V, K), f32, dev)
    _need(d_out, "d_out", (B, H, K), f32, dev)
    desc = make_desc(B, T, H, K, V, dtype=_dtype_code(q), eta=eta, d_min=d_min, d_max=d_max,
                     clamp=clamp, eps=eps, q_scale=q_scale, beta_aware=beta_aware, r_per_key=rvec,
                     o_f32=o_f32)
    _check(load().osdn_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r),
                              _ptr(alpha), _ptr(d1), _ptr(S0), _ptr(o), _ptr(S_out), _ptr(d_out),
                              _stream(dev)))
    return o, S_out, d_out


def bwd_workspace_bytes(B, T, H, K, V, dtype=BF16) -> int:
    desc = make_desc(B, T, H, K, V, dtype=dtype)
    return int(load().osdn_bwd_workspace_bytes(ctypes.byref(desc)))


def bwd(q, k, v, beta, r=None, alpha=None, d1=None, S0=None, *, dout, dS=None, dd=None,
        eta=0.003, d_min=0.5, d_max=2.0, clamp=True, eps=1e-6, q_scale=1.0, beta_aware=True,
        workspace=None, o_f32=False):
    """Backward pass of fwd: gradients of L given dout = dL/do [B,T,H,V] (dtype
    of q), dS = dL/dS_T [B,H,V,K] f32 and dd = dL/dd_{T+1} [B,H,K] f32 (both
    optional).  Returns a dict: dq, dk [B,T,H,K] and dv [B,T,H,V] in q's dtype;
    dbeta [B,T,H], dr and dalpha [B,T,H] (None when r / alpha are None),
    dd1 [B,H,K], dS0 [B,H,V,K] in f32.  o_f32=True returns dq, dk, dv in float32
    (before the rounding to q's dtype)."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev, dt, f32 = q.device, q.dtype, torch.float32
    _need(k, "k", (B, T, H, K), dt, dev)
    _need(v, "v", (B, T, H, V), dt, dev)
    _need(beta, "beta", (B, T, H), f32, dev)
    rvec = _need_r(r, B, T, H, K, dev)
    _need(alpha, "alpha", (B, T, H), f32, dev)
    _need(d1, "d1", (B, H, K), f32, dev)
    _need(S0, "S0", (B, H, V, K), f32, dev)
    _need(dout, "dout", (B, T, H, V), dt, dev)
    _need(dS, "dS", (B, H, V, K), f32, dev)
    _need(dd, "dd", (B, H, K), f32, dev)
    gdt = f32 if o_f32 else dt
    out = {"dq": torch.empty_like(q, dtype=gdt), "dk": torch.empty_like(k, dtype=gdt),
           "dv": torch.empty_like(v, dtype=gdt),
           "dbeta": torch.empty((B, T, H), dtype=f32, device=dev),
           "dr": torch.empty((B, T, H), dtype=f32, device=dev) if r is not None else None,
           "dalpha": torch.empty((B, T, H), dtype=f32, device=dev) if alpha is not None else None,
           "dd1": torch.empty((B, H, K), dtype=f32, device=dev),
           "dS0": torch.empty((B, H, V, K), dtype=f32, device=dev)}
    desc = make_desc(B, T, H, K, V, dtype=_dtype_code(q), eta=eta, d_min=d_min, d_max=d_max,
                     clamp=clamp, eps=eps, q_scale=q_scale, beta_aware=beta_aware, r_per_key=rvec,
                     o_f32=o_f32)
    need = int(load().osdn_bwd_workspace_bytes(ctypes.byref(desc)))
    workspace = _workspace(workspace, need, dev)
    _check(load().osdn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r),
                           _ptr(alpha), _ptr(d1), _ptr(S0), _ptr(dout), _ptr(dS), _ptr(dd),
                           _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
                           _ptr(out["dr"]), _ptr(out["dalpha"]), _ptr(out["dd1"]),
                           _ptr(out["dS0"]), _ptr(workspace), ctypes.c_size_t(_nbytes(workspace)),
                           _stream(dev)))
    return out


def kernel_times(fn, device=None):
    """Run fn() with a launch profile open on the current stream; returns
    [(kernel_name, milliseconds)] for every kernel the library launched."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    lib = load()
    _check(lib.osdn_profile_begin(_stream(dev)))
    try:
        fn()
    finally:
        cap = 1024
        names = (ctypes.c_char_p * cap)()
        ms = (ctypes.c_float * cap)()
        n = ctypes.c_int(0)
        _check(lib.osdn_profile_end(names, ms, cap, ctypes.byref(n)))
    return [(names[i].decode(), float(ms[i])) for i in range(min(n.value, cap))]
