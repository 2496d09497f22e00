"""OSDN CPU oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, sequential fp64 reference of the OSDN forward pass, written from
"OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
Attention" (arXiv:2605.13473).  The arithmetic lives in ``osdn_oracle.c``
(phase 1: Section 4.2 Eq.(4), Algorithm 1, Section 4.4 Eq.(7), Appendix B;
phase 2: Eq.(5), Appendix C Algorithm 2 (2b), Appendix B.1; the OSKDA phase 2
of Appendix B.2 / Table 3; vector retention, Proposition A.3); this module only
builds that file with gcc and marshals numpy arrays through ctypes.
``osdn_oracle_bwd.c`` (same library) holds the backward pass: reverse-mode
derivatives of that forward, pinned by finite differences of it.
``chunk_model.py`` holds an independent fp64 NumPy statement of the chunkwise
WY form (Appendix A.2 Eqs.(8)-(11), Appendix B.1 Eqs.(13)-(15), and the OSKDA
chunk form of Appendix B.2).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  It shares no code with the GPU library and never
imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "osdn_oracle.c")
_SRC_BWD = os.path.join(_HERE, "osdn_oracle_bwd.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile osdn_oracle.c and osdn_oracle_bwd.c into liboracle.so with gcc
    (OpenMP over sequences)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, _SRC, _SRC_BWD, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    i64, ci, cd = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.osdn_oracle_precond_scan.argtypes = [
        i64, i64, i64, i64, _dp, _dp, _dp, ci, _dp, cd, cd, cd, ci, cd, ci,
        _dp, _dp, _dp, ci]
    lib.osdn_oracle_precond_scan.restype = ci
    lib.osdn_oracle_delta_rule.argtypes = [
        i64, i64, i64, i64, i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp, cd,
        _dp, _dp, _dp, _dp, ci]
    lib.osdn_oracle_delta_rule.restype = ci
    lib.osdn_oracle_kda_rule.argtypes = [
        i64, i64, i64, i64, i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp, cd, _dp, _dp, ci]
    lib.osdn_oracle_kda_rule.restype = ci
    lib.osdn_oracle_diagnostics.argtypes = [
        i64, i64, i64, i64, i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
    lib.osdn_oracle_diagnostics.restype = ci
    if hasattr(lib, "osdn_oracle_backward"):
        lib.osdn_oracle_backward.argtypes = [
            i64, i64, i64, i64, i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
            cd, cd, cd, ci, cd, ci, cd, _dp, _dp, _dp,
            _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ci]
        lib.osdn_oracle_backward.restype = ci
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
                os.path.getmtime(_SRC), os.path.getmtime(_SRC_BWD)):
            build(force=True)
        _lib = bind(ctypes.CDLL(_LIB))
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return ctypes.cast(None, _dp)
    return x.ctypes.data_as(_dp)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)


def precond_scan(k, beta, r=None, d1=None, *, eta=0.003, d_min=0.5, d_max=2.0,
                 clamp=True, eps=1e-6, beta_aware=True, trajectory=False,
                 threads=None):
    """Phase 1 in fp64.  k [B,T,H,K], beta [B,T,H], d1 [B,H,K]; r [B,T,H] (one
    retention per token and head) or [B,T,H,K] (vector retention).

    Returns (k_tilde [B,T,H,K], d_out [B,H,K]) and, with trajectory=True, also
    d_traj [B,H,T+1,K] holding d_1 .. d_{T+1}.
    """
    k, beta, r, d1 = _f64(k), _f64(beta), _f64(r), _f64(d1)
    B, T, H, K = k.shape
    assert beta.shape == (B, T, H)
    r_per_key = r is not None and r.ndim == 4
    if r is not None:
        assert r.shape in ((B, T, H), (B, T, H, K))
    if d1 is not None:
        assert d1.shape == (B, H, K)
    kt = np.empty_like(k)
    d_out = np.empty((B, H, K), np.float64)
    d_traj = np.empty((B, H, T + 1, K), np.float64) if trajectory else None
    rc = _load().osdn_oracle_precond_scan(
        B, T, H, K, _ptr(k), _ptr(beta), _ptr(r), int(r_per_key), _ptr(d1), float(eta),
        float(d_min), float(d_max), int(bool(clamp)), float(eps),
        int(bool(beta_aware)), _ptr(kt), _ptr(d_out), _ptr(d_traj),
        int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle precond_scan rejected its arguments (%d)" % rc)
    return (kt, d_out, d_traj) if trajectory else (kt, d_out)


def delta_rule(q, k, k_tilde, v, beta, alpha=None, S0=None, *, q_scale=1.0,
               trajectory=False, threads=None):
    """Phase 2 token by token in fp64.

    Returns (o [B,T,H,V], S_out [B,H,V,K]); with trajectory=True also
    S_traj [B,H,T+1,V,K] and u [B,T,H,V].
    """
    q, k, k_tilde, v, beta = map(_f64, (q, k, k_tilde, v, beta))
    alpha, S0 = _f64(alpha), _f64(S0)
    B, T, H, K = k.shape
    V = v.shape[-1]
    assert q.shape == k.shape == k_tilde.shape and v.shape == (B, T, H, V)
    assert beta.shape == (B, T, H)
    if alpha is not None:
        assert alpha.shape == (B, T, H)
    if S0 is not None:
        assert S0.shape == (B, H, V, K)
    o = np.empty((B, T, H, V), np.float64)
    S_out = np.empty((B, H, V, K), np.float64)
    S_traj = np.empty((B, H, T + 1, V, K), np.float64) if trajectory else None
    u = np.empty((B, T, H, V), np.float64) if trajectory else None
    rc = _load().osdn_oracle_delta_rule(
        B, T, H, K, V, _ptr(q), _ptr(k), _ptr(k_tilde), _ptr(v), _ptr(beta),
        _ptr(alpha), _ptr(S0), float(q_scale), _ptr(o), _ptr(S_out),
        _ptr(S_traj), _ptr(u), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle delta_rule rejected its arguments (%d)" % rc)
    return (o, S_out, S_traj, u) if trajectory else (o, S_out)


def kda_rule(q, k, k_tilde, v, beta, alpha=None, S0=None, *, q_scale=1.0, threads=None):
    """OSKDA phase 2 token by token in fp64 (K x V state).  alpha [B,T,H,K]
    (channel-wise decay, or None), S0 [B,H,K,V].  Returns (o [B,T,H,V],
    S_out [B,H,K,V])."""
    q, k, k_tilde, v, beta = map(_f64, (q, k, k_tilde, v, beta))
    alpha, S0 = _f64(alpha), _f64(S0)
    B, T, H, K = k.shape
    V = v.shape[-1]
    assert q.shape == k.shape == k_tilde.shape and v.shape == (B, T, H, V)
    assert beta.shape == (B, T, H)
    if alpha is not None:
        assert alpha.shape == (B, T, H, K)
    if S0 is not None:
        assert S0.shape == (B, H, K, V)
    o = np.empty((B, T, H, V), np.float64)
    S_out = np.empty((B, H, K, V), np.float64)
    rc = _load().osdn_oracle_kda_rule(
        B, T, H, K, V, _ptr(q), _ptr(k), _ptr(k_tilde), _ptr(v), _ptr(beta), _ptr(alpha),
        _ptr(S0), float(q_scale), _ptr(o), _ptr(S_out), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle kda_rule rejected its arguments (%d)" % rc)
    return o, S_out


def kda_forward(q, k, v, beta, r=None, alpha=None, d1=None, S0=None, *, eta=0.003,
                d_min=0.5, d_max=2.0, clamp=True, eps=1e-6, beta_aware=True,
                q_scale=1.0, threads=None):
    """OSKDA, both phases (the phase-1 sweep is shared with OSDN, Eq.(12)):
    returns dict with k_tilde, d, o, S (S as [B,H,K,V]; all fp64)."""
    kt, d = precond_scan(k, beta, r, d1, eta=eta, d_min=d_min, d_max=d_max,
                         clamp=clamp, eps=eps, beta_aware=beta_aware,
                         threads=threads)
    o, S = kda_rule(q, k, kt, v, beta, alpha, S0, q_scale=q_scale, threads=threads)
    return {"k_tilde": kt, "d": d, "o": o, "S": S}


def diagnostics(k, k_tilde, v, beta, S_traj, u):
    """Per-token (a, n, f_pre, f_post, q, h) as [B,T,H,6] (see osdn_oracle.c)."""
    k, k_tilde, v, beta, S_traj, u = map(_f64, (k, k_tilde, v, beta, S_traj, u))
    B, T, H, K = k.shape
    V = v.shape[-1]
    diag = np.empty((B, T, H, 6), np.float64)
    rc = _load().osdn_oracle_diagnostics(
        B, T, H, K, V, _ptr(k), _ptr(k_tilde), _ptr(v), _ptr(beta),
        _ptr(S_traj), _ptr(u), _ptr(diag))
    if rc != 0:
        raise ValueError("oracle diagnostics rejected its arguments (%d)" % rc)
    return diag


def forward(q, k, v, beta, r=None, alpha=None, d1=None, S0=None, *, eta=0.003,
            d_min=0.5, d_max=2.0, clamp=True, eps=1e-6, beta_aware=True,
            q_scale=1.0, threads=None):
    """Both phases: returns dict with k_tilde, d, o, S (all fp64)."""
    kt, d = precond_scan(k, beta, r, d1, eta=eta, d_min=d_min, d_max=d_max,
                         clamp=clamp, eps=eps, beta_aware=beta_aware,
                         threads=threads)
    o, S = delta_rule(q, k, kt, v, beta, alpha, S0, q_scale=q_scale,
                      threads=threads)
    return {"k_tilde": kt, "d": d, "o": o, "S": S}


def backward(q, k, v, beta, r=None, alpha=None, d1=None, S0=None, *, dout, dS=None,
             dd=None, eta=0.003, d_min=0.5, d_max=2.0, clamp=True, eps=1e-6,
             beta_aware=True, q_scale=1.0, threads=None):
    """Gradients of L with dL/do = dout [B,T,H,V], dL/dS_T = dS [B,H,V,K] and
    dL/dd_{T+1} = dd [B,H,K] (both optional) through the forward above.

    Returns a dict with dq, dk [B,T,H,K], dv [B,T,H,V], dbeta [B,T,H] and, for
    the inputs given (r, alpha) or always (d1, S0), dr, dalpha [B,T,H],
    dd1 [B,H,K], dS0 [B,H,V,K] (all fp64).
    """
    q, k, v, beta, r, alpha, d1, S0 = map(_f64, (q, k, v, beta, r, alpha, d1, S0))
    dout, dS, dd = _f64(dout), _f64(dS), _f64(dd)
    B, T, H, K = k.shape
    V = v.shape[-1]
    assert q.shape == k.shape and v.shape == (B, T, H, V) and beta.shape == (B, T, H)
    assert dout.shape == (B, T, H, V)
    if dS is not None:
        assert dS.shape == (B, H, V, K)
    if dd is not None:
        assert dd.shape == (B, H, K)
    out = {"dq": np.zeros((B, T, H, K)), "dk": np.zeros((B, T, H, K)),
           "dv": np.zeros((B, T, H, V)), "dbeta": np.zeros((B, T, H)),
           "dr": np.zeros((B, T, H)) if r is not None else None,
           "dalpha": np.zeros((B, T, H)) if alpha is not None else None,
           "dd1": np.zeros((B, H, K)), "dS0": np.zeros((B, H, V, K))}
    rc = _load().osdn_oracle_backward(
        B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r), _ptr(alpha),
        _ptr(d1), _ptr(S0), float(eta), float(d_min), float(d_max), int(bool(clamp)),
        float(eps), int(bool(beta_aware)), float(q_scale), _ptr(dout), _ptr(dS), _ptr(dd),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
        _ptr(out["dr"]), _ptr(out["dalpha"]), _ptr(out["dd1"]), _ptr(out["dS0"]),
        int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle backward rejected its arguments (%d)" % rc)
    return out
