"""fp64 NumPy statement of the chunkwise WY form -- TEST INFRASTRUCTURE ONLY.

This is the second half of the oracle: it states the chunk-parallel algebra the
paper gives for phase 2, so that CPU tests can check, independently of any GPU
code, that chunkwise equals the token-by-token recurrence of osdn_oracle.c.

OSDN (Appendix A.2).  For one chunk of C tokens with physical keys K, write keys
K~ (both C x K), values V (C x V), gates B = diag(beta) and boundary state S:

    Tm  = (I + strict_lower(B K K~^T))^-1          Eq.(8)
    W   = Tm B K,   U = Tm B V                     Eq.(9)
    P   = I - W^T K~  (= prod_i (I - beta_i k_i k~_i^T))   Eq.(10)
    D   = U - W S^T                                (the chunk's state increments)
    S'  = S + D^T K~                               Eq.(11)
    O   = Q S^T + lower_incl_diag(Q K~^T) D        (readout o_t = S_t q_t of
                                                    Section 3, expanded per chunk)

Gated DeltaNet variant (Appendix B.1) with in-chunk cumulative decay
gamma_i = prod_{l<=i} alpha_l:

    A_ij = 1[j<i] beta_i (gamma_i/gamma_j) <k_i, k~_j>
    M    = (I + A)^-1 B                            Eq.(13)
    W    = M (gamma . K),  U = M V                 Eq.(14)
    S'   = gamma_C S + (U - W S^T)^T (rho . K~),  rho_i = gamma_C/gamma_i   Eq.(15)
    O    = (gamma . Q) S^T + [1[j<=i] (gamma_i/gamma_j) <q_i, k~_j>] (U - W S^T)

The readout of the gated form is the post-write readout o_t = S_t q_t expanded
the same way.

OSKDA (Appendix B.2), state S in R^{K x V}, channel-wise decay alpha_t in
R^K, Gamma_i = prod_{l<=i} alpha_l (per channel), gamma_C = Gamma_C:

    A_ij = 1[j<i] beta_i <Gamma_i . k_i, k~_j / Gamma_j>
    M    = (I + A)^-1 B
    W    = M (Gamma . K),  U = M V
    S'   = Diag(gamma_C) S + ((gamma_C / Gamma) . K~)^T (U - W S)
    O    = (Gamma . Q) S + lower_incl_diag((Gamma . Q)(K~ / Gamma)^T) (U - W S)  A partial last chunk (T not a multiple of C) is processed as a
shorter chunk.  Arrays use the [B,T,H,X] layout; everything is float64.
"""
from __future__ import annotations

import numpy as np


def wy_factors(K, Kt, V, beta):
    """Eq.(8)-(9): returns (Tm, W, U) for one chunk."""
    C = K.shape[0]
    Bm = np.diag(beta)
    A = np.tril(Bm @ K @ Kt.T, -1)
    Tm = np.linalg.inv(np.eye(C) + A)
    W = Tm @ Bm @ K
    U = Tm @ Bm @ V
    return Tm, W, U


def chunk_step(S, Q, K, Kt, V, beta, q_scale=1.0):
    """One OSDN chunk: returns (O [C,V], S_next [V,K])."""
    _, W, U = wy_factors(K, Kt, V, beta)
    D = U - W @ S.T
    Qs = q_scale * Q
    O = Qs @ S.T + np.tril(Qs @ Kt.T) @ D
    S_next = S + D.T @ Kt
    return O, S_next


def gated_chunk_step(S, Q, K, Kt, V, beta, alpha, q_scale=1.0):
    """One OSGDN chunk (Appendix B.1): returns (O [C,V], S_next [V,K])."""
    C = K.shape[0]
    gamma = np.cumprod(alpha)
    ratio = gamma[:, None] / gamma[None, :]          # gamma_i / gamma_j
    A = np.tril(beta[:, None] * ratio * (K @ Kt.T), -1)
    M = np.linalg.inv(np.eye(C) + A) @ np.diag(beta)
    W = M @ (gamma[:, None] * K)
    U = M @ V
    D = U - W @ S.T
    Qs = q_scale * Q
    O = (gamma[:, None] * Qs) @ S.T + np.tril(ratio * (Qs @ Kt.T)) @ D
    rho = gamma[-1] / gamma
    S_next = gamma[-1] * S + D.T @ (rho[:, None] * Kt)
    return O, S_next


def kda_chunk_step(S, Q, K, Kt, V, beta, alpha, q_scale=1.0):
    """One OSKDA chunk (Appendix B.2): S [K,V], alpha [C,K]; returns
    (O [C,V], S_next [K,V])."""
    C = K.shape[0]
    G = np.cumprod(alpha, axis=0)                     # Gamma [C,K]
    A = np.tril(beta[:, None] * ((G * K) @ (Kt / G).T), -1)
    M = np.linalg.inv(np.eye(C) + A) @ np.diag(beta)
    W = M @ (G * K)
    U = M @ V
    D = U - W @ S
    Qg = G * (q_scale * Q)
    O = Qg @ S + np.tril(Qg @ (Kt / G).T) @ D
    S_next = G[-1][:, None] * S + ((G[-1][None, :] / G) * Kt).T @ D
    return O, S_next


def kda_forward(q, k, k_tilde, v, beta, alpha=None, S0=None, *, chunk=64, q_scale=1.0):
    """Chunkwise OSKDA phase 2 over [B,T,H,*] inputs; alpha [B,T,H,K] or None,
    S0 [B,H,K,V].  Returns (o, S_out [B,H,K,V])."""
    q, k, k_tilde, v, beta = (np.asarray(x, np.float64) for x in (q, k, k_tilde, v, beta))
    B, T, H, Kd = k.shape
    Vd = v.shape[-1]
    o = np.zeros((B, T, H, Vd))
    S_out = np.zeros((B, H, Kd, Vd))
    for b in range(B):
        for h in range(H):
            S = np.zeros((Kd, Vd)) if S0 is None else np.array(S0[b, h], np.float64)
            for t0 in range(0, T, chunk):
                sl = slice(t0, min(T, t0 + chunk))
                al = (np.ones((sl.stop - t0, Kd)) if alpha is None
                      else np.asarray(alpha[b, sl, h], np.float64))
                O, S = kda_chunk_step(S, q[b, sl, h], k[b, sl, h], k_tilde[b, sl, h],
                                      v[b, sl, h], beta[b, sl, h], al, q_scale=q_scale)
                o[b, sl, h] = O
            S_out[b, h] = S
    return o, S_out


def forward(q, k, k_tilde, v, beta, alpha=None, S0=None, *, chunk=64,
            q_scale=1.0):
    """Chunkwise phase 2 over [B,T,H,*] inputs.  Returns (o, S_out)."""
    q, k, k_tilde, v, beta = (np.asarray(x, np.float64) for x in (q, k, k_tilde, v, beta))
    B, T, H, Kd = k.shape
    Vd = v.shape[-1]
    o = np.zeros((B, T, H, Vd))
    S_out = np.zeros((B, H, Vd, Kd))
    for b in range(B):
        for h in range(H):
            S = np.zeros((Vd, Kd)) if S0 is None else np.array(S0[b, h], np.float64)
            for t0 in range(0, T, chunk):
                sl = slice(t0, min(T, t0 + chunk))
                args = (S, q[b, sl, h], k[b, sl, h], k_tilde[b, sl, h],
                        v[b, sl, h], beta[b, sl, h])
                if alpha is None:
                    O, S = chunk_step(*args, q_scale=q_scale)
                else:
                    O, S = gated_chunk_step(*args, np.asarray(alpha[b, sl, h], np.float64),
                                            q_scale=q_scale)
                o[b, sl, h] = O
            S_out[b, h] = S
    return o, S_out
