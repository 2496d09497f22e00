"""Pins of the oracle's OSKDA phase 2 (Appendix B.2, Table 3) and of vector
retention in phase 1 (Appendix A.5, Proposition A.3), against statements that
do not share its code:

- the pages' chunk form of OSKDA (Appendix B.2: Gamma-scaled Gram, M, W, U, the
  suffix-decayed state propagation and the intra-chunk output), stated in
  oracle/chunk_model.py, at several chunk lengths;
- Table 3's product form S_t = (I - beta k~ k^T) Diag(alpha) S + beta k~ v^T,
  built as explicit matrices;
- special cases that reduce to the already pinned OSDN / OSGDN oracle (no
  decay; the same decay on every channel) with the state transposed;
- Proposition A.3's affine matrix form of the unclamped vector-retention step,
  and its reduction to the scalar retention of Eq.(7).
"""
import numpy as np
import pytest

import oracle
from oracle import chunk_model



def case(seed, B=1, T=37, H=2, K=8, V=6, decay=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    alpha = np.exp(-rng.uniform(0.0, decay, (B, T, H, K)))
    r = rng.uniform(0.8, 1.0, (B, T, H, K))
    S0 = rng.standard_normal((B, H, K, V))
    d1 = rng.uniform(0.6, 1.9, (B, H, K))
    return dict(q=q, k=k, v=v, beta=beta, alpha=alpha, r=r, S0=S0, d1=d1)


@pytest.mark.parametrize("chunk", [1, 5, 16, 64])
@pytest.mark.parametrize("decay", [0.05, 0.3, 3.0])
def test_kda_recurrence_equals_chunk_form(chunk, decay):
    c = case(1, T=70, decay=decay)
    kt, _ = oracle.precond_scan(c["k"], c["beta"], c["r"], c["d1"], eta=0.2)
    o, S = oracle.kda_rule(c["q"], c["k"], kt, c["v"], c["beta"], c["alpha"], c["S0"],
                           q_scale=0.7)
    o2, S2 = chunk_model.kda_forward(c["q"], c["k"], kt, c["v"], c["beta"], c["alpha"],
                                     c["S0"], chunk=chunk, q_scale=0.7)
    scale = max(1.0, np.abs(o).max())
    assert np.abs(o - o2).max() <= 1e-9 * scale
    assert np.abs(S - S2).max() <= 1e-9 * max(1.0, np.abs(S).max())


def test_kda_matches_table3_product_form():
    c = case(2, T=19, H=1, K=5, V=4)
    kt = c["k"] * np.random.default_rng(3).uniform(0.5, 2.0, c["k"].shape)
    o, S = oracle.kda_rule(c["q"], c["k"], kt, c["v"], c["beta"], c["alpha"], c["S0"])
    St = c["S0"][0, 0].copy()
    for t in range(19):
        kk, ww, vv = c["k"][0, t, 0], kt[0, t, 0], c["v"][0, t, 0]
        b = c["beta"][0, t, 0]
        St = (np.eye(5) - b * np.outer(ww, kk)) @ np.diag(c["alpha"][0, t, 0]) @ St \
            + b * np.outer(ww, vv)
        np.testing.assert_allclose(o[0, t, 0], St.T @ c["q"][0, t, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], St, rtol=1e-12, atol=1e-12)


def test_kda_without_decay_is_osdn_transposed():
    c = case(4)
    kt, _ = oracle.precond_scan(c["k"], c["beta"], eta=0.3)
    o, S = oracle.kda_rule(c["q"], c["k"], kt, c["v"], c["beta"], None, c["S0"], q_scale=0.5)
    o2, S2 = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"], None,
                               np.swapaxes(c["S0"], -1, -2), q_scale=0.5)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, np.swapaxes(S2, -1, -2), rtol=1e-12, atol=1e-12)


def test_kda_with_uniform_channel_decay_is_gated_deltanet_transposed():
    c = case(5)
    a = c["alpha"][..., 0]
    kt, _ = oracle.precond_scan(c["k"], c["beta"], eta=0.3)
    o, S = oracle.kda_rule(c["q"], c["k"], kt, c["v"], c["beta"],
                           np.repeat(a[..., None], 8, axis=-1), c["S0"])
    o2, S2 = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"], a,
                               np.swapaxes(c["S0"], -1, -2))
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, np.swapaxes(S2, -1, -2), rtol=1e-12, atol=1e-12)


def test_kda_decay_acts_on_key_rows_before_the_read():
    """One channel decays to (almost) nothing at token 1: the state row of that
    key coordinate holds only what token 1 wrote, and token 1's residual reads
    the decayed state (post-gate residual)."""
    K, V = 3, 2
    S0 = np.arange(1.0, 7.0).reshape(1, 1, K, V)
    alpha = np.ones((1, 1, 1, K))
    alpha[..., 1] = 1e-30
    k = np.array([0.0, 1.0, 0.0]).reshape(1, 1, 1, K)
    v = np.array([5.0, -1.0]).reshape(1, 1, 1, V)
    beta = np.full((1, 1, 1), 0.5)
    o, S = oracle.kda_rule(k, k, k, v, beta, alpha, S0)
    # row 1 decays to ~0, u = v - 0, the write adds beta * 1 * u to row 1
    np.testing.assert_allclose(S[0, 0, 1], 0.5 * v[0, 0, 0], atol=1e-12)
    np.testing.assert_allclose(S[0, 0, [0, 2]], S0[0, 0, [0, 2]])
    np.testing.assert_allclose(o[0, 0, 0], S[0, 0, 1])


def test_vector_retention_with_equal_entries_is_scalar_retention():
    c = case(6)
    rs = c["r"][..., 0]
    kv, dv = oracle.precond_scan(c["k"], c["beta"], np.repeat(rs[..., None], 8, axis=-1),
                                 c["d1"], eta=0.4)
    ks, ds = oracle.precond_scan(c["k"], c["beta"], rs, c["d1"], eta=0.4)
    np.testing.assert_array_equal(kv, ks)
    np.testing.assert_array_equal(dv, ds)


@pytest.mark.parametrize("beta_aware", [True, False])
def test_vector_retention_matches_proposition_a3_affine_form(beta_aware):
    """Unclamped: d_{t+1} = (diag(r_t) - eta b'^2/n s s^T) d_t + eta b'/n s."""
    c = case(7, T=25, H=1, K=6)
    eta, eps = 0.35, 1e-6
    _, _, traj = oracle.precond_scan(c["k"], c["beta"], c["r"], c["d1"], eta=eta, clamp=False,
                                     beta_aware=beta_aware, trajectory=True)
    d = c["d1"][0, 0].copy()
    for t in range(25):
        s = c["k"][0, t, 0] ** 2
        n = max(s.sum(), eps)
        b = c["beta"][0, t, 0] if beta_aware else 1.0
        Amat = np.diag(c["r"][0, t, 0]) - eta * b * b / n * np.outer(s, s)
        d = Amat @ d + eta * b / n * s
        np.testing.assert_allclose(traj[0, 0, t + 1], d, rtol=1e-12, atol=1e-13)


def test_vector_retention_one_hot_keys_decouple():
    """With one-hot keys only the hot coordinate gets a step; every other
    coordinate only decays by its own retention (then the box applies)."""
    K, T = 4, 30
    rng = np.random.default_rng(8)
    hot = rng.integers(0, K, T)
    k = np.zeros((1, T, 1, K))
    k[0, np.arange(T), 0, hot] = 1.0
    beta = rng.uniform(0.2, 0.9, (1, T, 1))
    r = rng.uniform(0.7, 1.0, (1, T, 1, K))
    eta = 0.3
    _, _, traj = oracle.precond_scan(k, beta, r, eta=eta, trajectory=True)
    d = np.ones(K)
    for t in range(T):
        j = hot[t]
        b = beta[0, t, 0]
        step = np.zeros(K)
        step[j] = eta * b * (1 - b * d[j])
        d = np.clip(r[0, t, 0] * d + step, 0.5, 2.0)
        np.testing.assert_allclose(traj[0, 0, t + 1], d, rtol=1e-13, atol=1e-14)
