"""Pins of the CPU oracle against what the paper fixes (no GPU needed).

Every test here checks the oracle against something other than itself: values
printed on the pages (tests/golden/), closed forms derived from the paper's
equations, identities proved in the paper, brute force on tiny inputs, or a
different statement of the same recurrence that the paper gives.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import chunk_model
from workloads import bf16_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def rand_case(rng, B=2, T=40, H=2, K=8, V=6, unit=True, apf=False, gdn=False):
    k = rng.standard_normal((B, T, H, K))
    if unit:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((B, T, H, K))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    r = 1.0 / (1.0 + np.exp(-(rng.standard_normal((B, T, H)) + 2.0))) if apf else None
    alpha = np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((B, T, H))))) if gdn else None
    return dict(q=q, k=k, v=v, beta=beta, r=r, alpha=alpha)


# ---------------------------------------------------------------- P-1
def test_p1_eta_zero_reduces_to_deltanet(oracle_lib):
    """eta=0, d_1=1: the write key equals the key bitwise and d never moves
    (Appendix C Algorithm 2: phase 1 is the only difference from DeltaNet);
    phase 2 then equals DeltaNet in its transition-matrix form (Table 3 row
    'DeltaNet': S_t = S_{t-1}(I - beta k k^T) + beta v k^T, o_t = S_t q_t)."""
    rng = np.random.default_rng(1)
    c = rand_case(rng, B=1, T=24, H=2, K=5, V=3)
    kt, d = oracle.precond_scan(c["k"], c["beta"], eta=0.0)
    assert np.array_equal(kt, c["k"])
    assert np.array_equal(d, np.ones_like(d))
    o, S = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"])
    for h in range(2):
        Sm = np.zeros((3, 5))
        for t in range(24):
            kk, vv, bb = c["k"][0, t, h], c["v"][0, t, h], c["beta"][0, t, h]
            Sm = Sm @ (np.eye(5) - bb * np.outer(kk, kk)) + bb * np.outer(vv, kk)
            np.testing.assert_allclose(o[0, t, h], Sm @ c["q"][0, t, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S[0, h], Sm, rtol=1e-12, atol=1e-13)


def test_p1_orthonormal_exact_recall(oracle_lib):
    """Textbook delta-rule property: with beta=1, d=1 and orthonormal keys every
    write makes S k_i = v_i and later writes to orthogonal keys leave it intact
    (Appendix A.1: the unit step replaces the stored value)."""
    K = V = 6
    rng = np.random.default_rng(2)
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys = Qm.T  # rows orthonormal
    k = keys[None, :, None, :]
    v = rng.standard_normal((1, K, 1, V))
    beta = np.ones((1, K, 1))
    kt, _ = oracle.precond_scan(k, beta, eta=0.0)
    S0 = rng.standard_normal((1, 1, V, K))
    _, S = oracle.delta_rule(k, k, kt, v, beta, S0=S0)
    for i in range(K):
        np.testing.assert_allclose(S[0, 0] @ keys[i], v[0, i, 0], atol=1e-12)


# ---------------------------------------------------------------- P-2
@pytest.mark.parametrize("apf", [False, True])
def test_p2_residual_identity(oracle_lib, apf):
    """Lemma 4.1 proof (Appendix A.3): S_t k_t - v_t = -u_t (1 - a_t) with
    a_t = beta_t <d_t, k_t^2> computed from the phase-1 trajectory d_t.
    A write key emitted after the update, a read with k~, or a misplaced beta
    all break it."""
    rng = np.random.default_rng(3)
    c = rand_case(rng, B=2, T=30, H=2, K=6, V=4, apf=apf)
    kt, d, dtr = oracle.precond_scan(c["k"], c["beta"], c["r"], eta=0.2,
                                     trajectory=True)
    o, S, Str, u = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"],
                                     trajectory=True)
    for b in range(2):
        for h in range(2):
            for t in range(30):
                kk = c["k"][b, t, h]
                a = c["beta"][b, t, h] * np.dot(dtr[b, h, t], kk * kk)
                lhs = Str[b, h, t + 1] @ kk - c["v"][b, t, h]
                rhs = -u[b, t, h] * (1.0 - a)
                np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-12)
                # u_t itself is the read with the physical key
                np.testing.assert_allclose(u[b, t, h], c["v"][b, t, h] - Str[b, h, t] @ kk,
                                           rtol=1e-12, atol=1e-13)
                # readout after the write, Section 3: o_t = S_t q_t
                np.testing.assert_allclose(o[b, t, h], Str[b, h, t + 1] @ c["q"][b, t, h],
                                           rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P-3
def _h_definition(S_prev, k, v, beta, d):
    """h_t(d) = (f_t(S_t(d)) - f_t(S_{t-1})) / ||grad f_t(S_{t-1})||_F^2 with
    S_t(d) = S_{t-1} - beta grad f_t(S_{t-1}) Diag(d)  (Section 4.2, Eq.(17))."""
    f = lambda S: 0.5 * np.sum((S @ k - v) ** 2)
    grad = np.outer(S_prev @ k - v, k)
    S_new = S_prev - beta * grad @ np.diag(d)
    return (f(S_new) - f(S_prev)) / np.sum(grad * grad)


def test_p3_hypergradient_and_phase1_direction(oracle_lib):
    """Eq.(3)/(18) and Lemma D.6 checked from the surrogate's definition:
    closed-form h equals the definition; the oracle's phase-1 step equals
    -eta * grad h (central differences of the definition); the Hessian is
    beta^2 s s^T / n."""
    rng = np.random.default_rng(4)
    K = V = 4
    for trial in range(5):
        S_prev = rng.standard_normal((V, K))
        k = rng.standard_normal(K) * (0.5 + trial * 0.3)
        v = rng.standard_normal(V)
        beta = float(rng.uniform(0.1, 0.9))
        d = rng.uniform(0.6, 1.8, K)
        eta = 0.01
        # oracle phase 2 from S_prev with this d, read its diagnostics
        kt = (d * k)[None, None, None, :]
        kk = k[None, None, None, :]
        vv = v[None, None, None, :]
        bb = np.array([[[beta]]])
        o, S, Str, u = oracle.delta_rule(kk, kk, kt, vv, bb, S0=S_prev[None, None],
                                         trajectory=True)
        diag = oracle.diagnostics(kk, kt, vv, bb, Str, u)
        h_def = _h_definition(S_prev, k, v, beta, d)
        assert diag[0, 0, 0, 5] == pytest.approx(h_def, rel=1e-10, abs=1e-13)
        # finite-difference gradient of the definition
        g = np.zeros(K)
        step = 1e-5
        for i in range(K):
            e = np.zeros(K)
            e[i] = step
            g[i] = (_h_definition(S_prev, k, v, beta, d + e)
                    - _h_definition(S_prev, k, v, beta, d - e)) / (2 * step)
        # the oracle's unclamped, unretained phase-1 step from d is -eta * grad h
        _, d_next = oracle.precond_scan(kk, bb, d1=d[None, None, :], eta=eta,
                                        clamp=False)
        np.testing.assert_allclose(d_next[0, 0] - d, -eta * g, rtol=1e-6, atol=1e-11)
        # Hessian: beta^2 s s^T / n
        s = k * k
        n = float(np.dot(k, k))
        Hfd = np.zeros((K, K))
        for i in range(K):
            for j in range(K):
                ei = np.zeros(K); ei[i] = 1e-3
                ej = np.zeros(K); ej[j] = 1e-3
                Hfd[i, j] = (_h_definition(S_prev, k, v, beta, d + ei + ej)
                             - _h_definition(S_prev, k, v, beta, d + ei - ej)
                             - _h_definition(S_prev, k, v, beta, d - ei + ej)
                             + _h_definition(S_prev, k, v, beta, d - ei - ej)) / (4e-6)
        np.testing.assert_allclose(Hfd, beta ** 2 * np.outer(s, s) / n, rtol=1e-5, atol=1e-8)


# ---------------------------------------------------------------- P-4 / P-15
def test_p4_monotone_descent_unit_keys(oracle_lib):
    """Corollary A.2 and Proposition A.1: unit keys, d in the box, beta in (0,1)
    give 0 < a_t < 2, loss ratio q_t = (1 - a_t)^2 < 1 and beta^2 sum k^4 <= 1;
    Theorem D.7's AM-GM step: prod q_t <= (mean q_t)^T."""
    rng = np.random.default_rng(5)
    c = rand_case(rng, B=2, T=50, H=2, K=8, V=5, apf=True)
    kt, d = oracle.precond_scan(c["k"], c["beta"], c["r"], eta=0.05)
    o, S, Str, u = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"],
                                     trajectory=True)
    diag = oracle.diagnostics(c["k"], kt, c["v"], c["beta"], Str, u)
    a, q = diag[..., 0], diag[..., 4]
    assert np.all(a > 0) and np.all(a < 2)
    np.testing.assert_allclose(q, (1 - a) ** 2, rtol=1e-9, atol=1e-12)
    assert np.all(q < 1)
    assert np.all(c["beta"] ** 2 * np.sum(c["k"] ** 4, -1) <= 1 + 1e-15)
    for b in range(2):
        for h in range(2):
            qs = q[b, :, h]
            assert np.prod(qs) <= np.mean(qs) ** len(qs) * (1 + 1e-12)


# ---------------------------------------------------------------- P-5
def test_p5_box_invariant(oracle_lib):
    """The clamp after every update (Algorithm 2 line 12): d_t in [d_min, d_max]
    for t >= 2; one stream pushes d to the upper bound (no retention, large
    step), the other to the lower bound (APF retention)."""
    rng = np.random.default_rng(6)
    hit = []
    for apf in (False, True):
        c = rand_case(rng, B=2, T=80, H=3, K=6, V=2, apf=apf)
        _, _, dtr = oracle.precond_scan(c["k"], c["beta"], c["r"], eta=0.5,
                                        d_min=0.7, d_max=1.3, trajectory=True)
        tail = dtr[:, :, 1:]
        assert tail.min() >= 0.7 and tail.max() <= 1.3
        hit.append((np.any(tail == 0.7), np.any(tail == 1.3)))
    assert hit[0][1] and hit[1][0]


# ---------------------------------------------------------------- P-6
def _onehot_stream(K, T, j, beta, r=None):
    k = np.zeros((1, T, 1, K))
    k[0, :, 0, j] = 1.0
    b = np.full((1, T, 1), beta)
    rr = None if r is None else np.full((1, T, 1), r)
    return k, b, rr


def test_p6_onehot_closed_form_upper_clamp(oracle_lib):
    """Derived from Eq.(4): a one-hot key e_j with constant beta gives, on
    coordinate j, d_{t+1} = (1 - eta beta^2) d_t + eta beta, i.e.
    d_{t+1} = 1/beta + (1 - 1/beta)(1 - eta beta^2)^t from d_1 = 1.  With
    beta=0.3, eta=0.05 it first exceeds 2 at t=125, so d_126 = 2 (upper clamp);
    other coordinates never move."""
    beta, eta, T = 0.3, 0.05, 140
    k, b, _ = _onehot_stream(3, T, 1, beta)
    _, _, dtr = oracle.precond_scan(k, b, eta=eta, trajectory=True)
    closed = [1 / beta + (1 - 1 / beta) * (1 - eta * beta ** 2) ** t for t in range(T + 1)]
    first = next(t for t in range(T + 1) if closed[t] > 2.0)
    assert first == 125
    for t in range(first):
        assert dtr[0, 0, t, 1] == pytest.approx(closed[t], rel=1e-12)
    assert np.all(dtr[0, 0, first:, 1] == 2.0)
    assert np.all(dtr[0, 0, :, 0] == 1.0) and np.all(dtr[0, 0, :, 2] == 1.0)


def test_p6_onehot_apf_lower_clamp(oracle_lib):
    """Eq.(7) with constant retention r: the hit coordinate follows
    d_{t+1} - d* = (r - eta beta^2)(d_t - d*), d* = eta beta / (1 - r + eta beta^2);
    an untouched coordinate follows d_{t+1} = r^t until the lower clamp:
    0.9^6 > 0.5 > 0.9^7, so d_8 = 0.5 and it stays there."""
    beta, eta, r, T = 0.5, 0.05, 0.9, 20
    k, b, rr = _onehot_stream(2, T, 0, beta, r)
    _, _, dtr = oracle.precond_scan(k, b, rr, eta=eta, trajectory=True)
    dstar = eta * beta / (1 - r + eta * beta ** 2)
    lam = r - eta * beta ** 2
    for t in range(T + 1):
        want = dstar + lam ** t * (1 - dstar)
        want = max(want, 0.5) if t > 0 else want
        assert dtr[0, 0, t, 0] == pytest.approx(want, rel=1e-12)
    # dtr[..., t, :] holds d_{t+1}: d_7 = 0.9^6 is the last value above 0.5
    for t in range(7):
        assert dtr[0, 0, t, 1] == pytest.approx(r ** t, rel=1e-12)
    assert np.all(dtr[0, 0, 7:, 1] == 0.5)


def test_p6_onehot_non_beta_aware(oracle_lib):
    """Appendix B, non-beta-aware phase 1: d_{t+1} = r d_t + eta (1 - <d_t,k^2>) k^2;
    for a one-hot key the fixed point is eta / (1 - r + eta) whatever beta is."""
    eta, r, T = 0.05, 0.95, 60
    k, b, rr = _onehot_stream(2, T, 0, 0.37, r)
    _, _, dtr = oracle.precond_scan(k, b, rr, eta=eta, beta_aware=False,
                                    clamp=False, trajectory=True)
    dstar = eta / (1 - r + eta)
    for t in range(T + 1):
        assert dtr[0, 0, t, 0] == pytest.approx(dstar + (r - eta) ** t * (1 - dstar), rel=1e-12)


# ---------------------------------------------------------------- P-7
def test_p7_worked_example_loss_ratio(oracle_lib):
    """The reading notes' teaching example (golden fixture): k=(1,0), beta=0.5,
    q=0.25 at d=(1,1) and 0.0625 at d=(1.5,1), read from the oracle's realised
    loss ratio f_t(S_t)/f_t(S_{t-1}) after one write from a random state."""
    with open(GOLDEN) as fh:
        g = json.load(fh)["residual_ratio_teaching_example"]
    rng = np.random.default_rng(7)
    k = np.array(g["k"])[None, None, None, :]
    bb = np.array([[[g["beta"]]]])
    for case in g["cases"]:
        d = np.array(case["d"])
        kt, _ = oracle.precond_scan(k, bb, d1=d[None, None, :], eta=0.0)
        v = rng.standard_normal((1, 1, 1, 3))
        S0 = rng.standard_normal((1, 1, 3, 2))
        _, _, Str, u = oracle.delta_rule(k, k, kt, v, bb, S0=S0, trajectory=True)
        diag = oracle.diagnostics(k, kt, v, bb, Str, u)
        assert diag[0, 0, 0, 4] == pytest.approx(case["q"], rel=1e-12)


def test_p7_one_step_update(oracle_lib):
    """One step of Eq.(4) by hand: k=(0.6,0.8), beta=0.5, eta=0.003, d=1:
    s=(0.36,0.64), n=1, <d,s>=1, c = 0.003*0.5*(1-0.5)/1 = 0.00075,
    d_2 = 1 + c s = (1.00027, 1.00048); the emitted write key is k itself."""
    k = np.array([0.6, 0.8])[None, None, None, :]
    kt, d = oracle.precond_scan(k, np.array([[[0.5]]]), eta=0.003)
    np.testing.assert_allclose(d[0, 0], [1.00027, 1.00048], rtol=1e-14)
    np.testing.assert_array_equal(kt[0, 0, 0], [0.6, 0.8])


# ---------------------------------------------------------------- P-8
def test_p8_exact_write_counterexample(oracle_lib):
    """Appendix D.4 (golden fixture): K=V=1, k_t=1, v_t=(-1)^t, beta=0.5, d_1=2:
    the phase-1 step is proportional to 1 - 0.5*2 = 0, so d stays 2, every write
    is exact and S_t = (-1)^t; also in float32 arithmetic."""
    with open(GOLDEN) as fh:
        g = json.load(fh)["exact_write_counterexample"]
    T = g["T"]
    k = np.ones((1, T, 1, 1))
    v = np.array([(-1.0) ** t for t in range(1, T + 1)])[None, :, None, None]
    bb = np.full((1, T, 1), 0.5)
    kt, d, dtr = oracle.precond_scan(k, bb, d1=np.full((1, 1, 1), 2.0), eta=0.003,
                                     trajectory=True)
    assert np.all(dtr == 2.0)
    o, S, Str, u = oracle.delta_rule(k, k, kt, v, bb, trajectory=True)
    np.testing.assert_array_equal(Str[0, 0, 1:, 0, 0], np.array(g["S_t"]))
    np.testing.assert_array_equal(o[0, :, 0, 0], np.array(g["S_t"]))


# ---------------------------------------------------------------- P-9
def test_p9_repeated_key_contraction(oracle_lib):
    """Corollary D.8: one-hot class keys on disjoint coordinates with fixed
    targets give prod_c F_c(S_T)/F_c(S_0) = prod_t q_t."""
    rng = np.random.default_rng(9)
    K, V, T = 4, 3, 40
    targets = rng.standard_normal((K, V))
    cls = np.concatenate([np.arange(K), rng.integers(0, K, T - K)])
    rng.shuffle(cls)
    k = np.zeros((1, T, 1, K))
    k[0, np.arange(T), 0, cls] = 1.0
    v = targets[cls][None, :, None, :]
    bb = (0.2 + 0.6 * rng.random((1, T, 1)))
    kt, _ = oracle.precond_scan(k, bb, eta=0.05)
    S0 = rng.standard_normal((1, 1, V, K))
    _, S, Str, u = oracle.delta_rule(k, k, kt, v, bb, S0=S0, trajectory=True)
    diag = oracle.diagnostics(k, kt, v, bb, Str, u)
    F = lambda Sm, c: 0.5 * np.sum((Sm @ np.eye(K)[c] - targets[c]) ** 2)
    lhs = np.prod([F(S[0, 0], c) / F(S0[0, 0], c) for c in range(K)])
    rhs = np.prod(diag[0, :, 0, 4])
    assert lhs == pytest.approx(rhs, rel=1e-9)


# ---------------------------------------------------------------- P-10
def test_p10_wy_product_identity():
    """Eq.(10): prod_{i=1..C}(I - beta_i k_i k~_i^T) (left to right) = I - W^T K~
    with W from Eqs.(8)-(9), by brute force at C <= 16."""
    rng = np.random.default_rng(10)
    for C in (1, 2, 5, 16):
        K = 7
        Km = rng.standard_normal((C, K)) / math.sqrt(K)
        Kt = Km * rng.uniform(0.5, 2.0, (C, K))
        beta = rng.uniform(0.05, 0.95, C)
        _, W, _ = chunk_model.wy_factors(Km, Kt, np.zeros((C, 1)), beta)
        P = np.eye(K)
        for i in range(C):
            P = P @ (np.eye(K) - beta[i] * np.outer(Km[i], Kt[i]))
        np.testing.assert_allclose(P, np.eye(K) - W.T @ Kt, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P-11
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("C", [1, 2, 3, 16, 64, 70])
def test_p11_chunkwise_equals_sequential(oracle_lib, C, gdn):
    """The chunk form (Eqs.(8)-(11); Eqs.(13)-(15) for the gated form) equals the
    token-by-token recurrence for any chunk size, including a partial last chunk
    (T = 70 is not a multiple of 16 or 64)."""
    rng = np.random.default_rng(11)
    c = rand_case(rng, B=1, T=70, H=2, K=8, V=5, apf=True, gdn=gdn)
    kt, _ = oracle.precond_scan(c["k"], c["beta"], c["r"], eta=0.1)
    S0 = rng.standard_normal((1, 2, 5, 8))
    o_seq, S_seq = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"], c["alpha"],
                                     S0=S0, q_scale=0.7)
    o_ch, S_ch = chunk_model.forward(c["q"], c["k"], kt, c["v"], c["beta"], c["alpha"],
                                     S0=S0, chunk=C, q_scale=0.7)
    np.testing.assert_allclose(o_ch, o_seq, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(S_ch, S_seq, rtol=1e-10, atol=1e-11)


def test_gated_transition_form(oracle_lib):
    """Appendix B.1 / Table 3 row 'Gated DeltaNet + Online Scaling':
    S_t = S_{t-1}(alpha_t (I - beta_t k_t k~_t^T)) + beta_t v_t k~_t^T equals the
    oracle's post-gate residual form."""
    rng = np.random.default_rng(12)
    c = rand_case(rng, B=1, T=20, H=1, K=5, V=4, gdn=True)
    kt, _ = oracle.precond_scan(c["k"], c["beta"], eta=0.2)
    S0 = rng.standard_normal((1, 1, 4, 5))
    o, S = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"], c["alpha"], S0=S0)
    Sm = S0[0, 0].copy()
    for t in range(20):
        kk, w, vv = c["k"][0, t, 0], kt[0, t, 0], c["v"][0, t, 0]
        a, bb = c["alpha"][0, t, 0], c["beta"][0, t, 0]
        Sm = Sm @ (a * (np.eye(5) - bb * np.outer(kk, w))) + bb * np.outer(vv, w)
        np.testing.assert_allclose(o[0, t, 0], Sm @ c["q"][0, t, 0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], Sm, rtol=1e-11, atol=1e-12)


def test_osdn_transition_form(oracle_lib):
    """Eq.(5): S_t = S_{t-1}(I - beta_t k_t k~_t^T) + beta_t v_t k~_t^T (read key
    on the left, write key on the right) equals the oracle's residual form."""
    rng = np.random.default_rng(13)
    c = rand_case(rng, B=1, T=20, H=1, K=5, V=4)
    kt, _ = oracle.precond_scan(c["k"], c["beta"], eta=0.3)
    o, S = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"])
    Sm = np.zeros((4, 5))
    for t in range(20):
        kk, w, vv, bb = c["k"][0, t, 0], kt[0, t, 0], c["v"][0, t, 0], c["beta"][0, t, 0]
        Sm = Sm @ (np.eye(5) - bb * np.outer(kk, w)) + bb * np.outer(vv, w)
    np.testing.assert_allclose(S[0, 0], Sm, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P-12
@pytest.mark.parametrize("gdn", [False, True])
def test_p12_state_passing(oracle_lib, gdn):
    """Carrying (d, S) from a run over [0, T1) into a run over [T1, T) gives the
    same outputs as one run over [0, T) (initial_d / initial_state of the
    paper's chunk interface; the prefill + decode check of Appendix L)."""
    rng = np.random.default_rng(14)
    c = rand_case(rng, B=2, T=33, H=2, K=6, V=4, apf=True, gdn=gdn)
    T1 = 19
    full = oracle.forward(c["q"], c["k"], c["v"], c["beta"], c["r"], c["alpha"], eta=0.1)
    sl = lambda x, a, b: None if x is None else x[:, a:b]
    p1 = oracle.forward(*(sl(c[n], 0, T1) for n in ("q", "k", "v", "beta", "r", "alpha")),
                        eta=0.1)
    p2 = oracle.forward(*(sl(c[n], T1, 33) for n in ("q", "k", "v", "beta", "r", "alpha")),
                        d1=p1["d"], S0=p1["S"], eta=0.1)
    np.testing.assert_allclose(np.concatenate([p1["k_tilde"], p2["k_tilde"]], 1),
                               full["k_tilde"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(np.concatenate([p1["o"], p2["o"]], 1), full["o"],
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p2["S"], full["S"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p2["d"], full["d"], rtol=1e-13)


# ---------------------------------------------------------------- P-13
def test_p13_neutral_gates(oracle_lib):
    """r = 1 recovers Eq.(4) (Section 4.4), alpha = 1 recovers OSDN (Table 3),
    and beta_aware=0 is the beta-aware update with beta' = 1 in phase 1 only
    (Appendix B; the memory write keeps beta)."""
    rng = np.random.default_rng(15)
    c = rand_case(rng, B=1, T=25, H=2, K=6, V=3)
    ones = np.ones_like(c["beta"])
    a = oracle.precond_scan(c["k"], c["beta"], None, eta=0.1)
    b = oracle.precond_scan(c["k"], c["beta"], ones, eta=0.1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    o1, S1 = oracle.delta_rule(c["q"], c["k"], a[0], c["v"], c["beta"])
    o2, S2 = oracle.delta_rule(c["q"], c["k"], a[0], c["v"], c["beta"], ones)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    nb = oracle.precond_scan(c["k"], c["beta"], eta=0.1, beta_aware=False)
    b1 = oracle.precond_scan(c["k"], ones, eta=0.1, beta_aware=True)
    assert np.array_equal(nb[0], b1[0]) and np.array_equal(nb[1], b1[1])
    assert not np.allclose(nb[1], a[1])


# ---------------------------------------------------------------- P-14
def test_p14_unit_step_replaces_value(oracle_lib):
    """Appendix A.1: beta=1 with a unit key and d=1 replaces the value exactly:
    S_t k_t = v_t after each write."""
    rng = np.random.default_rng(16)
    c = rand_case(rng, B=1, T=15, H=1, K=7, V=5)
    bb = np.ones_like(c["beta"])
    kt, _ = oracle.precond_scan(c["k"], bb, eta=0.0)
    _, _, Str, _ = oracle.delta_rule(c["q"], c["k"], kt, c["v"], bb, trajectory=True)
    for t in range(15):
        np.testing.assert_allclose(Str[0, 0, t + 1] @ c["k"][0, t, 0], c["v"][0, t, 0],
                                   atol=1e-14)


# ---------------------------------------------------------------- edge cases
def test_zero_key_and_eps(oracle_lib):
    """A zero key: n is floored at eps (Eq.(4)), s = 0 so d moves only by the
    retention, the write key is 0 and the state is not written."""
    rng = np.random.default_rng(17)
    c = rand_case(rng, B=1, T=6, H=1, K=4, V=3, apf=True)
    c["k"][0, 3, 0] = 0.0
    kt, d, dtr = oracle.precond_scan(c["k"], c["beta"], c["r"], eta=0.5, trajectory=True)
    assert np.all(kt[0, 3, 0] == 0.0)
    np.testing.assert_allclose(dtr[0, 0, 4], np.clip(c["r"][0, 3, 0] * dtr[0, 0, 3], 0.5, 2.0),
                               rtol=1e-15)
    _, _, Str, _ = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"], trajectory=True)
    np.testing.assert_array_equal(Str[0, 0, 4], Str[0, 0, 3])


def test_q_scale_is_linear(oracle_lib):
    """The query scale (the paper's chunk listing multiplies q by K^-1/2; the
    main text reads o_t = S_t q_t) only rescales the readout."""
    rng = np.random.default_rng(18)
    c = rand_case(rng, B=1, T=12, H=2, K=4, V=3)
    kt, _ = oracle.precond_scan(c["k"], c["beta"], eta=0.1)
    o1, S1 = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"])
    o2, S2 = oracle.delta_rule(c["q"], c["k"], kt, c["v"], c["beta"], q_scale=0.5)
    np.testing.assert_allclose(o2, 0.5 * o1, rtol=1e-14)
    assert np.array_equal(S1, S2)


def test_empty_sequence(oracle_lib):
    """T = 0: nothing is emitted, d and S come back unchanged."""
    k = np.zeros((2, 0, 3, 4))
    d1 = np.full((2, 3, 4), 1.5)
    kt, d = oracle.precond_scan(k, np.zeros((2, 0, 3)), d1=d1)
    assert kt.shape == (2, 0, 3, 4) and np.array_equal(d, d1)
    S0 = np.ones((2, 3, 5, 4))
    o, S = oracle.delta_rule(k, k, k, np.zeros((2, 0, 3, 5)), np.zeros((2, 0, 3)), S0=S0)
    assert o.shape == (2, 0, 3, 5) and np.array_equal(S, S0)


# ---------------------------------------------------------------- P-16
def test_p16_bf16_rounding_matches_torch():
    """The input generator's bf16 rounding is round-to-nearest-even, checked
    against torch's float32 -> bfloat16 conversion on random and tie values."""
    import torch
    rng = np.random.default_rng(19)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 3,
                        np.array([1.00390625, 1.01171875, -2.00781250, 0.0, -0.0], np.float32)])
    ours = bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
