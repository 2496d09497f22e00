"""Pins of the oracle's backward pass (oracle/osdn_oracle_bwd.c).

Every gradient the oracle returns is checked against central finite
differences of the forward oracle (a separate code path: osdn_oracle.c), for
the scalar loss L = <Wo, o> + <WS, S_T> + <Wd, d_{T+1}> with random weights,
on tiny inputs: every input element (q, k, v, beta, r, alpha, d1, S0), cases
with the box clamp active and inactive, without clamp, non-beta-aware, gated
with retention, a key below the norm floor, and a sequence long enough to
cross the oracle's 64-token recomputation stretches.  The clamp and the norm
floor make the forward piecewise smooth; the cases keep every step at least
1e-4 away from a kink so that the differences see one smooth piece.
"""
import numpy as np
import pytest

import oracle

H_FD = 1e-6


def _forward_loss(inp, p, W):
    f = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp.get("r"), inp.get("alpha"),
                       inp.get("d1"), inp.get("S0"), eta=p["eta"], d_min=p["d_min"],
                       d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
                       beta_aware=p["beta_aware"], q_scale=p["q_scale"], threads=1)
    return float(np.sum(W["o"] * f["o"]) + np.sum(W["S"] * f["S"]) + np.sum(W["d"] * f["d"]))


def _kink_margin(inp, p):
    """Smallest distance of any step's pre-clip value y to a box bound, the
    smallest distance of any key's squared norm to the floor (the forward's
    kinks), and the number of clipped coordinates."""
    k, beta = inp["k"], inp["beta"]
    B, T, H, K = k.shape
    r = inp.get("r")
    _, _, traj = oracle.precond_scan(k, beta, r, inp.get("d1"), eta=p["eta"], d_min=p["d_min"],
                                     d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
                                     beta_aware=p["beta_aware"], trajectory=True, threads=1)
    margin, nmargin, clipped = np.inf, np.inf, 0
    for b in range(B):
        for h in range(H):
            for t in range(T):
                d = traj[b, h, t]
                s = k[b, t, h] ** 2
                nraw = s.sum()
                nmargin = min(nmargin, abs(nraw - p["eps"]))
                bp = beta[b, t, h] if p["beta_aware"] else 1.0
                c = p["eta"] * bp * (1 - bp * np.dot(d, s)) / max(nraw, p["eps"])
                y = (r[b, t, h] if r is not None else 1.0) * d + c * s
                if p["clamp"]:
                    margin = min(margin, np.min(np.abs(y - p["d_min"])), np.min(np.abs(y - p["d_max"])))
                    clipped += int(np.sum((y < p["d_min"]) | (y > p["d_max"])))
    return margin, nmargin, clipped


def make_case(name):
    rng = np.random.default_rng({"plain": 1, "clamp_active": 2, "gated_apf": 3, "no_clamp": 4,
                                 "tiny_key": 5, "long": 6}[name])
    p = dict(eta=0.3, d_min=0.5, d_max=2.0, clamp=True, eps=1e-6, beta_aware=True, q_scale=1.0)
    B, T, H, K, V = 1, 9, 2, 3, 2
    if name == "long":
        T, H, K, V = 150, 1, 2, 2
    inp = {}
    inp["q"] = rng.standard_normal((B, T, H, K))
    inp["k"] = rng.standard_normal((B, T, H, K)) / np.sqrt(K)
    inp["v"] = rng.standard_normal((B, T, H, V))
    inp["beta"] = rng.uniform(0.2, 0.9, (B, T, H))
    inp["d1"] = rng.uniform(0.8, 1.6, (B, H, K))
    inp["S0"] = 0.5 * rng.standard_normal((B, H, V, K))
    if name == "plain":
        p.update(d_min=0.05, d_max=20.0)  # box never reached
    if name == "clamp_active":
        inp["r"] = rng.uniform(0.6, 0.9, (B, T, H))
        p.update(eta=1.5)
    if name == "gated_apf":
        inp["r"] = rng.uniform(0.85, 1.0, (B, T, H))
        inp["alpha"] = rng.uniform(0.7, 1.0, (B, T, H))
        p.update(beta_aware=False, q_scale=0.5)
    if name == "no_clamp":
        p.update(clamp=False, eta=0.8)
    if name == "tiny_key":
        inp["k"][0, 4, 0] = 1e-4 * np.array([1.0, -2.0, 0.5])  # squared norm 5e-8, below eps
    if name == "long":
        inp["r"] = rng.uniform(0.9, 1.0, (B, T, H))
        inp["alpha"] = rng.uniform(0.9, 1.0, (B, T, H))
        p.update(eta=0.1)
    W = {"o": rng.standard_normal((B, T, H, V)), "S": rng.standard_normal((B, H, V, K)),
         "d": rng.standard_normal((B, H, K))}
    return inp, p, W


CASES = ["plain", "clamp_active", "gated_apf", "no_clamp", "tiny_key", "long"]
GRAD = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "r": "dr", "alpha": "dalpha",
        "d1": "dd1", "S0": "dS0"}


def fd_errors(name, sample=None):
    """Largest |analytic - finite difference| / max(1, |fd|) per input."""
    inp, p, W = make_case(name)
    margin, nmargin, clipped = _kink_margin(inp, p)
    # a difference step moves y by at most ~1e-6 and a squared norm by 2 |k| 1e-6
    assert margin > 1e-4 and nmargin > 1e-8, (name, margin, nmargin)
    if name == "clamp_active":
        assert clipped > 0
    g = oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp.get("r"), inp.get("alpha"),
                        inp.get("d1"), inp.get("S0"), dout=W["o"], dS=W["S"], dd=W["d"],
                        eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
                        eps=p["eps"], beta_aware=p["beta_aware"], q_scale=p["q_scale"], threads=1)
    rng = np.random.default_rng(99)
    errs = {}
    for key, gname in GRAD.items():
        if key not in inp:
            continue
        x = inp[key]
        idx = list(np.ndindex(x.shape))
        if sample is not None and len(idx) > sample:
            idx = [idx[i] for i in rng.choice(len(idx), sample, replace=False)]
        worst = 0.0
        for ix in idx:
            save = x[ix]
            x[ix] = save + H_FD
            lp = _forward_loss(inp, p, W)
            x[ix] = save - H_FD
            lm = _forward_loss(inp, p, W)
            x[ix] = save
            fd = (lp - lm) / (2 * H_FD)
            worst = max(worst, abs(g[gname][ix] - fd) / max(1.0, abs(fd)))
        errs[key] = worst
    return errs


@pytest.mark.parametrize("name", CASES)
def test_backward_matches_finite_differences(name):
    errs = fd_errors(name, sample=24 if name == "long" else None)
    assert max(errs.values()) < 1e-6, errs


def test_backward_linear_in_upstream_gradients():
    """The backward is linear in (dout, dS, dd): a property of any VJP, which
    catches a term computed from the wrong upstream gradient."""
    inp, p, W = make_case("gated_apf")
    kw = dict(eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
              beta_aware=p["beta_aware"], q_scale=p["q_scale"], threads=1)
    args = (inp["q"], inp["k"], inp["v"], inp["beta"], inp["r"], inp["alpha"], inp["d1"], inp["S0"])
    g1 = oracle.backward(*args, dout=W["o"], dS=None, dd=None, **kw)
    g2 = oracle.backward(*args, dout=np.zeros_like(W["o"]), dS=W["S"], dd=W["d"], **kw)
    g12 = oracle.backward(*args, dout=W["o"], dS=W["S"], dd=W["d"], **kw)
    for key in g12:
        if g12[key] is not None:
            assert np.allclose(g12[key], g1[key] + g2[key], rtol=1e-12, atol=1e-12), key


def test_backward_empty_sequence():
    """T = 0: the gradients of the initial state are the upstream ones."""
    rng = np.random.default_rng(0)
    z = np.zeros((2, 0, 3, 4))
    dS = rng.standard_normal((2, 3, 5, 4))
    dd = rng.standard_normal((2, 3, 4))
    g = oracle.backward(z, z, np.zeros((2, 0, 3, 5)), np.zeros((2, 0, 3)),
                        dout=np.zeros((2, 0, 3, 5)), dS=dS, dd=dd)
    assert np.array_equal(g["dS0"], dS) and np.array_equal(g["dd1"], dd)
