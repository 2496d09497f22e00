"""GPU parity of the decode step (osdn_decode: the single-token recurrence of
the paper's Appendix L, up to 64 new tokens per call from a carried (d, S))
against the CPU oracle, plus the prefill + decode check of the same appendix.

The decode kernel keeps S and the write keys in fp32, so its state is held to
the fp32 bar even for bf16 inputs; bf16 readouts are rounded once on store and
are held to the bf16 bar.
"""
import numpy as np
import pytest

import oracle
import preconditioned_delta_rule_amd as osdn
from tests.helpers import (BF16_OS, F32_D, F32_OS, check_bf16_readout, o_err, rel_err, rms_err, s_err,
                           to_dev, to_np)
from workloads import make_inputs, random_state

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    osdn.load()
    yield
    torch.cuda.synchronize()


def spec(**kw):
    base = dict(B=2, T=8, H=3, K=128, V=128, dtype="f32", seed=21, apf=True)
    base.update(kw)
    return base


CASES = {
    "t1": spec(B=3, H=4, T=1),
    "t16_gdn": spec(T=16, gdn=True),
    "t37_ragged_blocks": spec(B=1, T=37),
    "t64_max": spec(B=1, H=2, T=64, gdn=True, q_scale="rsqrt_k"),
    "k16": spec(K=16, V=16, T=20, apf=False),
    "k33_v37_scalar_rows": spec(K=33, V=37, T=20, gdn=True),
    "k100_v64": spec(K=100, V=64, T=9),
    "k1_v1": spec(K=1, V=1, T=12),
    "v8_k128": spec(K=128, V=8, T=5),
    "non_beta_aware": spec(K=32, V=32, T=40, beta_aware=False, eta=0.05),
    "no_clamp": spec(K=32, V=32, T=40, clamp=False, eta=0.2),
    "clamp_hi": spec(K=16, V=16, T=64, keys="onehot", onehot_bias=0.6, eta=0.3, beta_mu=-1.5,
                     apf=False),
    "apf_to_dmin": spec(K=16, V=16, T=64, keys="sparse", apf_const=0.9, eta=0.05, apf=False),
}


def with_state(inp, seed=0, s_scale=0.3):
    d1, S0 = random_state(inp, seed=seed, s_scale=s_scale)
    return dict(inp, d1=d1, S0=S0)


def run_decode(inp, dtype=None, o_f32=False, **over):
    p = dict(inp["params"])
    p.update(over)
    dt = dtype or p["dtype"]
    o, S, d = osdn.decode(to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
                          to_dev(inp["beta"], "f32"), to_dev(inp["r"], "f32"),
                          to_dev(inp["alpha"], "f32"), to_dev(inp["d1"], "f32"),
                          to_dev(inp["S0"], "f32"), eta=p["eta"], d_min=p["d_min"],
                          d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
                          q_scale=p["q_scale"], beta_aware=p["beta_aware"], o_f32=o_f32)
    torch.cuda.synchronize()
    return to_np(o), to_np(S), to_np(d)


def oracle_fwd(inp):
    p = inp["params"]
    return oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["r"], inp["alpha"],
                          inp["d1"], inp["S0"], eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"],
                          clamp=p["clamp"], eps=p["eps"], beta_aware=p["beta_aware"],
                          q_scale=p["q_scale"])


def check(o, S, d, ref, dtype, tag, o32=None):
    """d and the fp32 state within the fp32 bars (decode keeps every
    intermediate in fp32); the readout within the bar of its dtype (for bf16:
    the fp32 readout o32 of the same call tensor-wide, the bf16 one its
    nearest-even rounding)."""
    assert rel_err(d, ref["d"]) <= F32_D, (tag, rel_err(d, ref["d"]))
    assert rel_err(S, ref["S"]) <= F32_OS, (tag, rel_err(S, ref["S"]))
    if dtype == "f32":
        assert rel_err(o, ref["o"]) <= F32_OS, (tag, rel_err(o, ref["o"]))
    else:
        check_bf16_readout(o, o32, ref["o"], tag)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_parity(case, dtype):
    inp = with_state(make_inputs(dict(CASES[case], dtype=dtype)), seed=3)
    o, S, d = run_decode(inp)
    o32 = run_decode(inp, o_f32=True)[0] if dtype == "bf16" else None
    ref = oracle_fwd(inp)
    check(o, S, d, ref, dtype, case, o32)
    if case == "clamp_hi":
        assert np.any(ref["d"] == 2.0)
    if case == "apf_to_dmin":
        assert np.any(ref["d"] == 0.5)


@pytest.mark.parametrize("gated", [False, True], ids=["osdn", "gdn"])
def test_prefill_then_decode_matches_forward(gated):
    """Appendix L's layer check: prefill 128 tokens with osdn_fwd, decode token
    129 from the carried (S, d); the result matches one forward over 129
    tokens (oracle and GPU chunk path)."""
    inp = make_inputs(dict(B=2, T=129, H=4, K=128, V=128, dtype="bf16", chunk=64, seed=41,
                           apf=True, gdn=gated))
    p = inp["params"]
    dev = lambda n, dt="bf16": to_dev(inp[n], dt)
    cut = lambda x, a, b: None if x is None else x[:, a:b].contiguous()
    q, k, v = dev("q"), dev("k"), dev("v")
    beta, r, alpha = dev("beta", "f32"), dev("r", "f32"), dev("alpha", "f32")
    kw = dict(eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
              q_scale=p["q_scale"], beta_aware=p["beta_aware"])
    o_pre, S, d = osdn.fwd(cut(q, 0, 128), cut(k, 0, 128), cut(v, 0, 128), cut(beta, 0, 128),
                           cut(r, 0, 128), cut(alpha, 0, 128), chunk=64, **kw)
    # state updated in place
    o_dec, S2, d2 = osdn.decode(cut(q, 128, 129), cut(k, 128, 129), cut(v, 128, 129),
                                cut(beta, 128, 129), cut(r, 128, 129), cut(alpha, 128, 129),
                                d, S, S_out=S, d_out=d, **kw)
    o_full, S_full, d_full = osdn.fwd(q, k, v, beta, r, alpha, chunk=64, **kw)
    # the same decode step from the carried state, with an fp32 readout
    _, S_pre, d_pre = osdn.fwd(cut(q, 0, 128), cut(k, 0, 128), cut(v, 0, 128), cut(beta, 0, 128),
                               cut(r, 0, 128), cut(alpha, 0, 128), chunk=64, **kw)
    o_dec32, _, _ = osdn.decode(cut(q, 128, 129), cut(k, 128, 129), cut(v, 128, 129),
                                cut(beta, 128, 129), cut(r, 128, 129), cut(alpha, 128, 129),
                                d_pre, S_pre, o_f32=True, **kw)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr() and d2.data_ptr() == d.data_ptr()
    ref = oracle_fwd(inp)
    o_dec, S2, d2 = to_np(o_dec), to_np(S2), to_np(d2)
    check_bf16_readout(o_dec, to_np(o_dec32), ref["o"][:, 128:], "prefill+decode")
    assert o_err(o_dec, ref["o"][:, 128:]) <= BF16_OS
    assert s_err(S2, ref["S"]) <= BF16_OS
    assert rms_err(S2, ref["S"]) <= BF16_OS
    assert rel_err(d2, ref["d"]) <= F32_D
    assert o_err(o_dec, to_np(o_full)[:, 128:]) <= BF16_OS
    assert s_err(S2, to_np(S_full)) <= BF16_OS
    assert rel_err(d2, to_np(d_full)) <= F32_D


def test_token_by_token_equals_one_call():
    """Eight single-token calls carrying the state in place give bit for bit
    the outputs of one eight-token call (same arithmetic, same order)."""
    inp = with_state(make_inputs(spec(B=2, H=2, T=8, dtype="bf16", gdn=True)), seed=5)
    dt = "bf16"
    q, k, v = (to_dev(inp[n], dt) for n in ("q", "k", "v"))
    beta, r, alpha = (to_dev(inp[n], "f32") for n in ("beta", "r", "alpha"))
    o1, S1, d1 = osdn.decode(q, k, v, beta, r, alpha, to_dev(inp["d1"], "f32"),
                             to_dev(inp["S0"], "f32"))
    S, d = to_dev(inp["S0"], "f32"), to_dev(inp["d1"], "f32")
    outs = []
    for t in range(8):
        sl = lambda x: x[:, t:t + 1].contiguous()
        o, _, _ = osdn.decode(sl(q), sl(k), sl(v), sl(beta), sl(r), sl(alpha), d, S,
                              S_out=S, d_out=d)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, 1), o1)
    assert torch.equal(S, S1) and torch.equal(d, d1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_empty(dtype):
    """T = 0: d_out = d1 and S_out = S0, nothing else is touched."""
    K, V = 128, 96
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    z = torch.zeros((2, 0, 3, K), device="cuda:0", dtype=tdt)
    d1 = torch.rand((2, 3, K), device="cuda:0") + 0.5
    S0 = torch.randn((2, 3, V, K), device="cuda:0")
    o, S, d = osdn.decode(z, z, torch.zeros((2, 0, 3, V), device="cuda:0", dtype=tdt),
                          torch.zeros((2, 0, 3), device="cuda:0"), d1=d1, S0=S0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, V)
    assert torch.equal(d, d1) and torch.equal(S, S0)


def test_decode_defaults_equal_forward_start():
    """Without d1 and S0 the decode step starts from d = 1, S = 0, like
    osdn_fwd: a short sequence gives the oracle's forward."""
    inp = make_inputs(spec(B=2, H=2, T=10, dtype="f32"))
    o, S, d = run_decode(inp)
    check(o, S, d, oracle_fwd(inp), "f32", "defaults")


def test_decode_exact_write_counterexample():
    """Appendix D.4: K=V=1, k=1, v=(-1)^t, beta=0.5, d_1=2 keeps d = 2 and
    gives S_t = (-1)^t exactly; decoded in two calls it is reproduced bit for
    bit."""
    T = 32
    k = np.ones((1, T, 1, 1), np.float32)
    v = np.array([(-1.0) ** t for t in range(1, T + 1)], np.float32)[None, :, None, None]
    beta = np.full((1, T, 1), 0.5, np.float32)
    kt, vt, bt = to_dev(k, "f32"), to_dev(v, "f32"), to_dev(beta, "f32")
    S = torch.zeros((1, 1, 1, 1), device="cuda:0")
    d = torch.full((1, 1, 1), 2.0, device="cuda:0")
    outs = []
    for a, b in ((0, 20), (20, 32)):
        o, _, _ = osdn.decode(kt[:, a:b].contiguous(), kt[:, a:b].contiguous(),
                              vt[:, a:b].contiguous(), bt[:, a:b].contiguous(), d1=d, S0=S,
                              S_out=S, d_out=d)
        outs.append(o)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(torch.cat(outs, 1))[0, :, 0, 0], v[0, :, 0, 0])
    assert d.item() == 2.0 and S.item() == 1.0


DECODE_FULL = ["decode_1p3b", "decode_1p3b_b256"]


@pytest.mark.parametrize("name", DECODE_FULL)
def test_decode_full_size(name):
    """The decode workloads the bench times (one new token per sequence), in
    the same launch; every (b,h) sequence against the oracle."""
    inp = make_inputs(name)
    o, S, d = run_decode(inp)
    o32 = run_decode(inp, o_f32=True)[0]
    ref = oracle_fwd(inp)
    check(o, S, d, ref, "bf16", name, o32)


def test_decode_rejects_long_input():
    q = torch.zeros((1, osdn.DECODE_MAX_T + 1, 1, 16), device="cuda:0")
    with pytest.raises(osdn.OsdnError, match="at most"):
        osdn.decode(q, q, q, torch.zeros((1, osdn.DECODE_MAX_T + 1, 1), device="cuda:0"))
