"""GPU parity of the OSKDA forward (osdn_kda_fwd: Appendix B.2, the online-scaled
KDA row of Table 3) and of vector retention (Proposition A.3) against the
oracle, on the same seeded inputs, through the C ABI.

Bars as for the OSDN forward: fp32 inputs within 1e-4 (o, S) and 1e-5 (d),
relative with an RMS floor; bf16 inputs within 2e-2 of the per-row / per-head
RMS for o and S.  The chunk operands are fp32 on the device, so fp32 cases are
held to the fp32 bar.
"""
import numpy as np
import pytest

import oracle
import preconditioned_delta_rule_amd as osdn
from tests.helpers import (F32_D, F32_OS, check_bf16_readout, check_bf16_state, rel_err, to_dev,
                           to_np)
from workloads import make_inputs

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
    base = dict(B=2, T=130, H=2, K=128, V=128, seed=71, kda=True, apf=True)
    base.update(kw)
    return base


CASES = {
    "k128": spec(),
    "k128_t1": spec(T=1),
    "k128_t64": spec(T=64, B=1),
    "k128_t65": spec(T=65, B=1),
    "k128_t200_rsqrt": spec(T=200, B=1, q_scale="rsqrt_k"),
    "k16": spec(K=16, V=16, T=70),
    "k33_v37": spec(K=33, V=37, T=90),
    "k100_v64": spec(K=100, V=64, T=67),
    "k64_v128": spec(K=64, V=128, T=100),
    "no_decay": spec(kda=False),
    "no_retention": spec(apf=False, T=100),
    "strong_decay": spec(kda_decay=3.0, T=150),       # every chunk takes the exact path
    "mixed_decay": spec(kda_decay=0.9, T=200),        # some chunks exact, some factorised
    "vector_retention": spec(apf=True, r_vec=True, T=140),
    "non_beta_aware": spec(beta_aware=False, eta=0.05, T=100),
    "no_clamp": spec(clamp=False, eta=0.2, T=100),
}


def kda_state(inp, seed):
    """d1 ~ U(0.6, 1.9) [B,H,K] and S0 ~ 0.3 N(0,1) [B,H,K,V] (KDA layout)."""
    B, _, H, K = inp["k"].shape
    V = inp["v"].shape[-1]
    rng = np.random.default_rng(seed)
    d1 = rng.uniform(0.6, 1.9, (B, H, K)).astype(np.float32)
    S0 = (0.3 * rng.standard_normal((B, H, K, V))).astype(np.float32)
    return d1, S0


def run_kda(inp, d1, S0, k_tilde=False, o_f32=False):
    p = inp["params"]
    dt = p["dtype"]
    q, k, v = (to_dev(inp[n], dt) for n in ("q", "k", "v"))
    kt = torch.empty_like(k) if k_tilde else None
    o, S, d = osdn.kda_fwd(q, k, v, to_dev(inp["beta"], "f32"), to_dev(inp["r"], "f32"),
                           to_dev(inp["alpha"], "f32"), to_dev(d1, "f32"), to_dev(S0, "f32"),
                           eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
                           eps=p["eps"], q_scale=p["q_scale"], beta_aware=p["beta_aware"],
                           k_tilde_out=kt, o_f32=o_f32)
    torch.cuda.synchronize()
    return to_np(o), to_np(S), to_np(d), (to_np(kt) if k_tilde else None)


def oracle_kda(inp, d1, S0):
    p = inp["params"]
    return oracle.kda_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["r"], inp["alpha"], d1,
                              S0, eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"],
                              clamp=p["clamp"], eps=p["eps"], beta_aware=p["beta_aware"],
                              q_scale=p["q_scale"])


def check(o, S, d, ref, dtype, tag, o32=None):
    """fp32: every output within the fp32 bars.  bf16: the fp32 readout o32
    of the same call within 2e-2 tensor-wide, the bf16 readout its
    nearest-even rounding (and 2e-2 per row), the state 2e-2 tensor-wide and
    per head."""
    ed = rel_err(d, ref["d"])
    assert ed <= F32_D, (tag, ed)
    if dtype == "f32":
        eo, es = rel_err(o, ref["o"]), rel_err(S, ref["S"])
        print(tag, "o %.2e S %.2e d %.2e" % (eo, es, ed))
        assert eo <= F32_OS and es <= F32_OS, (tag, eo, es)
    else:
        check_bf16_readout(o, o32, ref["o"], tag)
        check_bf16_state(S, ref["S"], tag)


BF16_KEYS_LIMIT = pytest.mark.xfail(
    strict=True, reason="without the box the write keys cross the phases in bf16 (2^-9 relative "
    "error each); the final state reaches 2.05e-2 tensor-wide on this case")


@pytest.mark.parametrize("dtype,case", [(dt, c) if (dt, c) != ("bf16", "no_clamp")
                                        else pytest.param(dt, c, marks=BF16_KEYS_LIMIT)
                                        for dt in ("f32", "bf16") for c in sorted(CASES)])
def test_kda_parity(case, dtype):
    inp = make_inputs(dict(CASES[case], dtype=dtype))
    d1, S0 = kda_state(inp, seed=5)
    o, S, d, _ = run_kda(inp, d1, S0)
    o32 = run_kda(inp, d1, S0, o_f32=True)[0] if dtype == "bf16" else None
    check(o, S, d, oracle_kda(inp, d1, S0), dtype, case, o32)


def test_kda_defaults_without_state():
    """No d1, S0 (ones, zeros), no retention, no decay."""
    inp = make_inputs(spec(kda=False, apf=False, dtype="f32", T=100))
    o, S, d, _ = run_kda(inp, None, None)
    check(o, S, d, oracle_kda(inp, None, None), "f32", "defaults")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kda_k_tilde_out(dtype):
    inp = make_inputs(spec(dtype=dtype, T=100))
    d1, S0 = kda_state(inp, seed=6)
    o, S, d, kt = run_kda(inp, d1, S0, k_tilde=True)
    o32 = run_kda(inp, d1, S0, k_tilde=True, o_f32=True)[0] if dtype == "bf16" else None
    ref = oracle_kda(inp, d1, S0)
    check(o, S, d, ref, dtype, "k_tilde_out", o32)
    if dtype == "f32":
        assert rel_err(kt, ref["k_tilde"]) <= 1e-5
    else:
        # rounded once to bf16: within one bf16 ulp of the fp64 write key
        assert np.all(np.abs(kt - ref["k_tilde"]) <= np.maximum(np.abs(ref["k_tilde"]) * 2.0 ** -8, 1e-30))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kda_empty_sequence(dtype):
    """T = 0: S_out = S0 and d_out = d1."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    z = torch.zeros((2, 0, 3, 32), device="cuda:0", dtype=tdt)
    zv = torch.zeros((2, 0, 3, 48), device="cuda:0", dtype=tdt)
    d1 = torch.rand((2, 3, 32), device="cuda:0") + 0.5
    S0 = torch.randn((2, 3, 32, 48), device="cuda:0")
    o, S, d = osdn.kda_fwd(z, z, zv, torch.zeros((2, 0, 3), device="cuda:0"), d1=d1, S0=S0)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(d, d1)


def test_kda_without_decay_matches_osdn_transposed():
    """With alpha = None OSKDA is OSDN with the state transposed: the two GPU
    paths (different kernels) agree to the fp32 bar."""
    inp = make_inputs(spec(kda=False, dtype="f32", T=150))
    d1, S0 = kda_state(inp, seed=7)
    o, S, d, _ = run_kda(inp, d1, S0)
    p = inp["params"]
    o2, S2, d2 = osdn.fwd(*(to_dev(inp[n], "f32") for n in ("q", "k", "v", "beta", "r")), None,
                          to_dev(d1, "f32"), to_dev(np.swapaxes(S0, -1, -2), "f32"), eta=p["eta"],
                          d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
                          q_scale=p["q_scale"], beta_aware=p["beta_aware"])
    torch.cuda.synchronize()
    assert rel_err(o, to_np(o2)) <= F32_OS
    assert rel_err(S, np.swapaxes(to_np(S2), -1, -2)) <= F32_OS
    assert np.array_equal(d, to_np(d2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_osdn_fwd_vector_retention(dtype):
    """osdn_fwd and osdn_precond_scan with vector retention (r [B,T,H,K])."""
    inp = make_inputs(dict(B=2, T=150, H=2, K=128, V=128, seed=72, apf=True, r_vec=True, gdn=True,
                           dtype=dtype))
    p = inp["params"]
    args = [to_dev(inp[n], dtype) for n in ("q", "k", "v")]
    args += [to_dev(inp[n], "f32") for n in ("beta", "r", "alpha")]
    kw = dict(eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
              beta_aware=p["beta_aware"])
    o, S, d = osdn.fwd(*args, **kw, q_scale=p["q_scale"])
    o32 = osdn.fwd(*args, **kw, q_scale=p["q_scale"], o_f32=True)[0]
    kt, d_p1 = osdn.precond_scan(args[1], args[3], args[4], **kw)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["r"], inp["alpha"], **kw,
                         q_scale=p["q_scale"])
    check(to_np(o), to_np(S), to_np(d), ref, dtype, "fwd_vector_retention", to_np(o32))
    assert rel_err(to_np(d_p1), ref["d"]) <= F32_D


def test_vector_retention_unsupported_paths():
    inp = make_inputs(dict(B=1, T=8, H=1, K=16, V=16, seed=73, apf=True, r_vec=True))
    args = [to_dev(inp[n], "f32") for n in ("q", "k", "v", "beta", "r")]
    with pytest.raises(osdn.OsdnError) as e:
        osdn.decode(*args)
    assert e.value.status == osdn.EUNSUPPORTED


def test_kda_full_size():
    """The bench's OSKDA workload (B=8, T=2048, H=8, K=V=128, bf16, APF,
    channel-wise decay) in one call; every head against the oracle."""
    inp = make_inputs("kda_340m_apf")
    o, S, d, _ = run_kda(inp, None, None)
    o32 = run_kda(inp, None, None, o_f32=True)[0]
    check(o, S, d, oracle_kda(inp, None, None), "bf16", "kda_340m_apf", o32)


@pytest.mark.parametrize("case", ["k128", "no_retention", "strong_decay"])
def test_kda_folded_residual_is_bitwise_the_emitted_one(case):
    """bf16, K = 128 without k_tilde_out: the intra pass forms the write-key
    residual from the phase-1 marks and step scalars; with k_tilde_out the
    phase-1 emit kernel writes it.  Both give the same bits."""
    inp = make_inputs(dict(CASES[case], dtype="bf16"))
    d1, S0 = kda_state(inp, seed=9)
    o1, S1, dd1, _ = run_kda(inp, d1, S0)
    o2, S2, dd2, _ = run_kda(inp, d1, S0, k_tilde=True)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2) and np.array_equal(dd1, dd2), case
