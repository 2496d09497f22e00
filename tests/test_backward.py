"""GPU parity of the backward pass (osdn_bwd) against the oracle's backward
(oracle/osdn_oracle_bwd.c, itself pinned by finite differences of the forward
oracle), on the same seeded inputs and upstream gradients.

The kernels compute in fp32 throughout, so every fp32 output (and every
output for fp32 inputs) is held to the fp32 bar of the forward's o and S
(1e-4, relative with an RMS floor); gradients stored in bf16 (dq, dk, dv for
bf16 inputs) are rounded once on store and held to the bf16 bar.
"""
import numpy as np
import pytest

import oracle
import preconditioned_delta_rule_amd as osdn
from tests.helpers import BF16_OS, F32_OS, check_bf16_readout, rel_err, to_dev, to_np
from workloads import make_inputs, random_cotangent, random_state, sample_sequences

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
    base = dict(B=2, T=40, H=2, K=16, V=16, dtype="f32", seed=51, apf=True)
    base.update(kw)
    return base


CASES = {
    "k16": spec(),
    "k16_gdn": spec(gdn=True),
    "k128_t37": spec(B=1, T=37, K=128, V=128),
    "k128_t70_gdn": spec(B=1, T=70, K=128, V=128, gdn=True, q_scale="rsqrt_k"),
    "k33_v37": spec(K=33, V=37, T=20, gdn=True),
    "k100_v64": spec(K=100, V=64, T=18),
    "t1": spec(T=1),
    "t16": spec(T=16),
    "t17": spec(T=17),
    "non_beta_aware": spec(K=32, V=32, beta_aware=False, eta=0.05),
    "no_clamp": spec(K=32, V=32, clamp=False, eta=0.2),
    "clamp_hi": spec(K=16, V=16, T=64, keys="onehot", onehot_bias=0.6, eta=0.3, beta_mu=-1.5,
                     apf=False),
    "apf_to_dmin": spec(K=16, V=16, T=64, keys="sparse", apf_const=0.9, eta=0.05, apf=False),
}

FP32_OUT = ("dbeta", "dr", "dalpha", "dd1", "dS0")


def run_bwd(inp, dout, dS, dd, o_f32=False):
    p = inp["params"]
    dt = p["dtype"]
    g = osdn.bwd(to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
                 to_dev(inp["beta"], "f32"), to_dev(inp["r"], "f32"), to_dev(inp["alpha"], "f32"),
                 to_dev(inp["d1"], "f32"), to_dev(inp["S0"], "f32"), dout=to_dev(dout, dt),
                 dS=to_dev(dS, "f32"), dd=to_dev(dd, "f32"), eta=p["eta"], d_min=p["d_min"],
                 d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"], q_scale=p["q_scale"],
                 beta_aware=p["beta_aware"], o_f32=o_f32)
    torch.cuda.synchronize()
    return {k: (None if v is None else to_np(v)) for k, v in g.items()}


def oracle_bwd(inp, dout, dS, dd):
    p = inp["params"]
    return oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["r"], inp["alpha"],
                           inp["d1"], inp["S0"], dout=dout, dS=dS, dd=dd, eta=p["eta"],
                           d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
                           beta_aware=p["beta_aware"], q_scale=p["q_scale"])


def check(g, ref, dtype, tag, g32=None):
    """fp32 gradients within 1e-4 relative.  Gradients stored in the input
    dtype (dq, dk, dv) for bf16: the float32 ones of the same call (g32,
    o_f32) within 2e-2 tensor-wide, the bf16 ones their nearest-even rounding
    and within 2e-2 per row."""
    errs = {}
    for key, val in ref.items():
        if val is None:
            assert g[key] is None, (tag, key)
            continue
        if dtype == "bf16" and key not in FP32_OUT:
            check_bf16_readout(g[key], g32[key], val, "%s %s" % (tag, key))
        else:
            errs[key] = (rel_err(g[key], val), F32_OS)
    print(tag, {k: "%.2e" % e for k, (e, _) in errs.items()})
    for key, (e, bar) in errs.items():
        assert e <= bar, (tag, key, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_parity(case, dtype):
    inp = make_inputs(dict(CASES[case], dtype=dtype))
    d1, S0 = random_state(inp, seed=7)
    inp = dict(inp, d1=d1, S0=S0)
    dout, dS, dd = random_cotangent(inp, seed=8)
    g = run_bwd(inp, dout, dS, dd)
    g32 = run_bwd(inp, dout, dS, dd, o_f32=True) if dtype == "bf16" else None
    ref = oracle_bwd(inp, dout, dS, dd)
    check(g, ref, dtype, case, g32)


def test_backward_defaults_and_no_upstream_state_gradient():
    """Without d1, S0, dS and dd (ones, zeros, zero, zero)."""
    inp = make_inputs(spec(K=32, V=32, T=30, gdn=True))
    dout, _, _ = random_cotangent(inp, seed=9)
    g = run_bwd(inp, dout, None, None)
    check(g, oracle_bwd(inp, dout, None, None), "f32", "defaults")


def test_backward_zero_upstream_is_zero():
    inp = make_inputs(spec(K=32, V=32, T=30))
    z = np.zeros((2, 30, 2, 32), np.float32)
    g = run_bwd(inp, z, None, None)
    for key, val in g.items():
        if val is not None:
            assert not np.any(val), key


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_empty_sequence(dtype):
    """T = 0: dS0 = dS and dd1 = dd."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    z = torch.zeros((2, 0, 3, 32), device="cuda:0", dtype=tdt)
    zv = torch.zeros((2, 0, 3, 48), device="cuda:0", dtype=tdt)
    dS = torch.randn((2, 3, 48, 32), device="cuda:0")
    dd = torch.randn((2, 3, 32), device="cuda:0")
    g = osdn.bwd(z, z, zv, torch.zeros((2, 0, 3), device="cuda:0"), dout=zv, dS=dS, dd=dd)
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dS) and torch.equal(g["dd1"], dd)


def test_backward_full_size_sampled():
    """The forward bench's workload (B=4, T=4096, H=16, K=V=128, bf16, APF) in
    one osdn_bwd call; the oracle recomputes the gradients of eight whole
    (b,h) sequences (two heads of every batch element)."""
    inp = make_inputs("1p3b_apf")
    dout, dS, dd = random_cotangent(inp, seed=10)
    g = run_bwd(inp, dout, dS, dd)
    g32 = run_bwd(inp, dout, dS, dd, o_f32=True)
    pairs = [(b, h) for b in range(4) for h in (b, 15 - b)]
    sub = sample_sequences(dict(inp), pairs)
    sub_dout = np.stack([dout[b, :, h] for b, h in pairs])[:, :, None, :]
    sub_dS = np.stack([dS[b, h] for b, h in pairs])[:, None]
    sub_dd = np.stack([dd[b, h] for b, h in pairs])[:, None]
    ref = oracle_bwd(sub, sub_dout, sub_dS, sub_dd)
    def pick(gr):
        gi = {}
        for key, val in gr.items():
            if val is None:
                gi[key] = None
            elif key in ("dq", "dk", "dv", "dbeta", "dr"):
                gi[key] = np.stack([val[b, :, h] for b, h in pairs])[:, :, None]
            else:
                gi[key] = np.stack([val[b, h] for b, h in pairs])[:, None]
        return gi
    check(pick(g), ref, "bf16", "1p3b_apf x8", pick(g32))


def test_backward_rejects_aliasing():
    q = torch.zeros((1, 4, 1, 16), device="cuda:0")
    beta = torch.zeros((1, 4, 1), device="cuda:0")
    d = osdn.make_desc(1, 4, 1, 16, 16, dtype=osdn.F32)
    import ctypes
    lib = osdn.load()
    ws = torch.empty(osdn.bwd_workspace_bytes(1, 4, 1, 16, 16, osdn.F32), dtype=torch.uint8,
                     device="cuda:0")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    null = ctypes.c_void_p(None)
    k, v, dout = torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q)
    dk, dv, dbeta = torch.empty_like(q), torch.empty_like(q), torch.empty_like(beta)
    st = lib.osdn_bwd(ctypes.byref(d), p(q), p(k), p(v), p(beta), null, null, null, null, p(dout),
                      null, null, p(q), p(dk), p(dv), p(dbeta), null, null, null, null, p(ws),
                      ctypes.c_size_t(ws.numel()), null)
    assert st == osdn.EINVAL and "alias" in lib.osdn_last_error().decode()
