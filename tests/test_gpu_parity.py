"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases are compared element by element on every output; the full-size
workloads run on the GPU exactly as the bench launches them and every (b,h)
sequence is compared with the oracle.
"""
import math

import numpy as np
import pytest

import oracle
import preconditioned_delta_rule_amd as osdn
from tests.helpers import (BF16_OS, F32_D, F32_KT, F32_OS, check_bf16_readout, check_bf16_state,
                           dtype_round, o_err, rel_err, rms_err, s_err, to_dev, to_np, ulp_err)
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    osdn.load()
    yield
    torch.cuda.synchronize()


def small(**kw):
    base = dict(B=2, T=100, H=3, K=16, V=16, dtype="f32", chunk=16, seed=11)
    base.update(kw)
    return base


SCAN_CASES = {
    "tiny": "tiny",
    "k16_apf": small(apf=True),
    "k64": small(K=64, T=90),
    "k100_tail": small(K=100, T=70, apf=True),
    "k128": small(K=128, V=128, T=130),
    "k256": small(K=256, T=40),
    "clamp_hi": small(K=16, T=300, keys="onehot", onehot_bias=0.6, eta=0.05, beta_mu=-1.5),
    "apf_interior": small(K=16, T=200, keys="sparse", apf_const=0.99, eta=0.05),
    "non_beta_aware": small(K=32, T=120, apf=True, beta_aware=False, eta=0.05),
    "no_clamp": small(K=32, T=120, clamp=False, eta=0.2),
    "zero_keys": small(K=16, T=50, keys="onehot", eta=0.1),
}


def run_scan(inp, dtype, chunked=True, counters=False):
    p = inp["params"]
    k = to_dev(inp["k"], dtype)
    B, T, H, K = inp["k"].shape
    code = osdn.BF16 if dtype == "bf16" else osdn.F32
    ws = None
    if chunked:
        ws = torch.empty(osdn.precond_scan_workspace_bytes(B, T, H, K, code), dtype=torch.uint8,
                         device="cuda:0")
    kt, d = osdn.precond_scan(k, to_dev(inp["beta"], "f32"), to_dev(inp["r"], "f32"),
                              to_dev(inp["d1"], "f32"), eta=p["eta"], d_min=p["d_min"],
                              d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
                              beta_aware=p["beta_aware"], chunked=chunked, workspace=ws)
    torch.cuda.synchronize()
    if counters:
        return to_np(kt), to_np(d), osdn.scan_counters(ws, B, T, H, K, code).numpy()
    return to_np(kt), to_np(d)


def oracle_scan(inp):
    p = inp["params"]
    return oracle.precond_scan(inp["k"], inp["beta"], inp["r"], inp["d1"], eta=p["eta"],
                               d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
                               eps=p["eps"], beta_aware=p["beta_aware"])


@pytest.mark.parametrize("chunked", [False, True], ids=["sequential", "chunked"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", sorted(SCAN_CASES))
def test_scan_parity(case, dtype, chunked):
    spec = SCAN_CASES[case]
    if isinstance(spec, str):
        spec = dict(WORKLOADS[spec])
    inp = make_inputs(dict(spec, dtype=dtype))
    if case == "zero_keys":
        inp["k"][:, ::7] = 0.0
    kt, d = run_scan(inp, dtype, chunked)
    kt_ref, d_ref = oracle_scan(inp)
    assert rel_err(d, d_ref) <= F32_D, case
    if dtype == "f32":
        assert rel_err(kt, kt_ref) <= F32_KT, case
    else:
        assert ulp_err(kt, kt_ref) <= 1.0, case
    if case == "clamp_hi":
        assert np.any(d_ref == 2.0)       # the upper bound is reached
    if case == "apf_interior":
        assert np.any((d_ref > 0.5) & (d_ref < 2.0))


# Chunked phase 1: which path each 64-token chunk takes (counters per (b,h):
# pinned on d_min, closed form with a fixed active set, token by token).
PATH_CASES = {
    # no retention, keys spread over all coordinates: d stays inside the box
    "free": (dict(B=2, T=700, H=2, K=128, V=128, dtype="bf16", seed=31), "active"),
    # retention pulls every coordinate onto d_min within the first chunk
    "pinned": (dict(B=2, T=700, H=2, K=128, V=128, dtype="bf16", seed=32, apf=True), "pinned"),
    # retention 0.99 with sparse keys: coordinates split between d_min and the
    # interior, a fixed active set most of the time
    "mixed": (dict(B=1, T=1000, H=2, K=64, V=64, dtype="f32", seed=33, keys="sparse",
                   apf_const=0.99, eta=0.05), "any"),
    # one-hot keys, a coordinate drawn often climbs to d_max and stays there
    "upper": (dict(B=1, T=900, H=2, K=16, V=16, dtype="f32", seed=34, keys="onehot",
                   onehot_bias=0.6, eta=0.05, beta_mu=-1.5), "any"),
    # a large step crosses the bounds often: many chunks swept token by token
    "crossing": (dict(B=1, T=400, H=1, K=16, V=16, dtype="f32", seed=35, keys="onehot",
                      eta=0.9), "seq"),
}


@pytest.mark.parametrize("case", sorted(PATH_CASES))
def test_scan_chunk_paths(case):
    spec, expect = PATH_CASES[case]
    inp = make_inputs(spec)
    dtype = spec["dtype"]
    kt, d, cnt = run_scan(inp, dtype, chunked=True, counters=True)
    kt_ref, d_ref = oracle_scan(inp)
    B, T, H, K = inp["k"].shape
    N = -(-T // 64)
    print(case, "counters [pinned, active, seq] per (b,h):", cnt.reshape(-1, 3).tolist())
    assert np.all(cnt.sum(-1) == N)
    assert rel_err(d, d_ref) <= F32_D
    if dtype == "f32":
        assert rel_err(kt, kt_ref) <= F32_KT
    else:
        assert ulp_err(kt, kt_ref) <= 1.0
    if expect == "active":
        assert np.all(cnt[..., 1] == N)
    elif expect == "pinned":
        assert np.all(cnt[..., 0] >= N - 2)
    elif expect == "seq":
        assert np.all(cnt[..., 2] >= 1)
    if case == "upper":
        assert np.any(d_ref == 2.0)


CHUNK_CASES = {
    # generic fp32-arithmetic kernel
    "tiny_c16": dict(B=1, T=64, H=1, K=16, V=16, chunk=16),
    "k128_c64_tail": dict(B=1, T=150, H=2, K=128, V=128, chunk=64),
    "k64_v32_c32": dict(B=2, T=100, H=1, K=64, V=32, chunk=32),
    "k48_v80_c7": dict(B=1, T=40, H=2, K=48, V=80, chunk=7),
    # MFMA kernel (bf16, K = V = 128, C = 64) and, for f32, the generic one
    "mfma_one_chunk": dict(B=1, T=64, H=1, K=128, V=128, chunk=64),
    "mfma_tail": dict(B=1, T=200, H=3, K=128, V=128, chunk=64),
    "mfma_t1": dict(B=2, T=1, H=1, K=128, V=128, chunk=64),
    "mfma_grid_pad": dict(B=3, T=130, H=3, K=128, V=128, chunk=64),
}


def run_chunk_case(name, dtype, gated, s0, q_scale, seed=21, two_pass=True, o_f32=False):
    spec = dict(CHUNK_CASES[name], dtype=dtype, seed=seed, gdn=gated, apf=True)
    inp = make_inputs(spec)
    B, T, H, K = inp["k"].shape
    V = inp["v"].shape[-1]
    rng = np.random.default_rng(seed + 1)
    kt_ref, _ = oracle_scan(dict(inp, params=dict(inp["params"], eta=0.05)))
    kt_in = dtype_round(kt_ref, dtype)   # the write keys both sides consume
    S0 = (0.3 * rng.standard_normal((B, H, V, K))).astype(np.float32) if s0 else None
    o, S = osdn.chunk_fwd(to_dev(inp["q"], dtype), to_dev(inp["k"], dtype), to_dev(kt_in, dtype),
                          to_dev(inp["v"], dtype), to_dev(inp["beta"], "f32"),
                          to_dev(inp["alpha"], "f32"), to_dev(S0, "f32"), chunk=spec["chunk"],
                          q_scale=q_scale, two_pass=two_pass, o_f32=o_f32)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.delta_rule(inp["q"], inp["k"], kt_in, inp["v"], inp["beta"],
                                     inp["alpha"], S0, q_scale=q_scale)
    return to_np(o), to_np(S), o_ref, S_ref


@pytest.mark.parametrize("two_pass", [True, False], ids=["two_pass", "one_pass"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("name", sorted(CHUNK_CASES))
def test_chunk_parity(name, dtype, gated, two_pass):
    spec = CHUNK_CASES[name]
    mfma = dtype == "bf16" and spec["K"] == spec["V"] == 128 and spec["chunk"] == 64
    if not two_pass and not mfma:
        pytest.skip("only the matrix-core shapes have a second phase-2 path")
    s0 = name in ("mfma_tail", "k128_c64_tail", "tiny_c16")
    q_scale = 1.0 / math.sqrt(spec["K"]) if name in ("mfma_grid_pad", "k64_v32_c32") else 1.0
    o, S, o_ref, S_ref = run_chunk_case(name, dtype, gated, s0, q_scale, two_pass=two_pass)
    if dtype == "f32":
        assert rel_err(o, o_ref) <= F32_OS, (name, rel_err(o, o_ref))
        assert rel_err(S, S_ref) <= F32_OS, (name, rel_err(S, S_ref))
    else:
        o32, S32, _, _ = run_chunk_case(name, dtype, gated, s0, q_scale, two_pass=two_pass, o_f32=True)
        assert np.array_equal(S32, S)
        check_bf16_readout(o, o32, o_ref, name)
        check_bf16_state(S, S_ref, name)


def run_fwd(inp, dtype=None, o_f32=False, **over):
    p = dict(inp["params"])
    p.update(over)
    dt = dtype or p["dtype"]
    o, S, d = osdn.fwd(to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
                       to_dev(inp["beta"], "f32"), to_dev(inp["r"], "f32"),
                       to_dev(inp["alpha"], "f32"), to_dev(inp["d1"], "f32"),
                       to_dev(inp["S0"], "f32"), chunk=p["chunk"], eta=p["eta"],
                       d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
                       q_scale=p["q_scale"], beta_aware=p["beta_aware"], o_f32=o_f32)
    torch.cuda.synchronize()
    return o, S, d


def oracle_fwd(inp):
    p = inp["params"]
    return oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["r"], inp["alpha"],
                          inp["d1"], inp["S0"], eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"],
                          clamp=p["clamp"], eps=p["eps"], beta_aware=p["beta_aware"],
                          q_scale=p["q_scale"])


def test_fwd_tiny_workload():
    """The tiny oracle workload (B=1, H=1, T=64, K=V=16, fp32, C=16, seed 0)
    end to end, every element."""
    inp = make_inputs("tiny")
    o, S, d = run_fwd(inp)
    ref = oracle_fwd(inp)
    assert rel_err(to_np(d), ref["d"]) <= F32_D
    assert rel_err(to_np(o), ref["o"]) <= F32_OS
    assert rel_err(to_np(S), ref["S"]) <= F32_OS


FULL = ["340m", "1p3b_apf", "1p3b", "1p3b_clamp", "recall", "long_apf", "long_apf_gdn"]


@pytest.mark.parametrize("name", FULL)
def test_fwd_full_size(name):
    """Full-size workload on the GPU (one osdn_fwd call, as the bench runs it),
    every (b,h) sequence against the oracle: d per element, the readout and
    the state tensor-wide (the readout on the float32 outputs of a second
    call, whose nearest-even rounding must be the bf16 outputs bit for bit)."""
    inp = make_inputs(name)
    print(name, "shape", inp["k"].shape, flush=True)
    o, S, d = (to_np(x) for x in run_fwd(inp))
    o32, S32, d32 = (to_np(x) for x in run_fwd(inp, o_f32=True))
    assert np.array_equal(S32, S) and np.array_equal(d32, d)
    ref = oracle_fwd(inp)
    assert rel_err(d, ref["d"]) <= F32_D, (name, rel_err(d, ref["d"]))
    check_bf16_readout(o, o32, ref["o"], name)
    check_bf16_state(S, ref["S"], name)


@pytest.mark.parametrize("name,path", [("1p3b_apf", 0), ("340m", 1), ("recall", 1)])
def test_scan_full_size_write_keys(name, path):
    """At full size the emitted write keys are within one bf16 ulp of the fp64
    values on every sequence, and the chunked sweep takes its fast path
    (pinned with retention, closed form without) on all but the first chunks."""
    inp = make_inputs(name)
    kt, d, cnt = run_scan(inp, "bf16", chunked=True, counters=True)
    B, T, H, K = inp["k"].shape
    N = -(-T // 64)
    print(name, "chunks per path, summed over (b,h):", cnt.reshape(-1, 3).sum(0).tolist())
    assert np.all(cnt[..., path] >= N - 2)
    kt_ref, d_ref = oracle_scan(inp)
    assert ulp_err(kt, kt_ref) <= 1.0
    assert rel_err(d, d_ref) <= F32_D


def test_exact_write_counterexample_on_gpu():
    """Appendix D.4: K=V=1, k=1, v=(-1)^t, beta=0.5, d_1=2 gives S_t = (-1)^t
    exactly; in fp32 the device reproduces it bit for bit."""
    T = 32
    k = np.ones((1, T, 1, 1), np.float32)
    v = np.array([(-1.0) ** t for t in range(1, T + 1)], np.float32)[None, :, None, None]
    beta = np.full((1, T, 1), 0.5, np.float32)
    d1 = np.full((1, 1, 1), 2.0, np.float32)
    o, S, d = osdn.fwd(to_dev(k, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), to_dev(beta, "f32"),
                       d1=to_dev(d1, "f32"), chunk=8)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(o)[0, :, 0, 0], v[0, :, 0, 0])
    assert to_np(d)[0, 0, 0] == 2.0 and to_np(S)[0, 0, 0, 0] == 1.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_sequence(dtype):
    """T = 0: nothing to emit; d_out = d1 and S_out = S0."""
    K = V = 128
    q = torch.zeros((2, 0, 3, K), device="cuda:0",
                    dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
    beta = torch.zeros((2, 0, 3), device="cuda:0")
    d1 = torch.rand((2, 3, K), device="cuda:0") + 0.5
    S0 = torch.randn((2, 3, V, K), device="cuda:0")
    o, S, d = osdn.fwd(q, q, torch.zeros((2, 0, 3, V), device="cuda:0", dtype=q.dtype), beta,
                       d1=d1, S0=S0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, V)
    assert torch.equal(d, d1) and torch.equal(S, S0)


def test_in_place_state_and_determinism():
    """S_out may alias S0 and d_out may alias d1; repeated runs are bitwise
    identical (no atomics on the path)."""
    inp = make_inputs(dict(B=2, T=190, H=2, K=128, V=128, dtype="bf16", chunk=64, seed=5, apf=True))
    rng = np.random.default_rng(0)
    S0 = (0.2 * rng.standard_normal((2, 2, 128, 128))).astype(np.float32)
    d1 = rng.uniform(0.6, 1.5, (2, 2, 128)).astype(np.float32)
    args = [to_dev(inp[n], "bf16") for n in ("q", "k", "v")] + [to_dev(inp["beta"], "f32"),
                                                                 to_dev(inp["r"], "f32")]
    o1, S1, d1o = osdn.fwd(*args, d1=to_dev(d1, "f32"), S0=to_dev(S0, "f32"))
    S_buf, d_buf = to_dev(S0, "f32"), to_dev(d1, "f32")
    o2, S2, d2 = osdn.fwd(*args, d1=d_buf, S0=S_buf, S_out=S_buf, d_out=d_buf)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S_buf) and torch.equal(d1o, d_buf)
    o32, _, _ = osdn.fwd(*args, d1=to_dev(d1, "f32"), S0=to_dev(S0, "f32"), o_f32=True)
    ref = oracle_fwd(dict(inp, d1=d1, S0=S0))
    check_bf16_readout(to_np(o1), to_np(o32), ref["o"], "in_place")
    check_bf16_state(to_np(S1), ref["S"], "in_place")


def test_state_passing_on_gpu():
    """Prefill [0, T1) then continue [T1, T) carrying (S, d) equals one run over
    [0, T) within the bf16 bar (the prefill + decode check of Appendix L)."""
    inp = make_inputs(dict(B=1, T=300, H=2, K=128, V=128, dtype="bf16", chunk=64, seed=8, apf=True))
    T1 = 129
    full_o, full_S, full_d = run_fwd(inp)
    cut = lambda x, a, b: None if x is None else np.ascontiguousarray(x[:, a:b])
    first = dict(inp, **{n: cut(inp[n], 0, T1) for n in ("q", "k", "v", "beta", "r")})
    o1, S1, d1 = run_fwd(first)
    second = dict(inp, **{n: cut(inp[n], T1, 300) for n in ("q", "k", "v", "beta", "r")})
    second["S0"], second["d1"] = to_np(S1).astype(np.float32), to_np(d1).astype(np.float32)
    o2, S2, d2 = run_fwd(second)
    o2_32, _, _ = run_fwd(second, o_f32=True)
    o1_32, _, _ = run_fwd(first, o_f32=True)
    o_cat = np.concatenate([to_np(o1), to_np(o2)], axis=1)
    o_cat32 = np.concatenate([to_np(o1_32), to_np(o2_32)], axis=1)
    assert rel_err(to_np(d2), to_np(full_d)) <= F32_D
    ref = oracle_fwd(inp)
    check_bf16_readout(o_cat, o_cat32, ref["o"], "state_passing")
    check_bf16_state(to_np(S2), ref["S"], "state_passing")
    assert o_err(o_cat, to_np(full_o)) <= BF16_OS
    assert s_err(to_np(S2), to_np(full_S)) <= BF16_OS


def test_bad_pointer_is_reported_not_launched():
    """A misaligned device pointer is rejected with OSDN_EINVAL."""
    k = torch.zeros((1, 8, 1, 16), device="cuda:0")
    beta = torch.zeros(40, device="cuda:0")[1:9].view(1, 8, 1)
    with pytest.raises(osdn.OsdnError, match="aligned"):
        osdn.precond_scan(k, beta)


def test_fwd_write_keys_output_and_residual_path():
    """osdn_fwd with k_tilde_out: the bf16 write keys it returns are within one
    ulp of the fp64 ones, and the outputs (phase 2 fed through the bf16
    residual workspace) equal those of a call without k_tilde_out."""
    inp = make_inputs(dict(B=2, T=150, H=2, K=128, V=128, dtype="bf16", chunk=64, seed=7, apf=True))
    args = [to_dev(inp[n], "bf16") for n in ("q", "k", "v")] + [to_dev(inp["beta"], "f32"),
                                                                 to_dev(inp["r"], "f32")]
    kt = torch.empty_like(args[1])
    o1, S1, d1 = osdn.fwd(*args, k_tilde_out=kt)
    o2, S2, d2 = osdn.fwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(d1, d2)
    kt_ref, _ = oracle_scan(inp)
    assert ulp_err(to_np(kt), kt_ref) <= 1.0
    o32, _, _ = osdn.fwd(*args, o_f32=True)
    ref = oracle_fwd(inp)
    check_bf16_readout(to_np(o1), to_np(o32), ref["o"], "write_keys")
    check_bf16_state(to_np(S1), ref["S"], "write_keys")


BF16_KEYS_LIMIT = pytest.mark.xfail(
    strict=True, reason="write keys crossing the phases in bf16 (the box does not keep d >= 1/2) carry "
    "2^-9 relative error each; on the gated cases max|o|/rms is about 12 and the float32 readout "
    "reaches 3.4e-2 tensor-wide")


@pytest.mark.parametrize("box,gated", [("no_clamp", False), ("low_d_min", False),
                                       pytest.param("low_d_min", True, marks=BF16_KEYS_LIMIT),
                                       pytest.param("no_clamp", True, marks=BF16_KEYS_LIMIT)],
                         ids=["no_clamp-osdn", "low_d_min-osdn", "low_d_min-gdn", "no_clamp-gdn"])
def test_fwd_bf16_without_half_bound(box, gated):
    """bf16 osdn_fwd when the box does not keep d >= 1/2 (no clamp, or
    d_min < 1/2): d can shrink far below 1, so the write keys must not cross
    as the residual (d - 1) k (it would cancel) and cross in bf16 instead."""
    kw = dict(clamp=False, eta=0.2) if box == "no_clamp" else dict(d_min=0.02, eta=0.2)
    inp = make_inputs(dict(B=2, T=200, H=2, K=128, V=128, dtype="bf16", chunk=64, seed=9,
                           apf=True, gdn=gated, **kw))
    p = inp["params"]
    outs = [osdn.fwd(*(to_dev(inp[n], "bf16") for n in ("q", "k", "v")),
                     *(to_dev(inp[n], "f32") for n in ("beta", "r", "alpha")), eta=p["eta"],
                     d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"], o_f32=f)
            for f in (False, True)]
    torch.cuda.synchronize()
    ref = oracle_fwd(inp)
    assert float(np.min(ref["d"])) < 0.1  # d really leaves [1/2, 2]
    check_bf16_readout(to_np(outs[0][0]), to_np(outs[1][0]), ref["o"], box)
    check_bf16_state(to_np(outs[0][1]), ref["S"], box)
