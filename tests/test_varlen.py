"""Variable-length (packed) sequences: osdn_fwd_varlen against osdn_fwd run on
each sequence alone (bit for bit: the same kernels see the same chunks) and
against the oracle run on each sequence alone (the state is reset at every
sequence boundary, as packed training batches require)."""
import numpy as np
import pytest

import oracle
import preconditioned_delta_rule_amd as osdn
from tests.helpers import (F32_D, F32_OS, check_bf16_readout, check_bf16_state, rel_err, to_dev,
                           to_np)
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


CASES = {
    # matrix-core path, phase 1 folded into the first phase-2 kernel
    "bf16_k128_apf": (dict(K=128, V=128, dtype="bf16", chunk=64, apf=True, seed=61),
                      [130, 64, 1, 0, 300, 63]),
    "bf16_k128_gdn": (dict(K=128, V=128, dtype="bf16", chunk=64, apf=True, gdn=True, seed=62),
                      [200, 5, 129]),
    # fp32: generic phase-2 kernel, chunk 16
    "f32_k16": (dict(K=16, V=16, dtype="f32", chunk=16, apf=True, seed=63), [40, 0, 17, 100, 64]),
    "f32_k33_v37": (dict(K=33, V=37, dtype="f32", chunk=16, seed=64, gdn=True), [23, 70]),
    # a single sequence
    "bf16_one": (dict(K=128, V=128, dtype="bf16", chunk=64, seed=65), [257]),
}


def packed(name):
    spec, lens = CASES[name]
    total = int(sum(lens))
    inp = make_inputs(dict(spec, B=1, T=total, H=3))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = len(lens)
    d1, S0 = random_state(dict(inp, k=np.zeros((S, 1, 3, spec["K"])), v=np.zeros((S, 1, 3, spec["V"]))),
                          seed=spec["seed"] + 100)
    return inp, cu, lens, d1, S0


def kwargs(p, **extra):
    kw = dict(chunk=p["chunk"], eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
              eps=p["eps"], q_scale=p["q_scale"], beta_aware=p["beta_aware"])
    kw.update(extra)
    return kw


def run_varlen(inp, cu, d1, S0, k_tilde=False, o_f32=False):
    p = inp["params"]
    dt = p["dtype"]
    args = [to_dev(inp[n], dt) for n in ("q", "k", "v")]
    args += [to_dev(inp[n], "f32") for n in ("beta", "r", "alpha")]
    kt = torch.empty_like(args[1]) if k_tilde else None
    o, S, d = osdn.fwd_varlen(*args, to_dev(d1, "f32"), to_dev(S0, "f32"),
                              cu_seqlens=torch.from_numpy(cu).to("cuda:0"), k_tilde_out=kt, o_f32=o_f32,
                              **kwargs(p))
    torch.cuda.synchronize()
    return o, S, d, kt


def seq_slice(inp, a, b):
    out = {}
    for n in ("q", "k", "v", "beta", "r", "alpha"):
        out[n] = None if inp[n] is None else np.ascontiguousarray(inp[n][:, a:b])
    return out


@pytest.mark.parametrize("k_tilde", [False, True], ids=["fused", "k_tilde_out"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_varlen_equals_each_sequence_alone(name, k_tilde):
    inp, cu, lens, d1, S0 = packed(name)
    p = inp["params"]
    dt = p["dtype"]
    o, S, d, kt = run_varlen(inp, cu, d1, S0, k_tilde)
    for i, L in enumerate(lens):
        a, b = int(cu[i]), int(cu[i + 1])
        sl = seq_slice(inp, a, b)
        args = [to_dev(sl[n], dt) for n in ("q", "k", "v")]
        args += [to_dev(sl[n], "f32") for n in ("beta", "r", "alpha")]
        kt1 = torch.empty_like(args[1]) if k_tilde else None
        o1, S1, d1o = osdn.fwd(*args, to_dev(d1[i:i + 1], "f32"), to_dev(S0[i:i + 1], "f32"),
                               k_tilde_out=kt1, **kwargs(p))
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:b], o1), (name, i)
        assert torch.equal(S[i:i + 1], S1), (name, i)
        assert torch.equal(d[i:i + 1], d1o), (name, i)
        if k_tilde:
            assert torch.equal(kt[:, a:b], kt1), (name, i)


def oracle_packed(inp, cu, d1, S0, heads=None):
    """The oracle run on each sequence alone (from its own d1 / S0 rows),
    laid out like the packed outputs: o [1,total,H,V], S [S,H,V,K], d [S,H,K]."""
    p = inp["params"]
    H = inp["k"].shape[2]
    o, S, d = np.zeros(inp["v"].shape), [], []
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        sl = seq_slice(inp, a, b)
        ref = oracle.forward(sl["q"], sl["k"], sl["v"], sl["beta"], sl["r"], sl["alpha"],
                             None if d1 is None else d1[i:i + 1], None if S0 is None else S0[i:i + 1],
                             eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
                             eps=p["eps"], beta_aware=p["beta_aware"], q_scale=p["q_scale"])
        o[:, a:b] = ref["o"]
        S.append(ref["S"])
        d.append(ref["d"])
    return o, np.concatenate(S), np.concatenate(d)


@pytest.mark.parametrize("name", sorted(CASES))
def test_varlen_parity_with_oracle(name):
    inp, cu, lens, d1, S0 = packed(name)
    p = inp["params"]
    o, S, d, _ = run_varlen(inp, cu, d1, S0)
    o, S, d = to_np(o), to_np(S), to_np(d)
    o_ref, S_ref, d_ref = oracle_packed(inp, cu, d1, S0)
    assert rel_err(d, d_ref) <= F32_D, name
    if p["dtype"] == "f32":
        assert rel_err(o, o_ref) <= F32_OS, name
        assert rel_err(S, S_ref) <= F32_OS, name
    else:
        o32 = to_np(run_varlen(inp, cu, d1, S0, o_f32=True)[0])
        check_bf16_readout(o, o32, o_ref, name)
        check_bf16_state(S, S_ref, name)


def test_varlen_all_empty():
    """Every sequence empty: d_out = d1 and S_out = S0."""
    K = V = 128
    q = torch.zeros((1, 0, 2, K), device="cuda:0", dtype=torch.bfloat16)
    d1 = torch.rand((3, 2, K), device="cuda:0") + 0.5
    S0 = torch.randn((3, 2, V, K), device="cuda:0")
    cu = torch.zeros(4, dtype=torch.int64, device="cuda:0")
    o, S, d = osdn.fwd_varlen(q, q, torch.zeros((1, 0, 2, V), device="cuda:0", dtype=torch.bfloat16),
                              torch.zeros((1, 0, 2), device="cuda:0"), d1=d1, S0=S0, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(d, d1) and torch.equal(S, S0)


def test_varlen_requires_cu_seqlens():
    import ctypes
    lib = osdn.load()
    d = osdn.make_desc(2, 8, 1, 16, 16, dtype=osdn.F32)
    null = ctypes.c_void_p(None)
    st = lib.osdn_fwd_varlen(ctypes.byref(d), null, *([null] * 13), ctypes.c_size_t(0), null)
    assert st == osdn.EINVAL and "cu_seqlens" in lib.osdn_last_error().decode()


def test_varlen_full_size():
    """The packed 65,536-token batch timed by the bench (sequences of 256-4,096
    tokens, H=16, K=V=128, bf16, APF) in one call; every (sequence, head)
    against the oracle run on that sequence alone."""
    from workloads import varlen_lengths
    inp = make_inputs("varlen_1p3b_65k")
    lens = varlen_lengths(inp["k"].shape[1], seed=inp["spec"]["seed"] + 3)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    o, S, d, _ = run_varlen(inp, cu, None, None)
    o32 = run_varlen(inp, cu, None, None, o_f32=True)[0]
    o_ref, S_ref, d_ref = oracle_packed(inp, cu, None, None)
    assert rel_err(to_np(d), d_ref) <= F32_D
    check_bf16_readout(to_np(o), to_np(o32), o_ref, "varlen_1p3b_65k")
    check_bf16_state(to_np(S), S_ref, "varlen_1p3b_65k")
