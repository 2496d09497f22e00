"""GPU parity of vector retention (r [B,T,H,K], the diag(r_t) form of
Appendix A.5 Proposition A.3) in phase 1: the chunked sweep (K <= 128) and the
token-by-token kernel against the oracle, and through osdn_fwd on packed
sequences.  Bars as for phase 1: d within 1e-5 relative; fp32 write keys
within 1e-5, bf16 ones within one bf16 ulp of the fp64 value."""
import numpy as np
import pytest

import oracle
import preconditioned_delta_rule_amd as osdn
from tests.helpers import F32_D, F32_KT, rel_err, to_dev, to_np, ulp_err
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


def case(K, T=150, retention="apf", eta=0.003, clamp=True, seed=81, B=2, H=2):
    inp = make_inputs(dict(B=B, T=T, H=H, K=K, V=16, seed=seed, apf=True, r_vec=True, eta=eta, clamp=clamp))
    if retention == "near_one":
        # retention close to 1 and a large step: d leaves d_min, chunks are swept
        rng = np.random.default_rng(seed + 7)
        inp["r"] = (1.0 - 0.02 * rng.random(inp["r"].shape)).astype(np.float32)
    return inp


CASES = {
    "k16_apf": dict(K=16),
    "k64_apf": dict(K=64, T=200),
    "k100_apf": dict(K=100, T=130),
    "k128_apf": dict(K=128, T=260),
    "k128_near_one": dict(K=128, T=260, retention="near_one", eta=0.3),
    "k33_near_one": dict(K=33, T=90, retention="near_one", eta=0.5),
    "k128_no_clamp": dict(K=128, T=130, retention="near_one", eta=0.2, clamp=False),
    "k256_token_kernel": dict(K=256, T=70),
    "t1": dict(K=128, T=1),
}


def oracle_scan(inp, d1):
    p = inp["params"]
    return oracle.precond_scan(inp["k"], inp["beta"], inp["r"], d1, eta=p["eta"], d_min=p["d_min"],
                               d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"], beta_aware=p["beta_aware"])


@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "token"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_vector_retention_phase1(name, dtype, chunked):
    inp = case(**CASES[name])
    p = inp["params"]
    B, T, H, K = inp["k"].shape
    d1 = np.random.default_rng(3).uniform(0.6, 1.9, (B, H, K)).astype(np.float32)
    kt, d = osdn.precond_scan(to_dev(inp["k"], dtype), to_dev(inp["beta"], "f32"), to_dev(inp["r"], "f32"),
                              to_dev(d1, "f32"), eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"],
                              clamp=p["clamp"], eps=p["eps"], beta_aware=p["beta_aware"], chunked=chunked)
    torch.cuda.synchronize()
    kin = inp["k"] if dtype == "f32" else to_np(to_dev(inp["k"], "bf16"))
    ref_kt, ref_d = oracle_scan(dict(inp, k=kin), d1)
    assert rel_err(to_np(d), ref_d) <= F32_D, name
    if dtype == "f32":
        assert rel_err(to_np(kt), ref_kt) <= F32_KT, name
    else:
        assert ulp_err(to_np(kt), ref_kt) <= 1.0, name


def test_vector_retention_chunked_skips_pinned_chunks():
    """APF-like retention keeps d on d_min: the chunked sweep takes most chunks
    as pinned (counters), and agrees with the token-by-token kernel."""
    inp = case(K=128, T=1024, B=1, H=4)
    p = inp["params"]
    k, beta, r = to_dev(inp["k"], "bf16"), to_dev(inp["beta"], "f32"), to_dev(inp["r"], "f32")
    ws = torch.empty(osdn.precond_scan_workspace_bytes(1, 1024, 4, 128, osdn.BF16), dtype=torch.uint8,
                     device="cuda:0")
    kt1, d1 = osdn.precond_scan(k, beta, r, eta=p["eta"], workspace=ws)
    kt2, d2 = osdn.precond_scan(k, beta, r, eta=p["eta"], chunked=False)
    torch.cuda.synchronize()
    cnt = osdn.scan_counters(ws, 1, 1024, 4, 128, osdn.BF16)
    assert int(cnt[..., 0].sum()) >= 32, cnt  # of 64 chunks
    assert rel_err(to_np(d1), to_np(d2)) <= F32_D
    assert ulp_err(to_np(kt1), to_np(kt2).astype(np.float64)) <= 1.0


def test_vector_retention_packed_sequences():
    """osdn_fwd_varlen with vector retention equals osdn_fwd on each sequence."""
    lens = [100, 1, 64, 0, 190]
    total = sum(lens)
    inp = make_inputs(dict(B=1, T=total, H=2, K=128, V=128, dtype="bf16", seed=82, apf=True, r_vec=True))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    args = [to_dev(inp[n], "bf16") for n in ("q", "k", "v")] + [to_dev(inp[n], "f32") for n in ("beta", "r")]
    o, S, d = osdn.fwd_varlen(*args, cu_seqlens=torch.from_numpy(cu).to("cuda:0"))
    torch.cuda.synchronize()
    for i, L in enumerate(lens):
        a, b = int(cu[i]), int(cu[i + 1])
        sl = [to_dev(np.ascontiguousarray(inp[n][:, a:b]), "bf16") for n in ("q", "k", "v")]
        sl += [to_dev(np.ascontiguousarray(inp[n][:, a:b]), "f32") for n in ("beta", "r")]
        o1, S1, d1 = osdn.fwd(*sl)
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:b], o1) and torch.equal(S[i:i + 1], S1) and torch.equal(d[i:i + 1], d1), i


def run_fwd_rvec(inp, **over):
    p = dict(inp["params"])
    p.update(over)
    args = [to_dev(inp[n], "bf16") for n in ("q", "k", "v")] + [to_dev(inp[n], "f32") for n in ("beta", "r")]
    out = osdn.fwd(*args, eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
                   eps=p["eps"], q_scale=p["q_scale"], beta_aware=p["beta_aware"],
                   **{k: v for k, v in over.items() if k in ("k_tilde_out", "o_f32")})
    torch.cuda.synchronize()
    return out


def oracle_fwd(inp):
    p = inp["params"]
    return oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["r"], None, eta=p["eta"],
                          d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
                          beta_aware=p["beta_aware"], q_scale=p["q_scale"])


FOLD_CASES = {
    # retention sigmoid(N(2,1)): d pinned on d_min after the first chunk
    "apf_t150": dict(T=150, retention="apf"),
    # retention close to 1 with a large step: chunks are swept and replayed
    # per coordinate, with a partial last chunk
    "near_one_t150": dict(T=150, retention="near_one", eta=0.3),
    "near_one_t256": dict(T=256, retention="near_one", eta=0.3),
}


@pytest.mark.parametrize("name", sorted(FOLD_CASES))
def test_vector_retention_folded_residual_is_bitwise_the_emitted_one(name):
    """bf16, K = 128, r [B,T,H,K]: without k_tilde_out the first phase-2 kernel
    replays d per coordinate and forms the write-key residual itself; with
    k_tilde_out the phase-1 emit kernel writes it.  Both give the same bits,
    and both meet the bf16 bars against the oracle."""
    c = FOLD_CASES[name]
    inp = case(128, T=c["T"], retention=c["retention"], eta=c.get("eta", 0.003), seed=91)
    inp = dict(inp)
    rng = np.random.default_rng(92)
    inp["v"] = np.asarray(rng.standard_normal(inp["k"].shape[:3] + (128,)), np.float32)
    from workloads import bf16_round
    inp["v"] = bf16_round(inp["v"])
    inp["q"] = bf16_round(inp["q"])
    inp["k"] = bf16_round(inp["k"])
    kt = torch.empty(inp["k"].shape, dtype=torch.bfloat16, device="cuda:0")
    o1, S1, d1 = run_fwd_rvec(inp)
    o2, S2, d2 = run_fwd_rvec(inp, k_tilde_out=kt)
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(d1, d2), name
    o32 = run_fwd_rvec(inp, o_f32=True)[0]
    ref = oracle_fwd(inp)
    from tests.helpers import check_bf16_readout, check_bf16_state
    assert rel_err(to_np(d1), ref["d"]) <= F32_D
    check_bf16_readout(to_np(o1), to_np(o32), ref["o"], name)
    check_bf16_state(to_np(S1), ref["S"], name)


def test_vector_retention_full_size():
    """The bench's vector-retention workload (osdn_fwd, B=4, T=4096, H=16,
    K=V=128, bf16, r [B,T,H,K]) in one call; every (b,h) against the oracle."""
    from tests.helpers import check_bf16_readout, check_bf16_state
    inp = make_inputs("1p3b_rvec")
    o, S, d = (to_np(x) for x in run_fwd_rvec(inp))
    o32 = to_np(run_fwd_rvec(inp, o_f32=True)[0])
    ref = oracle_fwd(inp)
    assert rel_err(d, ref["d"]) <= F32_D
    check_bf16_readout(o, o32, ref["o"], "1p3b_rvec")
    check_bf16_state(S, ref["S"], "1p3b_rvec")
