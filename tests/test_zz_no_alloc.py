"""osdn_fwd_noalloc: osdn_fwd with the library's built-in scratch as workspace
(for callers that cannot allocate).  Through the C ABI it gives the bits of
osdn_fwd with a caller workspace, on two calls in a row (the second smaller,
so it reuses a scratch the first one filled), and refuses problems whose
workspace does not fit the scratch before launching anything."""
import numpy as np
import pytest

import preconditioned_delta_rule_amd as osdn
from tests.helpers import to_dev
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


def call_pair(spec):
    inp = make_inputs(spec)
    p, dt = inp["params"], inp["params"]["dtype"]
    B, T, H, K = inp["k"].shape
    V = inp["v"].shape[-1]
    args = [to_dev(inp[n], dt) for n in ("q", "k", "v")] + [to_dev(inp[n], "f32") for n in ("beta", "r", "alpha")]
    kw = dict(chunk=p["chunk"], eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
              q_scale=p["q_scale"], beta_aware=p["beta_aware"])
    ref = osdn.fwd(*args, **kw)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = (torch.full((B, T, H, V), float("nan"), dtype=tdt, device="cuda:0"),
           torch.full((B, H, V, K), float("nan"), device="cuda:0"),
           torch.full((B, H, K), float("nan"), device="cuda:0"))
    got = osdn.fwd_noalloc(*args, o=out[0], S_out=out[1], d_out=out[2], **kw)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_fwd_on_two_calls_in_a_row():
    big = dict(B=2, T=700, H=4, K=128, V=128, dtype="bf16", chunk=64, seed=51, apf=True, gdn=True)
    small = dict(B=1, T=130, H=2, K=128, V=128, dtype="bf16", chunk=64, seed=52)
    for spec in (big, small):
        ref, got = call_pair(spec)
        for r_, g_ in zip(ref, got):
            assert torch.equal(r_, g_), spec


def test_noalloc_fp32_generic_shapes():
    ref, got = call_pair(dict(B=2, T=90, H=3, K=48, V=80, dtype="f32", chunk=16, seed=53, apf=True))
    for r_, g_ in zip(ref, got):
        assert torch.equal(r_, g_)


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    B, T, H, K = 4, 4096, 16, 128
    need = osdn.fwd_workspace_bytes(B, T, H, K, K)
    assert need > osdn.FWD_NOALLOC_MAX_WORKSPACE
    q = torch.zeros((B, T, H, K), dtype=torch.bfloat16, device="cuda:0")
    beta = torch.zeros((B, T, H), device="cuda:0")
    o = torch.zeros_like(q)
    S = torch.zeros((B, H, K, K), device="cuda:0")
    d = torch.zeros((B, H, K), device="cuda:0")
    with pytest.raises(osdn.OsdnError) as e:
        osdn.fwd_noalloc(q, q, q, beta, o=o, S_out=S, d_out=d)
    assert e.value.status == osdn.EUNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not torch.any(o) and not torch.any(S)  # nothing was launched
