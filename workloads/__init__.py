"""Seeded synthetic inputs for the OSDN forward pass.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Tests, the bench and the smoke check feed the same arrays
to the GPU library and to the CPU oracle.

Recipe (same for every named workload unless stated):
  * numpy ``default_rng(seed)``; draw order q, k, v, beta-logits, r-logits,
    alpha-logits, all float32 standard normals in the [B,T,H,*] layout;
  * q and k are L2-normalised per (b,t,h) in float32, then (bf16 workloads)
    q, k, v are rounded to bfloat16 with round-to-nearest-even;
  * beta = sigmoid(N(mu_b, 1)), retention r = sigmoid(N(2, 1)) when APF is on,
    Gated-DeltaNet decay alpha = exp(-softplus(N(0,1)) * 0.1);
  * d_1 = 1, S_0 = 0, eta = 0.003, box [0.5, 2], eps = 1e-6;
  * the backward pass's upstream gradients (``random_cotangent``): a third
    generator ``default_rng(seed + 2)`` draws dL/do ~ N(0, 1) [B,T,H,V]
    (rounded to bf16 for bf16 workloads), then dL/dS_T ~ N(0, 1) and
    dL/dd_{T+1} ~ N(0, 1), float32;
  * OSKDA workloads (``kda``) draw, after everything above, a channel-wise
    decay alpha = exp(-softplus(N(0,1)) * kda_decay) per key channel
    [B,T,H,K] (kda_decay 0.1 unless stated); ``r_vec`` then draws a vector
    retention r = sigmoid(N(2,1)) per key coordinate [B,T,H,K] in place of the
    scalar one;
  * packed variable-length batches (``varlen_lengths``): sequence lengths
    drawn with ``default_rng(seed + 3)`` uniformly from [256, 4096] until the
    packed length is reached (the last one cut to fit);
  * decode workloads (a few new tokens continuing a carried state) draw their
    tokens the same way and the state with ``random_state``: a second
    generator ``default_rng(seed + 1)`` draws d_1 ~ U(0.6, 1.9) per coordinate
    (inside the box), then S_0 ~ 0.3 N(0, 1), both float32.

Float arrays are returned as float32 holding the exact (bf16-representable, for
bf16 workloads) values that the device receives.
"""
from __future__ import annotations

import math

import numpy as np

# Named workloads: the shapes and distributions of the paper's single-layer
# settings (340M: 8 heads; 1.3B: 16 heads; head dims 128; chunk 64).
WORKLOADS = {
    "tiny": dict(B=1, T=64, H=1, K=16, V=16, dtype="f32", chunk=16, seed=0),
    "340m": dict(B=8, T=2048, H=8, K=128, V=128, dtype="bf16", chunk=64, seed=1),
    "1p3b_apf": dict(B=4, T=4096, H=16, K=128, V=128, dtype="bf16", chunk=64,
                     seed=2, apf=True),
    # the same layer without the APF retention
    "1p3b": dict(B=4, T=4096, H=16, K=128, V=128, dtype="bf16", chunk=64, seed=2),
    # the same layer with a tighter box and a larger step, so that the clamp
    # binds intermittently (some coordinate on a bound in about one chunk in
    # seven, more towards the end as d approaches d_max)
    "1p3b_clamp": dict(B=4, T=4096, H=16, K=128, V=128, dtype="bf16", chunk=64, seed=2,
                       eta=0.05, d_min=0.8, d_max=1.25),
    "recall": dict(B=8, T=2048, H=8, K=128, V=128, dtype="bf16", chunk=64,
                   seed=3, keys="recall", beta_mu=1.0),
    "long_apf": dict(B=1, T=20480, H=16, K=128, V=128, dtype="bf16", chunk=64,
                     seed=4, apf=True),
    "long_apf_gdn": dict(B=1, T=20480, H=16, K=128, V=128, dtype="bf16",
                         chunk=64, seed=4, apf=True, gdn=True),
    # decode: one new token per sequence of the 1.3B-shaped layer, carrying a
    # state; the small batch and a serving batch of 256 sequences
    # backward: the 1.3B-shaped layer at a shorter sequence
    "bwd_1p3b_t1024": dict(B=4, T=1024, H=16, K=128, V=128, dtype="bf16", chunk=64,
                           seed=7, apf=True),
    # packed variable-length batch (the training batches of the pages'
    # Appendix F): 65,536 tokens, sequence lengths from varlen_lengths
    "varlen_1p3b_65k": dict(B=1, T=65536, H=16, K=128, V=128, dtype="bf16", chunk=64,
                            seed=8, apf=True),
    # the 1.3B-shaped layer with vector retention (one retention per key
    # coordinate, Proposition A.3)
    "1p3b_rvec": dict(B=4, T=4096, H=16, K=128, V=128, dtype="bf16", chunk=64,
                      seed=10, apf=True, r_vec=True),
    # OSKDA on the 340M KDA-shaped layer (8 heads of 128), APF retention,
    # channel-wise decay
    "kda_340m_apf": dict(B=8, T=2048, H=8, K=128, V=128, dtype="bf16", chunk=64, seed=9,
                         apf=True, kda=True),
    "decode_1p3b": dict(B=4, T=1, H=16, K=128, V=128, dtype="bf16", chunk=64,
                        seed=5, apf=True, state=True),
    "decode_1p3b_b256": dict(B=256, T=1, H=16, K=128, V=128, dtype="bf16",
                             chunk=64, seed=6, apf=True, state=True),
}

DEFAULTS = dict(eta=0.003, d_min=0.5, d_max=2.0, eps=1e-6, clamp=True,
                beta_aware=True, q_scale=1.0, keys="normal", beta_mu=0.0,
                apf=False, apf_const=None, gdn=False, dtype="f32", chunk=64,
                seed=0, onehot_bias=None, sparse_nnz=3, state=False, kda=False,
                kda_decay=0.1, r_vec=False)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isfinite(x), out, x).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (for comparing rounded outputs)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return np.power(2.0, e - 7)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0)


def _normalise(x):
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def spec_of(name_or_spec) -> dict:
    if isinstance(name_or_spec, str):
        spec = dict(WORKLOADS[name_or_spec])
        spec["name"] = name_or_spec
    else:
        spec = dict(name_or_spec)
    full = dict(DEFAULTS)
    full.update(spec)
    return full


def _recall_keys(rng, B, T, H, K, V):
    """Repeated-context recall stream: per head a pool of 512 unit keys with
    fixed values; each token is a fresh distractor with probability 0.2, else a
    pool item drawn with Zipf(1.1) frequency over ranks 1..512 (rank order =
    pool order), its value perturbed by N(0, 0.1^2)."""
    P = 512
    pool = _normalise(rng.standard_normal((H, P, K), dtype=np.float32))
    vals = rng.standard_normal((H, P, V), dtype=np.float32)
    w = np.arange(1, P + 1, dtype=np.float64) ** -1.1
    w /= w.sum()
    idx = rng.choice(P, size=(B, T, H), p=w)
    fresh = rng.random((B, T, H)) < 0.2
    hh = np.broadcast_to(np.arange(H)[None, None, :], (B, T, H))
    k = pool[hh, idx]
    v = vals[hh, idx] + np.float32(0.1) * rng.standard_normal((B, T, H, V), dtype=np.float32)
    dk = _normalise(rng.standard_normal((B, T, H, K), dtype=np.float32))
    dv = rng.standard_normal((B, T, H, V), dtype=np.float32)
    k = np.where(fresh[..., None], dk, k).astype(np.float32)
    v = np.where(fresh[..., None], dv, v).astype(np.float32)
    return k, v


def make_inputs(name_or_spec, *, T=None, B=None, H=None) -> dict:
    """Draw one workload.  Returns a dict with q, k, v, beta, r, alpha, d1, S0
    (numpy float32 or None) and 'params' (the scalar arguments)."""
    s = spec_of(name_or_spec)
    if T is not None:
        s["T"] = T
    if B is not None:
        s["B"] = B
    if H is not None:
        s["H"] = H
    Bn, Tn, Hn, K, V = s["B"], s["T"], s["H"], s["K"], s["V"]
    rng = np.random.default_rng(s["seed"])
    q = rng.standard_normal((Bn, Tn, Hn, K), dtype=np.float32)
    kind = s["keys"]
    if kind == "recall":
        k, v = _recall_keys(rng, Bn, Tn, Hn, K, V)
    else:
        k = rng.standard_normal((Bn, Tn, Hn, K), dtype=np.float32)
        v = rng.standard_normal((Bn, Tn, Hn, V), dtype=np.float32)
        if kind == "onehot":
            # one-hot keys; with onehot_bias=p coordinate 0 is drawn with prob. p
            j = rng.integers(0, K, size=(Bn, Tn, Hn))
            if s["onehot_bias"] is not None:
                j = np.where(rng.random((Bn, Tn, Hn)) < s["onehot_bias"], 0, j)
            k = np.zeros_like(k)
            np.put_along_axis(k, j[..., None], 1.0, axis=-1)
        elif kind == "sparse":
            # a few non-zero coordinates per key (random support), unit norm
            nnz = s["sparse_nnz"]
            mask = np.zeros(k.shape, bool)
            sup = np.argsort(rng.random(k.shape), axis=-1)[..., :nnz]
            np.put_along_axis(mask, sup, True, axis=-1)
            k = np.where(mask, k, 0).astype(np.float32)
    q = _normalise(q)
    if kind not in ("onehot",):
        k = _normalise(k)
    beta = _sigmoid(rng.standard_normal((Bn, Tn, Hn), dtype=np.float32)
                    + np.float32(s["beta_mu"])).astype(np.float32)
    r = None
    if s["apf"]:
        logits = rng.standard_normal((Bn, Tn, Hn), dtype=np.float32) + np.float32(2.0)
        r = _sigmoid(logits).astype(np.float32)
    if s["apf_const"] is not None:
        r = np.full((Bn, Tn, Hn), s["apf_const"], np.float32)
    alpha = None
    if s["gdn"]:
        g = rng.standard_normal((Bn, Tn, Hn), dtype=np.float32)
        alpha = np.exp(-_softplus(g) * np.float32(0.1)).astype(np.float32)
    if s["kda"]:
        # channel-wise decay of the KDA backbone, one gate per key channel
        g = rng.standard_normal((Bn, Tn, Hn, K), dtype=np.float32)
        alpha = np.exp(-_softplus(g) * np.float32(s["kda_decay"])).astype(np.float32)
    if s["r_vec"]:
        # vector retention: one retention per key coordinate
        logits = rng.standard_normal((Bn, Tn, Hn, K), dtype=np.float32) + np.float32(2.0)
        r = _sigmoid(logits).astype(np.float32)
    if s["dtype"] == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    params = {key: s[key] for key in ("eta", "d_min", "d_max", "eps", "clamp",
                                       "beta_aware", "q_scale", "chunk", "dtype")}
    if params["q_scale"] == "rsqrt_k":
        params["q_scale"] = 1.0 / math.sqrt(K)
    out = dict(q=q, k=k, v=v, beta=beta, r=r, alpha=alpha, d1=None, S0=None,
               params=params, spec=s)
    if s["state"]:
        out["d1"], out["S0"] = random_state(out, seed=s["seed"] + 1)
    return out


def random_state(inputs: dict, seed: int = 0, s_scale: float = 0.3):
    """A carried state for the shapes of `inputs`: d_1 ~ U(0.6, 1.9) [B,H,K]
    and S_0 ~ s_scale * N(0, 1) [B,H,V,K], float32, from default_rng(seed)."""
    B, _, H, K = inputs["k"].shape
    V = inputs["v"].shape[-1]
    rng = np.random.default_rng(seed)
    d1 = rng.uniform(0.6, 1.9, (B, H, K)).astype(np.float32)
    S0 = (np.float32(s_scale) * rng.standard_normal((B, H, V, K), dtype=np.float32)).astype(np.float32)
    return d1, S0


def sample_sequences(inputs: dict, pairs) -> dict:
    """Restrict a workload to a list of (b, h) sequences (B'=len(pairs), H=1),
    so the oracle can check a bounded sample of a full-size run."""
    out = dict(inputs)
    for key in ("q", "k", "v"):
        out[key] = np.stack([inputs[key][b, :, h] for b, h in pairs])[:, :, None, :]
    for key in ("beta", "r", "alpha"):
        if inputs[key] is not None:
            out[key] = np.stack([inputs[key][b, :, h] for b, h in pairs])[:, :, None]
    for key in ("d1", "S0"):
        if inputs[key] is not None:
            out[key] = np.stack([inputs[key][b, h] for b, h in pairs])[:, None]
    return out


def random_cotangent(inputs: dict, seed: int = 0):
    """Upstream gradients for the shapes of `inputs`: dout [B,T,H,V] (bf16
    values for bf16 workloads), dS [B,H,V,K] and dd [B,H,K], float32, from
    default_rng(seed)."""
    B, T, H, K = inputs["k"].shape
    V = inputs["v"].shape[-1]
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((B, T, H, V), dtype=np.float32)
    if inputs["params"]["dtype"] == "bf16":
        dout = bf16_round(dout)
    dS = rng.standard_normal((B, H, V, K), dtype=np.float32)
    dd = rng.standard_normal((B, H, K), dtype=np.float32)
    return dout, dS, dd


def varlen_lengths(total: int, seed: int = 0, lo: int = 256, hi: int = 4096):
    """Sequence lengths of a packed batch: uniform integers in [lo, hi] from
    default_rng(seed), the last one cut so that they sum to total."""
    rng = np.random.default_rng(seed)
    out, acc = [], 0
    while acc < total:
        n = int(min(rng.integers(lo, hi + 1), total - acc))
        out.append(n)
        acc += n
    return out
