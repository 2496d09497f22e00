#!/usr/bin/env python3
"""OSDN forward throughput on one MI355X.

One step = one full forward of one layer: phase 1 (preconditioner scan) and
phase 2 (chunkwise WY delta rule) over a batch of synthetic inputs already in
HBM, through the C ABI entry point osdn_fwd.  The default workload is the
1.3B-shaped layer: B=4, H=16, T=4096, K=V=128, bf16 inputs, fp32 state,
chunk 64, APF retention on.

Prints ONE JSON line on stdout; progress goes to stderr.

Roofline bookkeeping (algorithmic, per token-head, K = V = 128, bf16):
  phase 1 bytes  = read k (2K) + beta (4) + r (4) + write k~ (2K)       = 520
  phase 2 bytes  = read q, k, k~ (2K each) + v (2V) + beta (4) + write o (2V)
                   (+4 for alpha)                                       = 1284
  phase 2 flops  = dense chunk form 2(3CK + 2CV + 3KV) at C = 64        = 180224
Peaks: HBM 8 TB/s, bf16 dense MFMA 2.5 PFLOP/s (MI355X published figures).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "OSDN fwd tokens/sec (phase1+phase2) at H=16,K=V=128,T=4096; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def phase_bytes(K, V, apf, gated, elem=2):
    p1 = elem * K * 2 + 4 + (4 if apf else 0)
    p2 = elem * (3 * K + V) + 4 + elem * V + (4 if gated else 0)
    return p1, p2


def phase2_flops(C, K, V):
    return 2 * (3 * C * K + 2 * C * V + 3 * K * V)


def cpu_baseline(inp, max_threads=None):
    """The CPU oracle (fp64, one (b,h) sequence per thread) on the same
    workload; returns tokens/s over the sample and the thread count."""
    import oracle
    B, T, H, _ = inp["k"].shape
    threads = min(B * H, max_threads or oracle.default_threads())
    p = inp["params"]
    t0 = time.perf_counter()
    oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["r"], inp["alpha"],
                   eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
                   eps=p["eps"], beta_aware=p["beta_aware"], q_scale=p["q_scale"],
                   threads=threads)
    wall = time.perf_counter() - t0
    return B * T / wall, threads, wall


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="1p3b_apf")
    ap.add_argument("--copies", type=int, default=4,
                    help="input sets rotated between steps (keeps the 256 MB MALL from "
                         "serving repeated reads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=16,
                    help="(b,h) sequences of the workload the CPU oracle runs")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the OSDN forward shards over (b,h) with no "
              "communication, so more GPUs just run independent shards; use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import preconditioned_delta_rule_amd as osdn
    from workloads import make_inputs, sample_sequences

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    osdn.load()
    dev = torch.device("cuda:0")
    log("generating workload", args.workload)
    inp = make_inputs(args.workload)
    spec, p = inp["spec"], inp["params"]
    B, T, H, K = inp["k"].shape
    V = inp["v"].shape[-1]
    C = p["chunk"]
    apf, gated = inp["r"] is not None, inp["alpha"] is not None
    tdt = torch.bfloat16 if p["dtype"] == "bf16" else torch.float32
    elem = 2 if p["dtype"] == "bf16" else 4

    def up(x, dt):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(dev)

    sets = []
    for c in range(max(1, args.copies)):
        sets.append(dict(q=up(inp["q"], tdt), k=up(inp["k"], tdt), v=up(inp["v"], tdt),
                         beta=up(inp["beta"], torch.float32), r=up(inp["r"], torch.float32),
                         alpha=up(inp["alpha"], torch.float32),
                         o=torch.empty((B, T, H, V), dtype=tdt, device=dev),
                         kt=torch.empty((B, T, H, K), dtype=tdt, device=dev),
                         ws=torch.empty(osdn.fwd_workspace_bytes(B, T, H, K, V, dtype=(
                             osdn.BF16 if p["dtype"] == "bf16" else osdn.F32), chunk=C),
                             dtype=torch.uint8, device=dev),
                         sws=torch.empty(osdn.precond_scan_workspace_bytes(B, T, H, K, dtype=(
                             osdn.BF16 if p["dtype"] == "bf16" else osdn.F32)),
                             dtype=torch.uint8, device=dev),
                         cws=torch.empty(max(1, osdn.chunk_fwd_workspace_bytes(
                             B, T, H, K, V, dtype=(osdn.BF16 if p["dtype"] == "bf16" else osdn.F32),
                             chunk=C)), dtype=torch.uint8, device=dev),
                         S=torch.empty((B, H, V, K), dtype=torch.float32, device=dev),
                         d=torch.empty((B, H, K), dtype=torch.float32, device=dev)))
    kw = dict(chunk=C, eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
              eps=p["eps"], q_scale=p["q_scale"], beta_aware=p["beta_aware"])

    def step(i):
        s = sets[i % len(sets)]
        osdn.fwd(s["q"], s["k"], s["v"], s["beta"], s["r"], s["alpha"], None, None,
                 o=s["o"], S_out=s["S"], d_out=s["d"], workspace=s["ws"], **kw)

    def scan(i, chunked=True):
        s = sets[i % len(sets)]
        osdn.precond_scan(s["k"], s["beta"], s["r"], None, eta=p["eta"], d_min=p["d_min"],
                          d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
                          beta_aware=p["beta_aware"], k_tilde=s["kt"], d_out=s["d"],
                          chunked=chunked, workspace=s["sws"] if chunked else None)

    def scan_seq(i):
        scan(i, chunked=False)

    def chunk(i):
        s = sets[i % len(sets)]
        osdn.chunk_fwd(s["q"], s["k"], s["kt"], s["v"], s["beta"], s["alpha"], None, chunk=C,
                       q_scale=p["q_scale"], o=s["o"], S_out=s["S"], workspace=s["cws"])

    def timed(fn, n):
        """Average device time of fn over n launches on the current stream
        (HIP events recorded on that stream)."""
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ms_step = timed(step, args.steps)
    wall = time.perf_counter() - w0
    log("step %.4f ms (wall %.3f s)" % (ms_step, wall))
    # per-phase average durations: phase 1 is three kernels (prep, solve,
    # emit), phase 2 one
    for i in range(2):
        scan(i)
        chunk(i)
        scan_seq(i)
    ms_scan = timed(scan, args.steps)
    ms_chunk = timed(chunk, args.steps)
    ms_scan_seq = timed(scan_seq, max(1, args.steps // 5))
    log("phase1 %.4f ms (token-by-token kernel %.4f ms)  phase2 %.4f ms"
        % (ms_scan, ms_scan_seq, ms_chunk))

    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    nth = B * T * H
    b1, b2 = phase_bytes(K, V, apf, gated, elem)
    f2 = phase2_flops(C, K, V)
    p1_gbs = b1 * nth / (ms_scan * 1e-3) / 1e9
    p2_gbs = b2 * nth / (ms_chunk * 1e-3) / 1e9
    p2_tfl = f2 * nth / (ms_chunk * 1e-3) / 1e12
    phases = {
        "precond_scan": {"kernel": "scan_prep_kernel + scan_solve_kernel + scan_emit_kernel",
                         "ms": ms_scan, "bound": "hbm", "bytes_per_token_head": b1,
                         "GB/s": p1_gbs, "hbm_frac": p1_gbs / HBM_PEAK_GBS,
                         "token_by_token_kernel_ms": ms_scan_seq},
        "chunk_fwd": {"kernel": "chunk_mfma_kernel", "ms": ms_chunk, "bound": "hbm",
                      "bytes_per_token_head": b2, "GB/s": p2_gbs,
                      "hbm_frac": p2_gbs / HBM_PEAK_GBS,
                      "flops_per_token_head": f2, "flop_count": "dense chunk form",
                      "TFLOP/s": p2_tfl, "mfma_bf16_frac": p2_tfl / MFMA_BF16_PEAK_TFLOPS},
    }
    dom = "precond_scan" if ms_scan >= ms_chunk else "chunk_fwd"
    dph = phases[dom]
    roofline = {"bound": "hbm", "kernel": dph["kernel"], "achieved": dph["GB/s"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dph["GB/s"] / HBM_PEAK_GBS,
                "traffic": None}

    cpu = None
    if not args.no_cpu_baseline:
        nseq = min(args.cpu_sample_seqs, B * H)
        pairs = [(i // H, i % H) for i in range(0, B * H, max(1, (B * H) // nseq))][:nseq]
        sub = sample_sequences(inp, pairs)
        log("cpu oracle on %d sequences x %d tokens" % (len(pairs), T))
        tps, threads, cwall = cpu_baseline(sub)
        # the sample is len(pairs) single-head sequences: tps counts token-heads,
        # a token of the workload carries all H heads
        value_cpu = tps / H
        cpu = {"value": value_cpu, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": "%d of %d (b,h) sequences x %d tokens (fp64 sequential oracle, one "
                         "sequence per thread), %.2f s wall; tokens/s scaled to all %d "
                         "heads" % (len(pairs), B * H, T, cwall, H)}
        log("cpu oracle %.1f s" % cwall)

    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": p["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V,
                   "chunk": C, "apf": apf, "gated": gated, "seed": spec["seed"],
                   "input_copies": len(sets)},
        "roofline": roofline, "phases": phases, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
