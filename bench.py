#!/usr/bin/env python3
"""OSDN forward throughput on one MI355X.

One step = one full forward of one layer through the C ABI entry point
osdn_fwd: phase 1 (preconditioner scan: scan_prep and scan_solve kernels)
and phase 2 (chunkwise WY delta rule: chunk_tinv, which also replays d to
form the write-key residual, and chunk_sweep) over a batch of synthetic inputs already resident in HBM.  The
default workload is the 1.3B-shaped layer: B=4, H=16, T=4096, K=V=128, bf16
inputs, fp32 state, chunk 64, APF retention on.

Prints ONE JSON line on stdout; progress goes to stderr.

Algorithmic work per token-head (K = V = 128, C = 64, bf16; +4 B for r or
alpha where present), used for the roofline figures:
  phase 1 (whole)   read k 2K + beta 4 (+ r 4), write k~ 2K             = 516 / 520 B
    scan_prep       read k 2K + beta 4 (+ r 4)                          = 260 / 264 B
    scan_solve      per-token scalars beta (+ r) and the key norm       =   8 /  12 B
    scan_emit       read k 2K (+ r 4) + step scalar 4, write k~ 2K      = 516 / 520 B
  phase 2 (whole)   read q, k, k~ 2K each + v 2V + beta 4, write o 2V   = 1284 B
    chunk_tinv      read k 2K, step scalar 4, beta 4 (+ r 4), write the
                    residual E 2K (the phase-1 replay is folded in)     = 520 / 524 B
                    flops: Gram 2 C K                                   = 16384
    chunk_sweep     read q, k, k~ 2K each + v 2V + beta 4, write o 2V   = 1284 B
                    (a chunk phase 1 took as pinned on d_min has write keys
                    d_min k: its k~ is not read, 1028 B)
                    flops: K S^T, Q S^T, S update 3 x 2 K V, scores
                    2 C K, Delta and O 2 x 2 C V                        = 147456
Both phases sit below the MFMA ridge (2.5 PFLOP/s / 8 TB/s = 312 flop/B),
so each kernel's roofline is HBM bandwidth (MI355X: 8 TB/s).  The bf16 MFMA
fraction (peak 2.5 PFLOP/s dense) is reported beside it for phase 2.

Per-kernel durations come from HIP events the library records on the launch
stream around every kernel of the timed steps (osdn_profile_begin/end).

With --backward a step is one osdn_bwd call (gradients of every input from
dL/do, dL/dS_T, dL/dd_{T+1}) on the forward's workload.  Its kernels are
recurrent, token by token per (b,h) in fp32, so each is reported against the
fp32 vector peak (157.3 TFLOP/s) with its arithmetic per token-head (K = V =
128: record 6 V K = 98,304 flops, the phase-2 reverse 14 V K = 229,376, the
phase-1 reverse 30 K = 3,840) and against HBM with its bytes.

With --varlen a step is one osdn_fwd_varlen call over a packed batch of
variable-length sequences (default: 65,536 tokens in sequences of 256-4,096,
H=16, K=V=128, bf16, APF); per-token-head work is that of the forward.

With --kda a step is one osdn_kda_fwd call (OSKDA: K x V state, channel-wise
decay; default B=8, T=2048, H=8, K=V=128, bf16, APF).  Its roofline is that of
the longest kernel, against whichever roof it comes closer to: HBM at its
algorithmic bytes, or the matrix cores at its algorithmic flops (bf16 peak for
bf16 inputs, whose sweep runs hi/lo bf16 pairs; fp32 peak for fp32 inputs).

With --decode a step is instead one osdn_decode call (the single-token
recurrence): T new tokens per (b,h) continuing a carried fp32 state, default
workload one token for each of 256 sequences of the 1.3B-shaped layer
(B=256, H=16, K=V=128, bf16, APF).  Its algorithmic bytes per (b,h) are the
state read and written once, 2 * 4 V K + 2 * 4 K, plus per token q, k (elem K
each), v, o (elem V each), beta (+ r, + alpha) 4 B; HBM bounds it.  The state
ping-pongs between two buffers, so every call reads the state the previous
one wrote.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "OSDN fwd tokens/sec (phase1+phase2) at H=16,K=V=128,T=4096; % HBM/MFMA roofline"
KDA_METRIC = "OSKDA fwd tokens/sec (osdn_kda_fwd) at H=8,K=V=128; % roofline of the dominant kernel"
VARLEN_METRIC = "OSDN fwd tokens/sec over a packed variable-length batch (osdn_fwd_varlen) at H=16,K=V=128; % HBM roofline"
BWD_METRIC = "OSDN bwd tokens/sec (osdn_bwd, both phases) at H=16,K=V=128,T=4096; % fp32 vector roofline"
FP32_VALU_PEAK_TFLOPS = 157.3
DECODE_METRIC = "OSDN decode tokens/sec (osdn_decode, new tokens x sequences per call) at H=16,K=V=128; % HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# where each kernel's source lives (for matching committed counter summaries)
KERNEL_SOURCE = {
    "scan_prep_kernel": "preconditioned_delta_rule_amd/csrc/precond_chunked.hip",
    "scan_factor_kernel": "preconditioned_delta_rule_amd/csrc/precond_chunked.hip",
    "scan_solve_kernel": "preconditioned_delta_rule_amd/csrc/precond_chunked.hip",
    "scan_emit_kernel": "preconditioned_delta_rule_amd/csrc/precond_chunked.hip",
    "chunk_tinv_kernel": "preconditioned_delta_rule_amd/csrc/chunk_wy.hip",
    "chunk_sweep_kernel": "preconditioned_delta_rule_amd/csrc/chunk_wy.hip",
    "decode_kernel": "preconditioned_delta_rule_amd/csrc/decode.hip",
    "bwd_record_kernel": "preconditioned_delta_rule_amd/csrc/backward.hip",
    "bwd_p2_kernel": "preconditioned_delta_rule_amd/csrc/backward.hip",
    "bwd_p1_kernel": "preconditioned_delta_rule_amd/csrc/backward.hip",
    "kda_intra_kernel": "preconditioned_delta_rule_amd/csrc/kda_chunk.hip",
    "kda_seq_kernel": "preconditioned_delta_rule_amd/csrc/kda_chunk.hip",
}
COPY_BYTES = 256 << 20  # calibration copy: 256 MiB read + 256 MiB written


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(name, K, V, C, apf, gated, elem=2, rvec=False, fused=True, swept=1.0):
    """(algorithmic bytes, flops) per token-head of one kernel (rvec: the
    retention is a [K] row per token).  fused: osdn_fwd, whose first phase-2
    kernel replays phase 1 and forms the write-key residual; otherwise
    osdn_precond_scan then osdn_chunk_fwd, where the emit kernel writes k~ and
    phase 2 reads it.  swept: the fraction of 64-token chunks that phase 1 did
    not take as pinned on d_min (only those chunks read the step scalars, the
    chunk-start d and the retention in the replay)."""
    r = (4 * K if rvec else 4) if apf else 0
    g = 4 if gated else 0
    if name == "precond_scan_kernel":
        # token-by-token phase 1 inside osdn_fwd: reads k, beta, r, writes the
        # bf16 write-key residual
        return elem * K + 4 + r + 2 * K, 0
    if name == "scan_prep_kernel":
        return elem * K + 4 + r, 0
    if name == "scan_factor_kernel":
        # per chunk not pinned by the prep pass: reads k, beta, r and the key
        # norms, writes the 64 x 64 fp32 inverse factor (4 C bytes per token)
        return swept * (elem * K + 4 + 4 + r + 4 * C), 0
    if name == "scan_solve_kernel":
        # vector retention rows are read only for the chunks it sweeps
        return 4 + 4 + (0 if rvec else r), 0
    if name == "scan_emit_kernel":
        return 2 * elem * K + 4 + r, 0
    if name == "chunk_tinv_kernel":
        if not fused:
            # reads k and k~, beta (and alpha)
            return 2 * elem * K + 4 + g, 2 * C * K
        # osdn_fwd (bf16): reads k, forms and writes the residual E = (d-1) k,
        # reads beta (and alpha); a swept chunk also reads its step scalars,
        # retention and chunk-start d
        return 2 * elem * K + 4 + g + swept * (4 + r + 4.0 * K / C), 2 * C * K
    if name == "chunk_sweep_kernel":
        # osdn_fwd reads no write keys for a pinned chunk
        kt = elem * K * (swept if fused else 1.0)
        return elem * (2 * K + V) + kt + 4 + elem * V + g, 2 * (3 * K * V + C * K + 2 * C * V)
    return 0, 0


def decode_work(K, V, T, apf, gated, elem=2):
    """Algorithmic bytes of one osdn_decode call per (b,h)."""
    return 8 * V * K + 8 * K + T * (2 * elem * K + 2 * elem * V + 4 + (4 if apf else 0)
                                    + (4 if gated else 0))


def source_sha(path):
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)


def mfma_file(workload):
    return os.path.join(ROOT, "profiles", "mfma_%s.json" % workload)


def load_traffic(workload, kernel):
    """Measured HBM bytes per launch of `kernel` from the committed counter
    summary, or None when there is none or the kernel source has changed."""
    try:
        with open(traffic_file(workload)) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get("kernels", {}).get(kernel)
    if not ent or kernel not in KERNEL_SOURCE or ent.get("source_sha256") != source_sha(KERNEL_SOURCE[kernel]):
        return None
    return ent


def pmc_summary(fetch_dir, write_dir, workload, command):
    """Turn two rocprofv3 --pmc runs of `bench.py --pmc-pass` (FETCH_SIZE,
    then WRITE_SIZE) into profiles/traffic_<workload>.json."""
    def read(d, counter):
        out = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    name = row["Kernel_Name"].replace("scan_prep128_kernel", "scan_prep_kernel")
                    name = name.replace("scan_solve4_kernel", "scan_solve_kernel")
                    name = name.replace("kda_seq_hilo_kernel", "kda_seq_kernel")
                    name = name.replace("kda_intra128_kernel", "kda_intra_kernel")
                    key = None
                    for k in KERNEL_SOURCE:
                        if k in name:
                            key = k
                    if key is None and ("copy" in name.lower() or "elementwise" in name.lower()):
                        key = "copy"
                    if key:
                        out.setdefault(key, []).append(float(row["Counter_Value"]))
        return out
    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("no calibration copy kernel in the counter runs")
    # counters are in KiB per dispatch; the plain copy moves COPY_BYTES each
    # way (small copies, e.g. input uploads, and the fill are left out)
    def calib(vals):
        big = [v for v in vals if v >= 0.25 * max(vals)]
        return float(np.median(big))
    fscale = COPY_BYTES / (1024.0 * calib(fetch["copy"]))
    wscale = COPY_BYTES / (1024.0 * calib(write["copy"]))
    kernels = {}
    for k in KERNEL_SOURCE:
        if k in fetch and k in write:
            fb = float(np.median(fetch[k])) * 1024.0 * fscale
            wb = float(np.median(write[k])) * 1024.0 * wscale
            kernels[k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                          "fetch_kib_raw": float(np.median(fetch[k])),
                          "write_kib_raw": float(np.median(write[k])),
                          "source": KERNEL_SOURCE[k], "source_sha256": source_sha(KERNEL_SOURCE[k])}
    out = {"workload": workload, "fetch_scale": fscale, "write_scale": wscale,
           "calibration": "plain device copy of %d MiB (torch copy_), counters per dispatch" %
                          (COPY_BYTES >> 20),
           "command": command, "kernels": kernels}
    os.makedirs(os.path.dirname(traffic_file(workload)), exist_ok=True)
    with open(traffic_file(workload), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out, indent=1, sort_keys=True))
    return 0


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
                 "SQ_INSTS_VALU_MFMA_BF16", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")
SIMD_NUM = 1024  # 256 CUs x 4 SIMDs
XCD_NUM = 8      # rocprofv3 reports GRBM_GUI_ACTIVE summed over the eight XCDs


def mfma_summary(pmc_dir, workload, command):
    """Matrix-core counters of one rocprofv3 --pmc run of `bench.py
    --pmc-pass` (MFMA_COUNTERS, one pass) into profiles/mfma_<workload>.json:
    per kernel, the median per dispatch of each counter, the bf16 MFMA flops
    (MOPS x 512), and MFMA busy cycles over (GRBM_GUI_ACTIVE / XCDs) x SIMDs
    (the share of the dispatch's wall time the average SIMD's matrix core was
    busy; the GRBM count as reported is the sum of the eight XCDs' own)."""
    vals = {}
    for path in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row["Kernel_Name"].replace("scan_prep128_kernel", "scan_prep_kernel").replace(
                    "scan_solve4_kernel", "scan_solve_kernel")
                key = None
                for k in KERNEL_SOURCE:
                    if k in name:
                        key = k
                if key and row.get("Counter_Name") in MFMA_COUNTERS:
                    vals.setdefault(key, {}).setdefault(row["Counter_Name"], []).append(
                        float(row["Counter_Value"]))
    kernels = {}
    for k, cs in vals.items():
        med = {c: float(np.median(v)) for c, v in cs.items()}
        ent = {"counters_median_per_dispatch": med, "dispatches": max(len(v) for v in cs.values()),
               "source": KERNEL_SOURCE[k], "source_sha256": source_sha(KERNEL_SOURCE[k])}
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
            ent["bf16_mfma_flops"] = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med and med.get("GRBM_GUI_ACTIVE"):
            ent["gui_active_cycles_per_xcd"] = med["GRBM_GUI_ACTIVE"] / XCD_NUM
            ent["mfma_busy_frac"] = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (med["GRBM_GUI_ACTIVE"] / XCD_NUM * SIMD_NUM)
        kernels[k] = ent
    out = {"workload": workload, "command": command, "simd_num": SIMD_NUM, "xcd_num": XCD_NUM,
           "kernels": kernels}
    with open(mfma_file(workload), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out, indent=1, sort_keys=True))
    return 0


def cpu_baseline(inp, min_seconds):
    """The CPU oracle (fp64, one (b,h) sequence per thread) on the whole
    workload (from its carried state, if any), repeated until `min_seconds`
    of wall time; returns tokens/s, the thread count, the wall time and the
    repetitions."""
    import oracle
    B, T, H, _ = inp["k"].shape
    threads = min(B * H, oracle.default_threads())
    p = inp["params"]
    reps, wall = 0, 0.0
    while wall < min_seconds or reps == 0:
        t0 = time.perf_counter()
        oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["r"], inp["alpha"],
                       inp["d1"], inp["S0"],
                       eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
                       eps=p["eps"], beta_aware=p["beta_aware"], q_scale=p["q_scale"],
                       threads=threads)
        wall += time.perf_counter() - t0
        reps += 1
    return reps * B * T / wall, threads, wall, reps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="named workload (default 1p3b_apf; with --decode decode_1p3b_b256)")
    ap.add_argument("--decode", action="store_true",
                    help="time osdn_decode (one call per step) instead of osdn_fwd")
    ap.add_argument("--kda", action="store_true",
                    help="time osdn_kda_fwd (default workload kda_340m_apf)")
    ap.add_argument("--varlen", action="store_true",
                    help="time osdn_fwd_varlen on a packed batch (default workload varlen_1p3b_65k)")
    ap.add_argument("--backward", action="store_true",
                    help="time osdn_bwd (one call per step) instead of osdn_fwd")
    ap.add_argument("--unfused", action="store_true",
                    help="time osdn_precond_scan then osdn_chunk_fwd (the write keys cross HBM "
                         "in the input dtype) instead of osdn_fwd")
    ap.add_argument("--copies", type=int, default=4,
                    help="input sets rotated between steps (keeps the 256 MB MALL from "
                         "serving repeated reads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=1.5,
                    help="minimum wall time of the CPU oracle run (whole workload, repeated)")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run the steps and a %d MiB calibration copy for rocprofv3 --pmc; "
                         "prints nothing" % (COPY_BYTES >> 20))
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc runs")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="write profiles/mfma_<workload>.json from one rocprofv3 --pmc run of the "
                         "matrix-core counters")
    ap.add_argument("--pmc-command", default="",
                    help="the commands that produced the --pmc-summary runs (recorded)")
    args = ap.parse_args(argv)
    if args.workload is None:
        args.workload = ("decode_1p3b_b256" if args.decode else
                         "varlen_1p3b_65k" if args.varlen else
                         "kda_340m_apf" if args.kda else "1p3b_apf")

    tag = args.workload + ("_unfused" if args.unfused else "")
    if args.pmc_summary:
        return pmc_summary(args.pmc_summary[0], args.pmc_summary[1], tag, args.pmc_command)
    if args.mfma_summary:
        return mfma_summary(args.mfma_summary, tag, args.pmc_command)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the OSDN forward shards over (b,h) with no "
              "communication, so more GPUs just run independent shards; use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import preconditioned_delta_rule_amd as osdn
    from workloads import make_inputs

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
    rvec = apf and inp["r"].ndim == 4
    tdt = torch.bfloat16 if p["dtype"] == "bf16" else torch.float32
    code = osdn.BF16 if p["dtype"] == "bf16" else osdn.F32
    elem = 2 if p["dtype"] == "bf16" else 4

    def up(x, dt):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(dev)

    if args.decode:
        return decode_bench(args, inp, dev)
    if args.backward:
        return bwd_bench(args, inp, dev)
    if args.varlen:
        return varlen_bench(args, inp, dev)
    if args.kda:
        return kda_bench(args, inp, dev)

    sets = []
    for c in range(max(1, args.copies)):
        st = dict(q=up(inp["q"], tdt), k=up(inp["k"], tdt), v=up(inp["v"], tdt),
                  beta=up(inp["beta"], torch.float32), r=up(inp["r"], torch.float32),
                  alpha=up(inp["alpha"], torch.float32),
                  o=torch.empty((B, T, H, V), dtype=tdt, device=dev),
                  S=torch.empty((B, H, V, K), dtype=torch.float32, device=dev),
                  d=torch.empty((B, H, K), dtype=torch.float32, device=dev))
        if args.unfused:
            st["kt"] = torch.empty((B, T, H, K), dtype=tdt, device=dev)
            st["sws"] = torch.empty(osdn.precond_scan_workspace_bytes(B, T, H, K, code),
                                    dtype=torch.uint8, device=dev)
            st["cws"] = torch.empty(max(1, osdn.chunk_fwd_workspace_bytes(B, T, H, K, V, code, C)),
                                    dtype=torch.uint8, device=dev)
        else:
            st["ws"] = torch.empty(osdn.fwd_workspace_bytes(B, T, H, K, V, dtype=code, chunk=C),
                                   dtype=torch.uint8, device=dev)
        sets.append(st)
    kw = dict(chunk=C, eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
              eps=p["eps"], q_scale=p["q_scale"], beta_aware=p["beta_aware"])
    skw = {n: kw[n] for n in ("eta", "d_min", "d_max", "clamp", "eps", "beta_aware")}

    def step(i):
        s = sets[i % len(sets)]
        if args.unfused:
            osdn.precond_scan(s["k"], s["beta"], s["r"], None, k_tilde=s["kt"], d_out=s["d"],
                              workspace=s["sws"], **skw)
            osdn.chunk_fwd(s["q"], s["k"], s["kt"], s["v"], s["beta"], s["alpha"], None, chunk=C,
                           q_scale=p["q_scale"], o=s["o"], S_out=s["S"], workspace=s["cws"])
        else:
            osdn.fwd(s["q"], s["k"], s["v"], s["beta"], s["r"], s["alpha"], None, None,
                     o=s["o"], S_out=s["S"], d_out=s["d"], workspace=s["ws"], **kw)

    if args.pmc_pass:
        for i in range(max(1, args.steps)):
            step(i)
        x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        return 0

    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    nsteps = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    launches = osdn.kernel_times(lambda: [step(i) for i in range(nsteps)], dev)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / nsteps
    log("step %.4f ms (wall %.3f s for %d steps)" % (ms_step, wall, nsteps))

    # which path phase 1 took per 64-token chunk (pinned on d_min, closed form,
    # token by token), summed over (b,h): a pinned chunk reads no step scalar
    if args.unfused:
        cnt = osdn.scan_counters(sets[0]["sws"], B, T, H, K, code).numpy()
    else:
        cnt = osdn.fwd_scan_counters(sets[0]["ws"], B, T, H, K, V, code, C).numpy()
    paths = cnt.reshape(-1, 3).sum(0).tolist()
    swept = 1.0 - paths[0] / max(1, sum(paths))
    log("phase-1 chunks [pinned, closed form, token by token]:", paths)

    # per-kernel durations over the timed steps
    per = {}
    for name, ms in launches:
        per.setdefault(name, []).append(ms)
    per_step = len(launches) // nsteps if nsteps else 0
    step_ms = [sum(ms for _, ms in launches[i * per_step:(i + 1) * per_step]) for i in range(nsteps)]
    nth = B * T * H
    kernels = {}
    for name, vals in per.items():
        ms = float(np.mean(vals))
        nbytes, flops = kernel_work(name, K, V, C, apf, gated, elem, rvec, fused=not args.unfused,
                                    swept=swept)
        gbs = nbytes * nth / (ms * 1e-3) / 1e9 if ms > 0 else None
        ent = {"ms": ms, "launches_per_step": len(vals) / nsteps, "ms_median": float(np.median(vals)),
               "bound": "hbm", "bytes_per_token_head": nbytes, "GB/s": gbs,
               "hbm_frac": gbs / HBM_PEAK_GBS if gbs else None}
        if flops:
            ent["flops_per_token_head"] = flops
            ent["TFLOP/s"] = flops * nth / (ms * 1e-3) / 1e12
            ent["mfma_bf16_frac"] = ent["TFLOP/s"] / MFMA_BF16_PEAK_TFLOPS
        kernels[name] = ent
        log("  %-20s %.4f ms  %.0f GB/s" % (name, ms, gbs or 0))
    dom = max(kernels, key=lambda n: kernels[n]["ms"] * kernels[n]["launches_per_step"])
    dk = kernels[dom]
    tr = load_traffic(tag, dom)
    traffic = tr["bytes_per_launch"] / (dk["ms"] * 1e-3) / 1e9 if tr else None
    roofline = {"bound": "hbm", "kernel": dom, "achieved": dk["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": dk["hbm_frac"], "traffic": traffic,
                "algorithmic_bytes_per_launch": dk["bytes_per_token_head"] * nth,
                "measured_bytes_per_launch": tr["bytes_per_launch"] if tr else None}
    p1 = sum(kernels[n]["ms"] * kernels[n]["launches_per_step"] for n in kernels if n.startswith("scan_"))
    p2 = sum(kernels[n]["ms"] * kernels[n]["launches_per_step"] for n in kernels if n.startswith("chunk_"))

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu oracle on the whole workload (%d sequences x %d tokens)" % (B * H, T))
        tps, threads, cwall, reps = cpu_baseline(inp, args.cpu_seconds)
        cpu = {"value": tps, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": "whole workload: %d (b,h) sequences x %d tokens, fp64 sequential oracle "
                         "(both phases), one sequence per thread, %d run(s) in %.2f s wall" %
                         (B * H, T, reps, cwall)}
        log("cpu oracle %.2f s" % cwall)

    metric = METRIC if (H, K, V, T) == (16, 128, 128, 4096) else (
        "OSDN fwd tokens/sec (phase1+phase2) at H=%d,K=%d,V=%d,T=%d; %% HBM/MFMA roofline" % (H, K, V, T))
    out = {
        "metric": metric, "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": nsteps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": p["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V,
                   "chunk": C, "apf": apf, "vector_retention": rvec, "gated": gated, "seed": spec["seed"],
                   "input_copies": len(sets),
                   "path": "unfused (osdn_precond_scan + osdn_chunk_fwd)" if args.unfused else "osdn_fwd",
                   "phase1_chunks_pinned_closed_token": paths},
        "roofline": roofline, "cpu_baseline": cpu,
        "phases": {"precond_scan_ms": p1, "chunk_fwd_ms": p2,
                   "step_device_ms_median": float(np.median(step_ms)) if step_ms else None,
                   "step_device_ms_p10": float(np.percentile(step_ms, 10)) if step_ms else None,
                   "step_device_ms_p90": float(np.percentile(step_ms, 90)) if step_ms else None},
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)
    return 0


def kda_work(name, K, V, C=64, elem=2):
    """Algorithmic (bytes, flops) per (token, head) of the OSKDA kernels.
    Sweep: X = V - (Gamma.K)S and P = (Gamma.Q)S (2KV flops each), D = TB X and
    M D (lower-triangular C x C times V: (C+1)V each), S += Kc^T D (2KV); it
    reads the fp32 chunk operands (Gamma.K, Gamma.Q, Kc: 3K floats per token;
    TB, M: 2C; gamma_C: K/C) and v, writes o.  Intra: reads q, k, the bf16
    write-key residual, alpha (K floats) and beta, writes those operands; its
    Gram and scores are the 10 lower 16x16 blocks of two C x C x K products.
    The intra count is that of the bf16 path, which forms the write-key
    residual itself (q, k, alpha, beta, the phase-1 step scalar and the
    retention in; no residual read)."""
    if name.startswith("kda_seq"):
        nbytes = 4 * (3 * K + 2 * C) + 4 * K / C + 2 * elem * V
        flops = 6 * K * V + 2 * (C + 1) * V
        return nbytes, flops
    if name.startswith("kda_intra"):
        nbytes = 2 * elem * K + 4 * K + 4 + 4 + 4 + 4 * (3 * K + 2 * C) + 4 * K / C
        flops = 2 * 2 * 10 * 16 * 16 * K / C
        return nbytes, flops
    return kernel_work(name, K, V, C, True, False, elem)


def kda_bench(args, inp, dev):
    """--kda: one osdn_kda_fwd call per step."""
    import torch
    import preconditioned_delta_rule_amd as osdn
    spec, p = inp["spec"], inp["params"]
    B, T, H, K = inp["k"].shape
    V = inp["v"].shape[-1]
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
                         S=torch.empty((B, H, K, V), dtype=torch.float32, device=dev),
                         d=torch.empty((B, H, K), dtype=torch.float32, device=dev)))
    ws = torch.empty(osdn.kda_fwd_workspace_bytes(B, T, H, K, V, dtype=osdn.BF16 if elem == 2 else osdn.F32),
                     dtype=torch.uint8, device=dev)
    kw = dict(eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
              q_scale=p["q_scale"], beta_aware=p["beta_aware"])

    def step(i):
        s = sets[i % len(sets)]
        osdn.kda_fwd(s["q"], s["k"], s["v"], s["beta"], s["r"], s["alpha"], o=s["o"], S_out=s["S"],
                     d_out=s["d"], workspace=ws, **kw)

    if args.pmc_pass:
        for i in range(max(1, args.steps)):
            step(i)
        x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        return 0

    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    nsteps = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launches = osdn.kernel_times(lambda: [step(i) for i in range(nsteps)], dev)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / nsteps
    nth = B * T * H
    kernels = {}
    for name in sorted(set(n for n, _ in launches)):
        vals = [ms for n, ms in launches if n == name]
        ms = float(np.mean(vals))
        nbytes, flops = kda_work(name, K, V, 64, elem)
        gbs = nbytes * nth / (ms * 1e-3) / 1e9 if ms > 0 else None
        ent = {"ms": ms, "bytes_per_token_head": nbytes, "GB/s": gbs,
               "hbm_frac": gbs / HBM_PEAK_GBS if gbs else None}
        if flops and name.startswith("kda_"):
            # the sweep multiplies bf16 hi/lo pairs for bf16 inputs, fp32 otherwise;
            # the intra kernel's Gram runs fp32 matrix instructions
            peak = MFMA_BF16_PEAK_TFLOPS if (elem == 2 and name.startswith("kda_seq")) else FP32_VALU_PEAK_TFLOPS
            ent["flops_per_token_head"] = flops
            ent["TFLOP/s"] = flops * nth / (ms * 1e-3) / 1e12
            ent["mfma_peak_TFLOP/s"] = peak
            ent["mfma_frac"] = ent["TFLOP/s"] / peak
        kernels[name] = ent
        log("  %-20s %.4f ms  %.0f GB/s" % (name, ms, gbs or 0))
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    dk = kernels[dom]
    if dk.get("mfma_frac", 0.0) > dk["hbm_frac"]:
        roofline = {"bound": "mfma", "kernel": dom, "achieved": dk["TFLOP/s"], "peak": dk["mfma_peak_TFLOP/s"],
                    "unit": "TFLOP/s", "frac": dk["mfma_frac"], "traffic": None,
                    "algorithmic_flops_per_launch": dk["flops_per_token_head"] * nth}
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": dk["GB/s"], "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": dk["hbm_frac"], "traffic": None,
                    "algorithmic_bytes_per_launch": dk["bytes_per_token_head"] * nth}
    tr = load_traffic(args.workload, dom)
    if tr:
        roofline["traffic"] = tr["bytes_per_launch"] / (dk["ms"] * 1e-3) / 1e9
        roofline["measured_bytes_per_launch"] = tr["bytes_per_launch"]
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        sl = lambda z: None if z is None else np.ascontiguousarray(z[:1])
        reps, wall = 0, 0.0
        while wall < args.cpu_seconds or reps == 0:
            t0 = time.perf_counter()
            oracle.kda_forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl(inp["r"]),
                               sl(inp["alpha"]), eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"],
                               clamp=p["clamp"], eps=p["eps"], beta_aware=p["beta_aware"],
                               q_scale=p["q_scale"], threads=min(H, oracle.default_threads()))
            wall += time.perf_counter() - t0
            reps += 1
        cpu = {"value": reps * T / wall, "unit": "tokens/s", "cores": min(H, oracle.default_threads()),
               "kind": "oracle",
               "sample": "batch element 0 (%d tokens, all %d heads), fp64 oracle, one head per thread, "
                         "%d run(s) in %.2f s" % (T, H, reps, wall)}
    out = {
        "metric": KDA_METRIC, "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": nsteps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p["dtype"], "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V,
                   "apf": inp["r"] is not None, "seed": spec["seed"], "input_copies": len(sets)},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(out), flush=True)
    return 0


def varlen_bench(args, inp, dev):
    """--varlen: one osdn_fwd_varlen call per step on a packed batch."""
    import torch
    import preconditioned_delta_rule_amd as osdn
    from workloads import varlen_lengths
    spec, p = inp["spec"], inp["params"]
    _, total, H, K = inp["k"].shape
    V = inp["v"].shape[-1]
    apf, gated = inp["r"] is not None, inp["alpha"] is not None
    tdt = torch.bfloat16 if p["dtype"] == "bf16" else torch.float32
    elem = 2 if p["dtype"] == "bf16" else 4
    lens = varlen_lengths(total, seed=spec["seed"] + 3)
    S, Tmax = len(lens), max(lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64, device=dev)

    def up(x, dt):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(dev)

    s = dict(q=up(inp["q"], tdt), k=up(inp["k"], tdt), v=up(inp["v"], tdt),
             beta=up(inp["beta"], torch.float32), r=up(inp["r"], torch.float32),
             alpha=up(inp["alpha"], torch.float32), o=torch.empty((1, total, H, V), dtype=tdt, device=dev),
             S=torch.empty((S, H, V, K), dtype=torch.float32, device=dev),
             d=torch.empty((S, H, K), dtype=torch.float32, device=dev))
    ws = torch.empty(osdn.fwd_workspace_bytes(S, Tmax, H, K, V, dtype=osdn.BF16 if elem == 2 else osdn.F32,
                                              chunk=p["chunk"]),
                     dtype=torch.uint8, device=dev)
    kw = dict(chunk=p["chunk"], eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"],
              eps=p["eps"], q_scale=p["q_scale"], beta_aware=p["beta_aware"])

    def step(i):
        osdn.fwd_varlen(s["q"], s["k"], s["v"], s["beta"], s["r"], s["alpha"], cu_seqlens=cu,
                        max_seqlen=Tmax, o=s["o"], S_out=s["S"], d_out=s["d"], workspace=ws, **kw)

    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    nsteps = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launches = osdn.kernel_times(lambda: [step(i) for i in range(nsteps)], dev)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / nsteps
    nth = total * H
    kernels = {}
    for name in sorted(set(n for n, _ in launches)):
        vals = [ms for n, ms in launches if n == name]
        ms = float(np.mean(vals))
        nbytes, flops = kernel_work(name, K, V, p["chunk"], apf, gated, elem)
        gbs = nbytes * nth / (ms * 1e-3) / 1e9 if ms > 0 else None
        kernels[name] = {"ms": ms, "bytes_per_token_head": nbytes, "GB/s": gbs,
                         "hbm_frac": gbs / HBM_PEAK_GBS if gbs else None}
        log("  %-20s %.4f ms  %.0f GB/s" % (name, ms, gbs or 0))
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    dk = kernels[dom]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": dk["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": dk["hbm_frac"], "traffic": None,
                "algorithmic_bytes_per_launch": dk["bytes_per_token_head"] * nth}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # a bounded sample: the first two sequences, all heads
        a, b = 0, int(cu[2].item()) if S > 1 else total
        reps, wall = 0, 0.0
        while wall < args.cpu_seconds or reps == 0:
            t0 = time.perf_counter()
            for i in range(min(2, S)):
                x, y = int(cu[i].item()), int(cu[i + 1].item())
                sl = lambda z: None if z is None else np.ascontiguousarray(z[:, x:y])
                oracle.forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl(inp["r"]),
                               sl(inp["alpha"]), eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"],
                               clamp=p["clamp"], eps=p["eps"], beta_aware=p["beta_aware"],
                               q_scale=p["q_scale"], threads=min(H, oracle.default_threads()))
            wall += time.perf_counter() - t0
            reps += 1
        cpu = {"value": reps * (b - a) / wall, "unit": "tokens/s", "cores": min(H, oracle.default_threads()),
               "kind": "oracle",
               "sample": "the first two sequences (%d tokens, all %d heads), fp64 oracle, one (sequence, "
                         "head) per thread, %d run(s) in %.2f s" % (b - a, H, reps, wall)}
    out = {
        "metric": VARLEN_METRIC, "value": total / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": nsteps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p["dtype"], "data": "synthetic",
        "config": {"workload": args.workload, "total_tokens": total, "sequences": S, "max_seqlen": Tmax,
                   "H": H, "K": K, "V": V, "apf": apf, "gated": gated, "seed": spec["seed"]},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(out), flush=True)
    return 0


def bwd_work(name, K, V, elem=2):
    """(algorithmic bytes, fp32 flops) per token-head of a backward kernel."""
    if name == "bwd_record_kernel":
        # k, v in; u out (fp32); state and d recorded every 16 tokens
        return elem * (K + V) + 4 + 4 + 4 * V + (4 * V * K + 4 * K) / 16, 6 * V * K
    if name == "bwd_p2_kernel":
        # q, k, dout, u in; dq, dv out; dk~ and the read-key part out (fp32);
        # a recorded state read every 16 tokens
        return (elem * (2 * K + V) + 4 * V + elem * (K + V) + 8 * K + 12 + (4 * V * K + 4 * K) / 16,
                14 * V * K)
    if name == "bwd_p1_kernel":
        # k, dk~, read-key part, phase-2 dbeta in; dk, dbeta, dr out
        return elem * K + 8 * K + 4 + 8 + elem * K + 8, 30 * K
    return 0, 0


def bwd_bench(args, inp, dev):
    """--backward: one osdn_bwd call per step on the forward's workload."""
    import torch
    import preconditioned_delta_rule_amd as osdn
    from workloads import random_cotangent
    spec, p = inp["spec"], inp["params"]
    B, T, H, K = inp["k"].shape
    V = inp["v"].shape[-1]
    apf, gated = inp["r"] is not None, inp["alpha"] is not None
    tdt = torch.bfloat16 if p["dtype"] == "bf16" else torch.float32
    code = osdn.BF16 if p["dtype"] == "bf16" else osdn.F32
    elem = 2 if p["dtype"] == "bf16" else 4
    dout, dS, dd = random_cotangent(inp, seed=spec["seed"] + 2)

    def up(x, dt):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(dev)

    s = dict(q=up(inp["q"], tdt), k=up(inp["k"], tdt), v=up(inp["v"], tdt),
             beta=up(inp["beta"], torch.float32), r=up(inp["r"], torch.float32),
             alpha=up(inp["alpha"], torch.float32), dout=up(dout, tdt),
             dS=up(dS, torch.float32), dd=up(dd, torch.float32))
    ws = torch.empty(osdn.bwd_workspace_bytes(B, T, H, K, V, code), dtype=torch.uint8, device=dev)
    kw = dict(eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
              q_scale=p["q_scale"], beta_aware=p["beta_aware"])

    def step(i):
        osdn.bwd(s["q"], s["k"], s["v"], s["beta"], s["r"], s["alpha"], None, None, dout=s["dout"],
                 dS=s["dS"], dd=s["dd"], workspace=ws, **kw)

    if args.pmc_pass:
        for i in range(max(1, args.steps)):
            step(i)
        torch.cuda.synchronize()
        return 0
    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    nsteps = args.steps
    log("timing %d backward calls" % nsteps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launches = osdn.kernel_times(lambda: [step(i) for i in range(nsteps)], dev)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / nsteps
    nth = B * T * H
    kernels = {}
    for name in ("bwd_record_kernel", "bwd_p2_kernel", "bwd_p1_kernel"):
        vals = [ms for n, ms in launches if n == name]
        ms = float(np.mean(vals))
        nbytes, flops = bwd_work(name, K, V, elem)
        kernels[name] = {"ms": ms, "ms_median": float(np.median(vals)),
                         "bytes_per_token_head": nbytes, "GB/s": nbytes * nth / (ms * 1e-3) / 1e9,
                         "flops_per_token_head": flops,
                         "TFLOP/s": flops * nth / (ms * 1e-3) / 1e12}
        kernels[name]["valu_fp32_frac"] = kernels[name]["TFLOP/s"] / FP32_VALU_PEAK_TFLOPS
        kernels[name]["hbm_frac"] = kernels[name]["GB/s"] / HBM_PEAK_GBS
        log("  %-18s %.4f ms  %.1f TFLOP/s  %.0f GB/s" % (name, ms, kernels[name]["TFLOP/s"],
                                                        kernels[name]["GB/s"]))
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    dk = kernels[dom]
    roofline = {"bound": "alu", "kernel": dom, "achieved": dk["TFLOP/s"], "peak": FP32_VALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": dk["valu_fp32_frac"], "traffic": None,
                "algorithmic_flops_per_launch": dk["flops_per_token_head"] * nth}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # a bounded sample: two whole (b,h) sequences of the workload
        pairs = [(0, 0), (B - 1, H - 1)]
        from workloads import sample_sequences
        sub = sample_sequences(dict(inp), pairs)
        sd = np.stack([dout[b, :, h] for b, h in pairs])[:, :, None, :]
        reps, wall = 0, 0.0
        while wall < args.cpu_seconds or reps == 0:
            t0 = time.perf_counter()
            oracle.backward(sub["q"], sub["k"], sub["v"], sub["beta"], sub["r"], sub["alpha"],
                            dout=sd, eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"],
                            clamp=p["clamp"], eps=p["eps"], beta_aware=p["beta_aware"],
                            q_scale=p["q_scale"], threads=len(pairs))
            wall += time.perf_counter() - t0
            reps += 1
        # tokens/s of the whole layer at this rate: B*T tokens carry B*H sequences
        cpu = {"value": reps * len(pairs) * T / wall / H, "unit": "tokens/s", "cores": len(pairs),
               "kind": "oracle",
               "sample": "%d whole (b,h) sequences of %d tokens, fp64 oracle backward (forward "
                         "replay included), one sequence per thread, %d run(s) in %.2f s; scaled to "
                         "layer tokens/s as sequences/s x T / H" % (len(pairs), T, reps, wall)}
    out = {
        "metric": BWD_METRIC, "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": nsteps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p["dtype"], "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V, "apf": apf,
                   "gated": gated, "seed": spec["seed"]},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(out), flush=True)
    return 0


def decode_bench(args, inp, dev):
    """--decode: one osdn_decode call per step on a decode workload."""
    import torch
    import preconditioned_delta_rule_amd as osdn
    spec, p = inp["spec"], inp["params"]
    B, T, H, K = inp["k"].shape
    V = inp["v"].shape[-1]
    apf, gated = inp["r"] is not None, inp["alpha"] is not None
    tdt = torch.bfloat16 if p["dtype"] == "bf16" else torch.float32
    elem = 2 if p["dtype"] == "bf16" else 4

    def up(x, dt):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(dev)

    sets = [dict(q=up(inp["q"], tdt), k=up(inp["k"], tdt), v=up(inp["v"], tdt),
                 beta=up(inp["beta"], torch.float32), r=up(inp["r"], torch.float32),
                 alpha=up(inp["alpha"], torch.float32),
                 o=torch.empty((B, T, H, V), dtype=tdt, device=dev))
            for _ in range(max(1, args.copies))]
    # two state buffers in turn: each call reads what the previous one wrote
    S = [up(inp["S0"], torch.float32), torch.empty((B, H, V, K), dtype=torch.float32, device=dev)]
    d = [up(inp["d1"], torch.float32), torch.empty((B, H, K), dtype=torch.float32, device=dev)]
    kw = dict(eta=p["eta"], d_min=p["d_min"], d_max=p["d_max"], clamp=p["clamp"], eps=p["eps"],
              q_scale=p["q_scale"], beta_aware=p["beta_aware"])

    def step(i):
        s = sets[i % len(sets)]
        a, b = i % 2, (i + 1) % 2
        osdn.decode(s["q"], s["k"], s["v"], s["beta"], s["r"], s["alpha"], d[a], S[a],
                    o=s["o"], S_out=S[b], d_out=d[b], **kw)

    if args.pmc_pass:
        for i in range(max(1, args.steps)):
            step(i)
        x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        return 0

    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    nsteps = args.steps
    log("timing %d decode calls" % nsteps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launches = osdn.kernel_times(lambda: [step(i) for i in range(nsteps)], dev)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / nsteps
    ks = [ms for name, ms in launches if name == "decode_kernel"]
    kms = float(np.mean(ks))
    per_seq = decode_work(K, V, T, apf, gated, elem)
    alg = per_seq * B * H
    gbs = alg / (kms * 1e-3) / 1e9
    log("call %.4f ms, kernel %.4f ms, %.0f GB/s" % (ms_step, kms, gbs))
    tr = load_traffic(args.workload, "decode_kernel")
    roofline = {"bound": "hbm", "kernel": "decode_kernel", "achieved": gbs, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "traffic": tr["bytes_per_launch"] / (kms * 1e-3) / 1e9 if tr else None,
                "algorithmic_bytes_per_launch": alg,
                "measured_bytes_per_launch": tr["bytes_per_launch"] if tr else None}
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu oracle on the whole decode workload (%d sequences x %d tokens)" % (B * H, T))
        tps, threads, cwall, reps = cpu_baseline(inp, args.cpu_seconds)
        cpu = {"value": tps, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": "whole workload: %d (b,h) sequences x %d new token(s) from the carried "
                         "state, fp64 sequential oracle, one sequence per thread, %d run(s) in "
                         "%.2f s wall" % (B * H, T, reps, cwall)}
    out = {
        "metric": DECODE_METRIC, "value": B * T / (ms_step * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": nsteps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": p["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V,
                   "apf": apf, "gated": gated, "seed": spec["seed"], "input_copies": len(sets)},
        "roofline": roofline, "cpu_baseline": cpu,
        "kernels": {"decode_kernel": {"ms": kms, "ms_median": float(np.median(ks)),
                                      "ms_p10": float(np.percentile(ks, 10)),
                                      "ms_p90": float(np.percentile(ks, 90)),
                                      "bytes_per_sequence": per_seq, "GB/s": gbs}},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
