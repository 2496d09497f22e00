"""Host logic of bench.py (CPU only): the one-GPU contract, and the algorithmic
byte and flop counts its rooflines are built on, checked against the sizes of
the operands each kernel must move (K = V = 128, 64-token chunks, bf16)."""
import subprocess
import sys

import pytest

import bench
from workloads import varlen_lengths

ROOT = bench.ROOT


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                         text=True, timeout=120)
    assert res.returncode != 0 and "one GPU" in res.stderr and res.stdout == ""


def test_forward_sweep_bytes():
    # q, k, E (bf16 residual) and v in (4 x 256 B), beta (4 B), o out (256 B)
    assert bench.kernel_work("chunk_sweep_kernel", 128, 128, 64, True, False)[0] == 1284
    # alpha adds 4 B per token-head
    assert bench.kernel_work("chunk_sweep_kernel", 128, 128, 64, True, True)[0] == 1288
    # inside osdn_fwd a chunk phase 1 took as pinned reads no write keys
    assert bench.kernel_work("chunk_sweep_kernel", 128, 128, 64, True, False, swept=0.0)[0] == 1028
    assert bench.kernel_work("chunk_sweep_kernel", 128, 128, 64, True, False, fused=False, swept=0.0)[0] == 1284


def test_forward_tinv_bytes():
    # osdn_fwd: k in, E out (2 x 256 B), beta; a swept chunk adds its step
    # scalar, retention and chunk-start d (512 B per 64 tokens)
    assert bench.kernel_work("chunk_tinv_kernel", 128, 128, 64, True, False, swept=0.0)[0] == 516
    assert bench.kernel_work("chunk_tinv_kernel", 128, 128, 64, True, False, swept=1.0)[0] == 516 + 4 + 4 + 8
    # vector retention: a [K] row per token, read only for swept chunks
    assert bench.kernel_work("chunk_tinv_kernel", 128, 128, 64, True, False, 2, True, swept=0.5)[0] == \
        516 + 0.5 * (4 + 512 + 8)
    # osdn_chunk_fwd: k and k~ in, beta
    assert bench.kernel_work("chunk_tinv_kernel", 128, 128, 64, True, False, fused=False)[0] == 516


def test_phase1_bytes_scalar_and_vector_retention():
    # prep: k (256 B), beta, r
    assert bench.kernel_work("scan_prep_kernel", 128, 128, 64, True, False)[0] == 256 + 4 + 4
    assert bench.kernel_work("scan_prep_kernel", 128, 128, 64, True, False, 2, True)[0] == 256 + 4 + 512
    # solve reads the retention rows only for swept chunks
    assert bench.kernel_work("scan_solve_kernel", 128, 128, 64, True, False, 2, True)[0] == 8
    # token-by-token phase 1: k, beta, r row, residual out
    assert bench.kernel_work("precond_scan_kernel", 128, 128, 64, True, False, 2, True)[0] == 256 + 4 + 512 + 256


def test_oskda_work_counts():
    nbytes, flops = bench.kda_work("kda_seq_kernel", 128, 128, 64, 2)
    # fp32 Gamma.K, Gamma.Q, Kc^T (3 x 512 B), TB and M rows (2 x 256 B),
    # gamma_C (512 B per 64 tokens), v and o (2 x 256 B)
    assert nbytes == 1536 + 512 + 8 + 512
    # X and P (2KV each), D and M D ((C+1)V each), state update (2KV)
    assert flops == 6 * 128 * 128 + 2 * 65 * 128 == 114944
    nbytes, flops = bench.kda_work("kda_intra_kernel", 128, 128, 64, 2)
    # q, k (2 x 256 B), alpha (512 B), beta, step scalar, retention; operands out
    assert nbytes == 2 * 256 + 512 + 12 + 2048 + 8 == 3092
    assert flops == 20480


def test_decode_bytes():
    # state read and written (2 x 64 KiB), d (2 x 512 B), q, k, v, o rows, beta, r
    assert bench.decode_work(128, 128, 1, True, False) == 133128


def test_varlen_lengths():
    for seed in range(5):
        lens = varlen_lengths(65536, seed=seed)
        assert sum(lens) == 65536
        assert all(1 <= n <= 4096 for n in lens)
        assert all(n >= 256 for n in lens[:-1])
    assert varlen_lengths(65536, seed=11) == varlen_lengths(65536, seed=11)
