"""Build libosdn.so: the gfx950 HIP kernels plus the C ABI (include/osdn.h).

Every source is compiled with hipcc for gfx950 only, with packed fp32 vector
instructions disabled, into objects under _build/, then linked into
preconditioned_delta_rule_amd/libosdn.so next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libosdn.so")

SOURCES = ["precond_scan.hip", "precond_chunked.hip", "chunk_generic.hip", "chunk_mfma.hip",
           "chunk_wy.hip", "decode.hip", "backward.hip", "kda_chunk.hip", "osdn_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libosdn.so)")


def common_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link libosdn.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
