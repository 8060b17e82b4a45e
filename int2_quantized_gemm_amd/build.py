"""Compile the HIP sources under csrc/ into libqgemm.so for gfx950 (in-tree).

hipcc cross-compiles without a GPU.  Every source is built with
`-Xclang -target-feature -Xclang -packed-fp32-ops` so that no packed FP32
instruction is generated, and without fast-math so that FP64 division and
rounding in the quantiser are IEEE-exact.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqgemm.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["qgemm.hip", "kernels_pack.hip", "kernels_gemm.hip", "kernels_gemv.hip",
           "kernels_prefill.hip", "kernels_loop.hip", "kernels_requant.hip"]
ARCH = os.environ.get("QG_OFFLOAD_ARCH", "gfx950")
# read-only bandwidth probe used by bench.py for its memory ceilings
BENCH_SOURCE = "membench.hip"
BENCH_LIB = os.path.join(HERE, "libqgbench.so")

CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=on",
]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    # the benchmark's read-bandwidth probe, a library of its own
    obj = _compile(BENCH_SOURCE)
    tmp = BENCH_LIB + ".tmp"
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed (bench probe)")
    os.replace(tmp, BENCH_LIB)
    if verbose:
        print(f"built {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
