"""Builds abi_roundtrip, the C ABI driver used by tests/test_gpu_c_abi.py:
host code only, compiled against include/qgemm.h and linked to
int2_quantized_gemm_amd/libqgemm.so (found at run time through its rpath)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_roundtrip.cpp")
EXE = os.path.join(HERE, "abi_roundtrip")


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    lib_dir = os.path.join(ROOT, "int2_quantized_gemm_amd")
    cmd = [hipcc, "-O2", "-std=c++17", "-Wall", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), SRC, "-o", EXE + ".tmp",
           "-L", lib_dir, "-lqgemm", "-Wl,-rpath,$ORIGIN/../../int2_quantized_gemm_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on abi_roundtrip.cpp")
    os.replace(EXE + ".tmp", EXE)
    if verbose:
        print(f"built {EXE}")
    return EXE


if __name__ == "__main__":
    build(verbose=True)
