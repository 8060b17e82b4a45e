"""Host-side AddressSanitizer build of the library, for the CPU test suite.

Compiles the HIP sources with the host code instrumented (each sanitizer
flag directly after -Xarch_host; the device code is built as usual, since
the host code registers it): every C-ABI entry point's host path --
argument validation, size and layout arithmetic, error reporting -- runs
under ASan, loaded from Python with the clang ASan runtime preloaded.  Usage:
    python tests/asan/build_host_asan.py OUT_DIR   -> OUT_DIR/libqgemm_asan.so
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.join(ROOT, "int2_quantized_gemm_amd"))
import build  # noqa: E402  (the library's own source list)

ASAN_HOST = ["-Xarch_host -fsanitize=address", "-Xarch_host -fno-omit-frame-pointer"]


def asan_runtime() -> str | None:
    """The clang ASan runtime matching hipcc's host compiler, if installed."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def main(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    flags = ["-O1", "-g", "-std=c++17", f"--offload-arch={build.ARCH}",
             "-fPIC", "-fno-fast-math"]
    for f in ASAN_HOST:
        flags += f.split()

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([build._hipcc(), *flags, "-c", os.path.join(build.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (host ASan) failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, build.SOURCES))
    lib = os.path.join(out_dir, "libqgemm_asan.so")
    r = subprocess.run([build._hipcc(), f"--offload-arch={build.ARCH}", "-shared", "-fPIC", "-o", lib,
                        *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (host ASan) failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(main(sys.argv[1]))
