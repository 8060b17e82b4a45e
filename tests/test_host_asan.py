"""The library's host code under AddressSanitizer (CPU, no GPU): the C-ABI
validation tests of test_abi.py, run against a host-instrumented build of
the same sources with the clang ASan runtime preloaded.  Any heap or stack
error in argument validation, size arithmetic or error reporting aborts the
run with an ASan report."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "asan"))
import build_host_asan  # noqa: E402


@pytest.mark.skipif(build_host_asan.asan_runtime() is None, reason="clang ASan runtime not installed")
def test_abi_validation_under_host_asan(tmp_path):
    lib = build_host_asan.main(str(tmp_path))
    env = dict(os.environ, QG_LIBRARY=lib, LD_PRELOAD=build_host_asan.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    root = os.path.dirname(HERE)
    # the library is instrumented, and it is the one the binding loads, with
    # the runtime in the process
    und = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in und and "__asan_report_store" in und
    r = subprocess.run([sys.executable, "-c", "import ctypes, int2_quantized_gemm_amd as q; "
                        "print(q.LIB_PATH); print(ctypes.CDLL(None).__asan_init is not None)"],
                       cwd=root, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == [lib, "True"], r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py"), "-m", "not gpu",
                        "-k", "not fails_loudly and not reference_the_oracle"],
                       cwd=root, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "AddressSanitizer" not in r.stdout + r.stderr, \
        (r.stdout[-3000:] + r.stderr[-3000:])
