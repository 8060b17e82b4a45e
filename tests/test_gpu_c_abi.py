"""The C ABI used from C++ alone: tests/c_abi/abi_roundtrip (built by
__graft_entry__.build()) links libqgemm.so, allocates with hipMalloc, and
calls qg_pack and qg_gemm_int4 / qg_gemm_int2 through include/qgemm.h with no
Python or torch in the process.  Its pack must equal the oracle's bit for
bit and its GEMM meet the GEMM tolerance, on the GEMV, skinny and tiled
paths."""
import os
import subprocess

import numpy as np
import pytest

import workloads
from conftest import ROOT
from helpers import assert_close

pytestmark = pytest.mark.gpu

EXE = os.path.join(ROOT, "tests", "c_abi", "abi_roundtrip")


@pytest.mark.parametrize("bits,M,K,N", [(4, 1, 2048, 2048), (2, 1, 1024, 520),
                                        (4, 16, 2048, 512), (2, 7, 4096, 264),
                                        (4, 300, 1024, 1032), (2, 129, 2048, 776)])
def test_c_abi_roundtrip(orc, tmp_path, bits, M, K, N):
    assert os.path.exists(EXE), f"{EXE} missing: run __graft_entry__.build()"
    W, X = workloads.single_gemm(M, K, N, seed=M + K + N + bits)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([K, N, M, bits], np.int32).tobytes())
        f.write(W.numpy().astype(np.float32).tobytes())
        f.write(X.numpy().view(np.uint16).tobytes())
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(dst, "rb").read()
    nc, ns = N * K * bits // 32, N * (K // 128)
    codes = np.frombuffer(raw, np.uint32, nc, 0).reshape(N, -1)
    scales = np.frombuffer(raw, np.uint16, ns, nc * 4).reshape(N, -1)
    zeros = np.frombuffer(raw, np.uint16, ns, nc * 4 + ns * 2).reshape(N, -1)
    Y = np.frombuffer(raw, np.float16, M * N, nc * 4 + ns * 4).reshape(M, N)
    op = orc.pack(W.numpy(), bits)
    assert np.array_equal(codes, op.codes) and np.array_equal(scales, op.scales)
    assert np.array_equal(zeros, op.zeros)
    assert_close(Y.astype(np.float64), orc.gemm(X.numpy(), op), f"c abi bits={bits} M={M}")
