"""The C ABI used from C++ alone: tests/c_abi/abi_roundtrip (built by
__graft_entry__.build()) links libqgemm.so, allocates with hipMalloc, and
calls qg_pack and qg_gemm_int4 / qg_gemm_int2 through include/qgemm.h with no
Python or torch in the process.  Its pack must equal the oracle's bit for
bit and its GEMM meet the GEMM tolerance, on the GEMV, skinny and tiled
paths.  In its --loop mode it packs a block, re-quantises it to INT2 when
asked, and runs qg_loop_range; h must meet the loop tolerance against the
oracle's loop driver on the same (re-quantised) weights."""
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


@pytest.mark.parametrize("bits,M,D,F,L0,L1", [(4, 1, 1024, 4096, 0, 3), (2, 5, 512, 1536, 1, 3),
                                              (4, 40, 768, 1536, 0, 2), (2, 1, 2048, 8192, 0, 2),
                                              (4, 200, 1024, 2048, 2, 3)])
def test_c_abi_loop(orc, tmp_path, bits, M, D, F, L0, L1):
    assert os.path.exists(EXE), f"{EXE} missing: run __graft_entry__.build()"
    inp = workloads.block(M, seed=M + D + F + bits, D=D, F=F)
    names = ("qkv", "out", "up", "down")
    h0 = inp.X.numpy().astype(np.float32)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([D, F, M, bits, L0, L1], np.int32).tobytes())
        for k in names:
            f.write(inp.W[k].numpy().astype(np.float32).tobytes())
        f.write(h0.tobytes())
    r = subprocess.run([EXE, "--loop", str(src), str(dst)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    h = np.frombuffer(open(dst, "rb").read(), np.float32, M * D).reshape(M, D)
    oblk = orc.pack_block({k: inp.W[k].numpy() for k in names}, 4, D, F)
    if bits == 2:
        oblk = orc.Block(D, F, *(orc.requant_4to2(getattr(oblk, k)) for k in names))
    href, _ = orc.loop_range(oblk, h0.astype(np.float64), L0, L1)
    rms = float(np.sqrt(np.mean(href ** 2)))
    assert_close(h.astype(np.float64), href, f"c abi loop bits={bits} M={M} D={D}",
                 max_abs=1e-2 * max(1.0, rms))
