"""qg_gemm_static_ws -- the GEMM on the library's static device workspace,
for callers that cannot allocate -- against qg_gemm_int4 / qg_gemm_int2 with
a caller workspace (the same kernels: results must agree bit for bit) and
against the FP64 oracle, on consecutive calls whose second input is smaller
than the first, so that a stale or mis-sized workspace would show."""
import numpy as np
import pytest
import torch

from helpers import assert_close, f16_bits, to_oracle

pytestmark = pytest.mark.gpu

qg = pytest.importorskip("int2_quantized_gemm_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda")


# (bits, [(M, K, N) of consecutive calls, the second smaller]); each first
# shape splits K, so the static workspace is really used.
CASES = [
    (4, [(256, 8192, 2048), (16, 8192, 2048)]),   # 128-row tiles with K split, then skinny parts
    (2, [(128, 8192, 2048), (24, 2048, 6144)]),   # INT2 ring tiles with K split, then fewer rows
    (4, [(96, 8192, 2048), (1, 8192, 2048)]),     # split, then the GEMV (no workspace)
]


@pytest.mark.parametrize("bits,shapes", CASES)
def test_static_ws_matches_caller_workspace(dev, orc, bits, shapes):
    import workloads
    ref_fn = qg.qg_gemm_int4 if bits == 4 else qg.qg_gemm_int2
    used = False
    for i, (M, K, N) in enumerate(shapes):
        W, X = workloads.single_gemm(M, K, N, seed=40 + i)
        p = qg.qg_pack(W.to(dev), bits)
        Xd = X.to(dev)
        used |= qg.qg_gemm_ws_bytes(p, M) > 0
        Y_ref = ref_fn(Xd, p)
        Y = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        qg.qg_gemm_static_ws(Xd, p, Y=Y)
        torch.cuda.synchronize()
        assert np.array_equal(f16_bits(Y), f16_bits(Y_ref)), (bits, M, K, N)
        # every row against the FP64 oracle, to the GEMM tolerance
        op = to_oracle(p, orc)
        assert_close(Y.float().cpu().numpy(), orc.gemm(X.numpy(), op), f"static ws {bits} {M}x{K}x{N}")
    assert used


def test_static_ws_repeat_is_bit_identical(dev):
    """A second identical call after a different shape gives the same bits."""
    import workloads
    W, X = workloads.single_gemm(64, 8192, 2048, seed=7)
    p = qg.qg_pack(W.to(dev), 4)
    Xd = X.to(dev)
    a = qg.qg_gemm_static_ws(Xd, p).clone()
    W2, X2 = workloads.single_gemm(300, 2048, 6144, seed=8)
    qg.qg_gemm_static_ws(X2.to(dev), qg.qg_pack(W2.to(dev), 4))
    b = qg.qg_gemm_static_ws(Xd, p)
    torch.cuda.synchronize()
    assert np.array_equal(f16_bits(a), f16_bits(b))
