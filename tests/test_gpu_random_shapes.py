"""GPU parity of qg_gemm_int4 / qg_gemm_int2 on seeded random shapes.

Eighty cases drawn once from two fixed seeds: M in 1..300 (every kernel family
and tile plan: GEMV, skinny with and without K parts, ring tiles of 32, 64
and 128 rows with and without a K split, the staged kernel), K a multiple of
128 up to 8192, N a multiple of 8 up to 3000, 4 or 2 bits, groups of 128 or
per row, activations with a leading dimension of K, K + 8 or K + 16.  Rows at both edges of every 32-row block are checked against the
oracle to the GEMM tolerance (rel-L2 <= 2e-3, max-abs <= 1e-2), with canary
bands around the output.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import Guarded, assert_close

qg = pytest.importorskip("int2_quantized_gemm_amd")
pytestmark = pytest.mark.gpu

GEMM = {4: qg.qg_gemm_int4, 2: qg.qg_gemm_int2}


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    pad_rng = np.random.default_rng(seed + 1)  # kept apart so the shapes of a seed never change
    out = []
    for _ in range(n):
        lo, hi = [(1, 2), (2, 17), (17, 129), (129, 301)][rng.choice(4, p=[0.2, 0.2, 0.3, 0.3])]
        M = int(rng.integers(lo, hi))
        # K: whole runs of 8 groups (the ring's DMA) 60 % of the time
        K = 1024 * int(rng.integers(1, 9)) if rng.random() < 0.6 else 128 * int(rng.integers(1, 65))
        N = 8 * int(rng.integers(1, 376))
        bits = int(rng.choice([4, 2]))
        per_row = bool(rng.random() < 0.3)
        out.append((M, K, N, bits, per_row, 8 * int(pad_rng.integers(0, 3))))
    return out


@pytest.mark.parametrize("M,K,N,bits,per_row,ldx_pad", _cases(40, 2024) + _cases(40, 4051))
def test_random_shape(orc, M, K, N, bits, per_row, ldx_pad):
    W, X = workloads.single_gemm(M, K, N, seed=M * 7 + K + N)
    group = K if per_row else 128
    p = qg.qg_pack(W.cuda(), bits, group=group)
    op = orc.pack(W.numpy(), bits, group=group)
    Xd = torch.zeros(M, K + ldx_pad, dtype=torch.float16, device="cuda")
    Xd[:, :K] = X.cuda()
    g = Guarded(M, N, N + 8)
    GEMM[bits](Xd[:, :K], p, Y=g.view)
    torch.cuda.synchronize()
    g.check()
    Y = g.view.float().cpu().numpy()
    assert_close(Y, orc.gemm(X.numpy(), op),
                 f"M={M} K={K} N={N} bits={bits} per_row={per_row} ldx={K + ldx_pad}")
