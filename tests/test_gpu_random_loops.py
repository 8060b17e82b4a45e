"""GPU parity of qg_loop_range on seeded random blocks.

Forty cases drawn once from a fixed seed: M in 1..300 (GEMV, skinny with and
without K parts, ring tiles with and without K splits), D in {256, ..., 2048}
(the fused and the separate LayerNorm routes), F = D, 2D or 4D, INT4 or INT2,
groups of 128 or per row, with or without the SwiGLU gate, and a range
[L0, L1) with L1 <= 3 (M halved until the FP64 oracle's work is at most
1.5e9 multiply-adds).  h is
checked in full against the oracle's loop driver (rel-L2 <= 2e-3, max-abs
<= 1e-2 * max(1, rms(h_ref))), and the same range run in two pieces from the
same start gives the same bits.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import assert_close

qg = pytest.importorskip("int2_quantized_gemm_amd")
pytestmark = pytest.mark.gpu

MAX_ORACLE_MACS = 1.5e9


def _cases(n=40, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = int(rng.choice([256, 512, 768, 1024, 1536, 2048]))
        F = D * int(rng.choice([1, 2, 4]))
        bits = int(rng.choice([4, 2]))
        gated = bool(rng.random() < 0.3)
        per_row = bool(rng.random() < 0.2)
        lo, hi = [(1, 2), (2, 17), (17, 129), (129, 301)][rng.choice(4, p=[0.25, 0.3, 0.25, 0.2])]
        M = int(rng.integers(lo, hi))
        L1 = int(rng.integers(1, 4))
        L0 = int(rng.integers(0, L1))
        macs = 4 * D * D + (3 if gated else 2) * D * F
        while M > 1 and M * (L1 - L0) * macs > MAX_ORACLE_MACS:
            M //= 2
        out.append((M, D, F, bits, gated, per_row, L0, L1))
    return out


@pytest.mark.parametrize("M,D,F,bits,gated,per_row,L0,L1", _cases())
def test_random_loop(orc, M, D, F, bits, gated, per_row, L0, L1):
    what = f"M={M} D={D} F={F} bits={bits} gated={gated} per_row={per_row} [{L0},{L1})"
    inp = workloads.block(M, seed=M + D + F + L1, D=D, F=F, gated=gated)
    blk = qg.pack_block(inp.W, bits, D, F, per_row=per_row)
    oblk = orc.pack_block({k: v.numpy() for k, v in inp.W.items()}, bits, D, F, per_row=per_row)
    scratch = qg.alloc_loop_scratch(blk, M)
    h = inp.X.float().cuda()
    qg.qg_loop_range(blk, h, L0, L1, scratch)
    href, _ = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), L0, L1)
    rms = float(np.sqrt(np.mean(href ** 2)))
    assert_close(h.cpu().numpy(), href, what, max_abs=1e-2 * max(1.0, rms))
    mid = (L0 + L1 + 1) // 2
    pieces = inp.X.float().cuda()
    qg.qg_loop_range(blk, pieces, L0, mid, scratch)
    qg.qg_loop_range(blk, pieces, mid, L1, scratch)
    assert torch.equal(pieces, h), what
