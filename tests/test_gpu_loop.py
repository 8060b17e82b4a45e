"""GPU parity of qg_loop_range against the oracle's loop driver.

Small blocks are checked in full; the measured D=2048/F=8192 workloads run at
their real M and L on the GPU and are checked on a sample of rows (the block
is row-independent, so the oracle runs just those rows).  The residual h must
meet rel-L2 <= 2e-3 and max-abs <= 1e-2*max(1, rms(h_ref)); the last
iteration's FP16 intermediates in the scratch meet the GEMM tolerance.
Invariants: an empty range leaves h untouched, [L0,L1) then [L1,L2) equals
[L0,L2) bit for bit, and repeated runs are bit-identical.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import assert_close

qg = pytest.importorskip("int2_quantized_gemm_amd")
pytestmark = pytest.mark.gpu


def _blocks(orc, M, bits, D, F, seed):
    inp = workloads.block(M, seed=seed, D=D, F=F)
    blk = qg.pack_block(inp.W, bits, D, F)
    oblk = orc.pack_block({k: v.numpy() for k, v in inp.W.items()}, bits, D, F)
    return inp, blk, oblk


def _check_h(h, href, what):
    rms = float(np.sqrt(np.mean(href ** 2)))
    assert_close(h, href, what, max_abs=1e-2 * max(1.0, rms))


def _check_scratch(views, last, rows, what):
    for k in ("norm", "qkv", "u", "y"):
        assert_close(views[k].float().cpu().numpy()[rows], last[k], f"{what} scratch {k}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M", [1, 3, 16, 33])
def test_loop_small_block_full(orc, bits, M):
    D, F, L = 256, 640, 3
    inp, blk, oblk = _blocks(orc, M, bits, D, F, seed=M)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    href, last = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    _check_h(h.cpu().numpy(), href, f"h bits={bits} M={M}")
    _check_scratch(qg.scratch_views(blk, M, scratch), last, slice(None), f"bits={bits} M={M}")


@pytest.mark.parametrize("M", [1, 16, 40])
def test_loop_empty_range_split_and_repeat(orc, M):
    D, F = 256, 512
    inp, blk, _ = _blocks(orc, M, 4, D, F, seed=11)
    h0 = inp.X.float().cuda()
    h = h0.clone()
    qg.qg_loop_range(blk, h, 5, 5)
    assert torch.equal(h, h0)
    full = h0.clone()
    qg.qg_loop_range(blk, full, 0, 4)
    split = h0.clone()
    qg.qg_loop_range(blk, split, 0, 1)
    qg.qg_loop_range(blk, split, 1, 3)
    qg.qg_loop_range(blk, split, 3, 4)
    assert torch.equal(full, split)
    again = h0.clone()
    qg.qg_loop_range(blk, again, 0, 4)
    assert torch.equal(full, again)
    assert not torch.equal(full, h0)


MEASURED = [
    # (name, bits, M, L, sampled rows)
    ("c2_int4_m1_l8", 4, 1, 8, [0]),
    ("c3_int4_m512_l8", 4, 512, 8, [0, 255, 511]),
    ("c4a_int2_m1_l16", 2, 1, 16, [0]),
    ("c4b_int2_m128_l8", 2, 128, 8, [0, 77, 127]),
    ("c5a_int4_m16_l32", 4, 16, 32, [0, 15]),
]


@pytest.mark.parametrize("name,bits,M,L,rows", MEASURED, ids=[m[0] for m in MEASURED])
def test_loop_measured_workloads_sampled_rows(orc, name, bits, M, L, rows):
    D, F = workloads.D_MODEL, workloads.D_FFN
    inp, blk, oblk = _blocks(orc, M, bits, D, F, seed=0)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    h = h.cpu().numpy()
    assert np.all(np.isfinite(h))
    href, last = orc.loop_range(oblk, inp.X.numpy()[rows].astype(np.float64), 0, L)
    _check_h(h[rows], href, name)
    _check_scratch(qg.scratch_views(blk, M, scratch), last, rows, name)
