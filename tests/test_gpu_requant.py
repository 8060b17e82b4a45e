"""GPU parity of qg_requant_4to2 (INT4 -> INT2 re-quantisation) against the
oracle's requant_4to2.  Codes, scales and zeros must match bit for bit, out
of place and in place -- the pages' form (INT2 rows kept at the INT4 row
stride, each over the front half of its own INT4 row, whose back half must be
left untouched; one launch up to K = 32768, launches ordered by group index
beyond) and compact INT2 rows over the front of the INT4 buffer (whose tail
must be left untouched) -- over ragged N and K up to 65536.  The re-quantised
weight then feeds the INT2 GEMM and the loop block, checked against the
oracle on the oracle's own re-quantised weight.  The pages' unit-test recipe
(N=64, K=256, error ratio against direct INT2 within 2x) is repeated on the
GPU result."""
import numpy as np
import pytest
import torch

import workloads
from helpers import assert_close, compact_codes

qg = pytest.importorskip("int2_quantized_gemm_amd")
pytestmark = pytest.mark.gpu


def _np(p):
    return (compact_codes(p), p.scales.cpu().numpy().view(np.uint16),
            p.zeros.cpu().numpy().view(np.uint16))


def _assert_same(p, op, what):
    c, s, z = _np(p)
    assert np.array_equal(c, op.codes), f"{what}: codes"
    assert np.array_equal(s, op.scales), f"{what}: scales"
    assert np.array_equal(z, op.zeros), f"{what}: zeros"


SHAPES = [(128, 1), (256, 64), (384, 3), (2048, 300), (8192, 72), (2048, 2), (1024, 5),
          (16384, 9), (32768, 3)]


# in_place: False (out of place), "stride" (the pages' form: INT2 rows kept
# at the INT4 row stride, each over the front half of its own INT4 row) or
# "compact" (INT2 rows packed over the front of the INT4 buffer).
MODES = [False, "stride", "compact"]


def _requant(p4, mode):
    if not mode:
        return qg.qg_requant_4to2(p4)
    return qg.qg_requant_4to2(p4, in_place=True, compact=mode == "compact")


@pytest.mark.parametrize("K,N", SHAPES)
@pytest.mark.parametrize("mode", MODES)
def test_requant_bit_exact(orc, K, N, mode):
    W, _ = workloads.single_gemm(1, K, N, seed=K + N)
    p4 = qg.qg_pack(W.cuda(), 4)
    op4 = orc.pack(W.numpy(), 4)
    ref = orc.requant_4to2(op4)
    before = p4.codes.clone()
    p2 = _requant(p4, mode)
    _assert_same(p2, ref, f"K={K} N={N} mode={mode}")
    if mode:
        assert p2.codes.data_ptr() == p4.codes.data_ptr()
    if mode == "compact":
        tail = before.view(-1)[N * K // 16:]
        assert torch.equal(p4.codes.view(-1)[N * K // 16:], tail), "INT4 tail was touched"
    elif mode == "stride":
        assert p2.codes.stride(0) == K // 8
        assert torch.equal(p4.codes[:, K // 16:], before[:, K // 16:]), \
            "the back half of an INT4 row was touched"


@pytest.mark.parametrize("mode", ["stride", "compact"])
def test_requant_block_shapes_in_place(orc, mode):
    inp = workloads.block(1, seed=3)
    for name, (K, N) in workloads.block_shapes(inp.D, inp.F).items():
        p4 = qg.qg_pack(inp.W[name].cuda(), 4)
        ref = orc.requant_4to2(orc.pack(inp.W[name].numpy(), 4))
        _assert_same(_requant(p4, mode), ref, f"{name} {mode}")


@pytest.mark.parametrize("K", [40960, 65536])
def test_requant_in_place_long_rows(orc, K):
    """Rows longer than one workgroup holds (K > 32768): in place at the INT4
    stride the groups of every row go in launches ordered by group index."""
    N = 6
    W, _ = workloads.single_gemm(1, K, N, seed=K)
    p4 = qg.qg_pack(W.cuda(), 4)
    ref = orc.requant_4to2(orc.pack(W.numpy(), 4))
    _assert_same(_requant(p4, "stride"), ref, f"long rows K={K}")


def test_requant_page_recipe_on_gpu(orc):
    K, N = 256, 64
    W = (torch.randn(K, N, generator=workloads.generator(11)) * 0.02).float()
    p2 = qg.qg_requant_4to2(qg.qg_pack(W.cuda(), 4))
    deq = qg.qg_dequant(p2)
    torch.cuda.synchronize()
    err = float(torch.sqrt(torch.mean((deq.cpu().T - W) ** 2)))
    direct = orc.dequant(orc.pack(W.numpy(), 2)).T
    err_direct = float(np.sqrt(np.mean((direct - W.numpy()) ** 2)))
    assert err / err_direct <= 2.0


@pytest.mark.parametrize("M", [1, 16, 300])
def test_int2_gemm_after_requant(orc, M):
    K, N = 2048, 8200 if M == 300 else 520
    W, X = workloads.single_gemm(M, K, N, seed=M)
    p2 = qg.qg_requant_4to2(qg.qg_pack(W.cuda(), 4), in_place=True)  # INT4 row stride
    assert p2.codes.stride(0) == K // 8
    ref_w = orc.requant_4to2(orc.pack(W.numpy(), 4))
    Y = qg.qg_gemm_int2(X.cuda(), p2).float().cpu().numpy()
    assert_close(Y, orc.gemm(X.numpy(), ref_w), f"int2 gemm after requant M={M}")


@pytest.mark.parametrize("M", [1, 3, 40])
@pytest.mark.parametrize("mode", MODES)
def test_loop_after_requant_block(orc, M, mode):
    """Tier switch of a whole block, then iterations through the INT2 path
    (GEMV, skinny and ring kernels reading each in-place form)."""
    D, F, L = 1024, 2048, 2
    inp = workloads.block(M, seed=5, D=D, F=F)
    blk2 = qg.requant_block(qg.pack_block(inp.W, 4, D, F), in_place=bool(mode),
                            compact=mode == "compact")
    assert all(getattr(blk2, k).bits == 2 for k in ("qkv", "out", "up", "down"))
    o4 = orc.pack_block({k: v.numpy() for k, v in inp.W.items()}, 4, D, F)
    o2 = orc.Block(D, F, *(orc.requant_4to2(getattr(o4, k)) for k in ("qkv", "out", "up", "down")))
    h = inp.X.float().cuda()
    qg.qg_loop_range(blk2, h, 0, L)
    href, _ = orc.loop_range(o2, inp.X.numpy().astype(np.float64), 0, L)
    h = h.cpu().numpy()
    rms = float(np.sqrt(np.mean(href ** 2)))
    assert_close(h, href, "loop after requant", max_abs=1e-2 * max(1.0, rms))


def test_requant_reports_non_finite_scale():
    W, _ = workloads.single_gemm(1, 256, 16, seed=2)
    p4 = qg.qg_pack(W.cuda(), 4)
    p4.scales.view(torch.int16)[3, 1] = 0x7C00  # +inf
    with pytest.raises(qg.QGValueError, match="non-finite"):
        qg.qg_requant_4to2(p4)
