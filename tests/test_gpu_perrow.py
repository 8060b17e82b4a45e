"""GPU parity of per-row groups (group size K: one scale and zero per output
channel) against the oracle.

Pack, unpack and dequant bit-exact; the GEMM through every kernel route a
per-row weight can take (M = 1 GEMV, the 2..16-row skinny kernel with and
without K parts, the ring kernel with 32- and 128-row tiles and with a K
split, the staged kernel where the tile plan keeps the shape off the ring) at
ragged shapes, to the GEMM tolerance; INT4 -> INT2
re-quantisation bit-exact out of place and in place; the loop block with
per-row weights, plain and gated.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import Guarded, assert_close, compact_codes, f16_bits

qg = pytest.importorskip("int2_quantized_gemm_amd")
pytestmark = pytest.mark.gpu

GEMM = {4: qg.qg_gemm_int4, 2: qg.qg_gemm_int2}


def _same(p, op, what):
    assert p.group == op.group == p.K, what
    assert np.array_equal(compact_codes(p), op.codes), f"{what}: codes"
    assert np.array_equal(f16_bits(p.scales), op.scales), f"{what}: scales"
    assert np.array_equal(f16_bits(p.zeros), op.zeros), f"{what}: zeros"


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("K,N", [(128, 3), (384, 300), (2048, 2048), (8192, 40)])
def test_perrow_pack_bit_exact(orc, bits, K, N):
    W, _ = workloads.single_gemm(1, K, N, seed=K + N + bits)
    p = qg.qg_pack(W.cuda(), bits, group=K)
    _same(p, orc.pack(W.numpy(), bits, group=K), f"bits={bits} K={K} N={N}")


@pytest.mark.parametrize("bits", [4, 2])
def test_perrow_unpack_and_dequant_bit_exact(orc, bits):
    W, _ = workloads.single_gemm(1, 1024, 96, seed=bits)
    p = qg.qg_pack(W.cuda(), bits, group=1024)
    op = orc.pack(W.numpy(), bits, group=1024)
    assert np.array_equal(qg.qg_unpack(p).cpu().numpy(), orc.unpack(op))
    ref = orc.dequant(op)
    assert np.array_equal(qg.qg_dequant(p, fp16=False).cpu().numpy().astype(np.float64), ref)
    assert np.array_equal(f16_bits(qg.qg_dequant(p, fp16=True)), orc.half_bits(ref))


# (M, K, N): GEMV; skinny in one part and in K parts; ring 32-row tiles (one
# part, and K = 8192 split in 8); ring 64-row tiles (K of 16 and 7 groups);
# ring 128-row tiles (K = 8192, >= 256 tiles); the staged kernel (K of 10
# groups, which the tile plan keeps off the ring).
PERROW_GEMM = [(1, 2048, 1000), (1, 512, 300), (5, 2048, 200), (16, 8192, 520),
               (40, 1024, 1000), (64, 8192, 2048), (300, 2048, 8200), (300, 896, 8200),
               (1100, 8192, 4000), (300, 1280, 8200)]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,K,N", PERROW_GEMM)
def test_perrow_gemm_paths(orc, bits, M, K, N):
    W, X = workloads.single_gemm(M, K, N, seed=M + K + N + bits)
    p = qg.qg_pack(W.cuda(), bits, group=K)
    op = orc.pack(W.numpy(), bits, group=K)
    g = Guarded(M, N, (N + 15) // 8 * 8)
    GEMM[bits](X.cuda(), p, Y=g.view)
    torch.cuda.synchronize()
    g.check()
    Y = g.view.float().cpu().numpy()
    assert_close(Y, orc.gemm(X.numpy(), op),
                 f"per-row bits={bits} M={M} K={K} N={N}")


@pytest.mark.parametrize("K,N", [(128, 1), (384, 3), (2048, 300), (8192, 72), (2048, 2)])
@pytest.mark.parametrize("mode", [False, "stride", "compact"])
def test_perrow_requant_bit_exact(orc, K, N, mode):
    W, _ = workloads.single_gemm(1, K, N, seed=K + N + 1)
    p4 = qg.qg_pack(W.cuda(), 4, group=K)
    ref = orc.requant_4to2(orc.pack(W.numpy(), 4, group=K))
    before = p4.codes.clone()
    p2 = (qg.qg_requant_4to2(p4) if not mode else
          qg.qg_requant_4to2(p4, in_place=True, compact=mode == "compact"))
    _same(p2, ref, f"K={K} N={N} mode={mode}")
    if mode:
        assert p2.codes.data_ptr() == p4.codes.data_ptr()
    if mode == "compact":
        assert torch.equal(p4.codes.view(-1)[N * K // 16:], before.view(-1)[N * K // 16:]), \
            "INT4 tail was touched"
    elif mode == "stride":
        assert torch.equal(p4.codes[:, K // 16:], before[:, K // 16:]), "back half touched"


def test_perrow_requant_rejects_mixed_groups():
    W, _ = workloads.single_gemm(1, 1024, 8, seed=0)
    p4 = qg.qg_pack(W.cuda(), 4, group=1024)
    out = qg.PackedWeight.empty(1024, 8, 2, "cuda")        # groups of 128
    with pytest.raises(qg.QGError, match="group"):
        qg.qg_requant_4to2(p4, out=out)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,gated", [(1, False), (1, True), (33, False), (33, True)])
def test_perrow_loop_block(orc, bits, M, gated):
    D, F, L = 1024, 2048, 2
    inp = workloads.block(M, seed=M + bits, D=D, F=F, gated=gated)
    blk = qg.pack_block(inp.W, bits, D, F, per_row=True)
    oblk = orc.pack_block({k: v.numpy() for k, v in inp.W.items()}, bits, D, F, per_row=True)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    href, _ = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    rms = float(np.sqrt(np.mean(href ** 2)))
    assert_close(h.cpu().numpy(), href, f"per-row loop bits={bits} M={M} gated={gated}",
                 max_abs=1e-2 * max(1.0, rms))


def test_perrow_measured_block_m1_l8(orc):
    """The measured per-row workload at its real size: the D=2048, F=8192
    INT4 block with one scale and zero per channel, M=1, L=8 (the bench's
    launch configuration: fused-LayerNorm GEMVs through the cached graph)."""
    D, F, L, M = workloads.D_MODEL, workloads.D_FFN, 8, 1
    inp = workloads.block(M, seed=0, D=D, F=F)
    blk = qg.pack_block(inp.W, 4, D, F, per_row=True)
    oblk = orc.pack_block({k: v.numpy() for k, v in inp.W.items()}, 4, D, F, per_row=True)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    href, _ = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    rms = float(np.sqrt(np.mean(href ** 2)))
    assert_close(h.cpu().numpy(), href, "per-row measured block", max_abs=1e-2 * max(1.0, rms))
