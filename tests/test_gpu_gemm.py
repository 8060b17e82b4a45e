"""GPU parity of qg_gemm_int4 / qg_gemm_int2 against the FP64 oracle.

Both sides quantise the same seeded FP32 weights independently (their packs
are bit-identical, see test_gpu_pack.py) and multiply the same FP16
activations.  Tolerance: rel-L2 <= 2e-3 and max-abs <= 1e-2.  Hand-built
integer-exact, one-hot and cancellation cases must match bit for bit.  All
three kernel families (GEMV M == 1, skinny MFMA 2 <= M <= 16, tiled MFMA
M > 16) are covered at ragged shapes, with canary bands around the output.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import Guarded, assert_close, f16_bits, to_gpu

qg = pytest.importorskip("int2_quantized_gemm_amd")
pytestmark = pytest.mark.gpu

GEMM = {4: qg.qg_gemm_int4, 2: qg.qg_gemm_int2} if hasattr(qg, "qg_gemm_int4") else {}


def _run(bits, X: torch.Tensor, p, ld_pad: int = 0):
    M = X.shape[0]
    g = Guarded(M, p.N, p.N + ld_pad)
    GEMM[bits](X, p, Y=g.view)
    torch.cuda.synchronize()
    g.check()
    return g.view.float().cpu().numpy()


def _case(orc, bits, M, K, N, seed, ld_pad=0, ldx_pad=0):
    W, X = workloads.single_gemm(M, K, N, seed=seed)
    p = qg.qg_pack(W.cuda(), bits)
    op = orc.pack(W.numpy(), bits)
    Xd = torch.zeros(M, K + ldx_pad, dtype=torch.float16, device="cuda")
    Xd[:, :K] = X.cuda()
    Y = _run(bits, Xd[:, :K], p, ld_pad)
    ref = orc.gemm(X.numpy(), op)
    return Y, ref


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M", [1, 2, 3, 7, 16, 17, 31, 64, 129])
@pytest.mark.parametrize("K,N", [(128, 8), (384, 40), (2048, 200), (8192, 72)])
def test_gemm_ragged_shapes(orc, bits, M, K, N):
    Y, ref = _case(orc, bits, M, K, N, seed=M * 131 + K + N, ld_pad=8, ldx_pad=8)
    assert_close(Y, ref, f"bits={bits} M={M} K={K} N={N}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("K", [512, 1024, 2048, 4096, 8192, 16384])
def test_gemv_k_variants(orc, bits, K):
    """Every lane/chunk arrangement of the M == 1 kernel."""
    Y, ref = _case(orc, bits, 1, K, 264, seed=K + bits)
    assert_close(Y, ref, f"gemv bits={bits} K={K}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("K,N", [(4096, 4096), (4096, 1000), (8192, 1536), (8192, 1032),
                                 (16384, 2048), (16384, 520)])
def test_gemv_k_parts_row_sets(orc, bits, K, N):
    """M == 1 with rows of several chunks per lane: K split over the
    workgroup's waves, every row-set size the launch picks (8, 4, 2 or 1 rows,
    from how many workgroups N gives), N ragged against the set size."""
    Y, ref = _case(orc, bits, 1, K, N, seed=K + N + bits)
    assert_close(Y, ref, f"gemv bits={bits} K={K} N={N}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,K,N", [(1, 2048, 2048), (1, 2048, 6144), (1, 2048, 8192),
                                   (1, 8192, 2048), (16, 2048, 6144), (16, 8192, 2048),
                                   (128, 2048, 8192), (512, 2048, 2048)])
def test_gemm_block_shapes(orc, bits, M, K, N):
    """The measured shapes (loop-block projections at the measured M)."""
    Y, ref = _case(orc, bits, M, K, N, seed=7)
    assert_close(Y, ref, f"bits={bits} M={M} K={K} N={N}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M", [1, 3, 33])
def test_gemm_maximum_k(orc, bits, M):
    """K at the ABI's limit (2^22): no GEMV lane arrangement covers it, so even
    M = 1 runs the tiled kernel with its K split; N ragged (24).  The outputs
    (std ~ 0.02 sqrt(K) ~ 41) are far above the configs' |Y| < 10, where one
    FP16 step of the required output rounding exceeds 1e-2: max-abs is
    therefore two FP16 steps at the largest reference value (rel-L2 stays
    2e-3)."""
    K, N = 1 << 22, 24
    Y, ref = _case(orc, bits, M, K, N, seed=M + bits)
    top = float(np.max(np.abs(ref)))
    ulp = 2.0 ** (np.floor(np.log2(max(top, 2.0 ** -14))) - 10)
    assert_close(Y, ref, f"max K bits={bits} M={M}", max_abs=max(1e-2, 2 * ulp))


def test_gemm_c1_seed0(orc):
    """Single INT4 GEMM, M=1, K=N=2048, seed 0 -- the single-pass workload."""
    Y, ref = _case(orc, 4, 1, 2048, 2048, seed=0)
    assert_close(Y, ref, "c1")


def test_gemm_long_prefill_down_proj_all_rows(orc):
    """M=2048 through the FFN down projection (K=8192 -> N=2048), in the
    launch configuration the bench times (128-row ring tiles: this shape has
    256 of them), every row against the oracle."""
    W, X = workloads.single_gemm(2048, 8192, 2048, seed=0)
    p = qg.qg_pack(W.cuda(), 4)
    op = orc.pack(W.numpy(), 4)
    Y = qg.qg_gemm_int4(X.cuda(), p).float().cpu().numpy()
    assert np.all(np.isfinite(Y))
    assert_close(Y, orc.gemm(X.numpy(), op), "m2048 down")


# Shapes whose tile plan runs the LDS-DMA ring kernel with 64- and 128-row
# tiles (ragged M and N edges): 64-row tiles without and with a K split (K =
# 8192 in 4 parts of 16 groups) and with scales and zeros in registers (K of
# 5 groups); 128-row tiles (K = 8192 with >= 256 tiles); and K of 10 groups,
# which no ring tile takes, on the staged kernel.  Every row is checked.
RING_CASES = [(300, 2048, 8200), (520, 8192, 1000), (1024, 2048, 6144), (1100, 8192, 4000),
              (300, 640, 8200), (300, 1280, 8200)]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,K,N", [(2, 6144, 40), (16, 8192, 2048), (5, 2304, 104),
                                   (16, 2048, 8192), (11, 4096, 200)])
def test_gemm_skinny_k_parts(orc, bits, M, K, N):
    """2 <= M <= 16 with K above the staging size: K split into parts and
    summed by the reduction kernel (uneven parts for K = 2304 and 6144)."""
    Y, ref = _case(orc, bits, M, K, N, seed=M + K + N, ld_pad=8, ldx_pad=8)
    assert_close(Y, ref, f"skinny parts bits={bits} M={M} K={K} N={N}")


# Shapes on which the skinny kernel takes two 16-channel tiles per workgroup
# (launches of at least 192 workgroups): ragged N leaves the last workgroup's
# second tile partly (N = 6168) or wholly (N = 6152, 2056, 1544) past N; with
# and without K parts.
SKINNY_PAIR_CASES = [(16, 2048, 6152), (3, 2048, 6168), (7, 6144, 2056), (16, 8192, 1544),
                     (2, 2048, 8192)]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,K,N", SKINNY_PAIR_CASES)
def test_gemm_skinny_column_pairs(orc, bits, M, K, N):
    Y, ref = _case(orc, bits, M, K, N, seed=M * 3 + K + N, ld_pad=8, ldx_pad=8)
    assert_close(Y, ref, f"skinny pairs bits={bits} M={M} K={K} N={N}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,K,N", RING_CASES)
def test_gemm_ring_path_all_rows(orc, bits, M, K, N):
    W, X = workloads.single_gemm(M, K, N, seed=M + K + N + bits)
    p = qg.qg_pack(W.cuda(), bits)
    op = orc.pack(W.numpy(), bits)
    g = Guarded(M, N, (N + 15) // 8 * 8)
    GEMM[bits](X.cuda(), p, Y=g.view)
    torch.cuda.synchronize()
    g.check()
    Y = g.view.float().cpu().numpy()
    assert_close(Y, orc.gemm(X.numpy(), op), f"ring bits={bits} M={M} K={K} N={N}")


# Shapes whose tile plan runs the ring kernel with 32-row tiles: M <= 128
# (batched decode) and larger M with too few 64-row tiles.  Scales and zeros
# come by DMA for parts of whole runs of 8 groups, from registers for K of 3,
# 5 and 7 groups; K split into 2 and 8 parts.  (200, 8192, 1500) and
# (2048, 2048, 8192) take 64-row tiles (K split in 4; 2048 tiles).
RING32_CASES = [(40, 1024, 1000), (17, 640, 300), (100, 384, 520), (33, 2048, 6144),
                (64, 8192, 2048), (200, 8192, 1500), (384, 2048, 2048), (700, 896, 700),
                (2048, 2048, 8192)]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,K,N", RING32_CASES)
def test_gemm_ring32_paths(orc, bits, M, K, N):
    W, X = workloads.single_gemm(M, K, N, seed=M + K + N + bits)
    p = qg.qg_pack(W.cuda(), bits)
    op = orc.pack(W.numpy(), bits)
    g = Guarded(M, N, (N + 15) // 8 * 8)
    GEMM[bits](X.cuda(), p, Y=g.view)
    torch.cuda.synchronize()
    g.check()
    Y = g.view.float().cpu().numpy()
    assert_close(Y, orc.gemm(X.numpy(), op), f"ring32 bits={bits} M={M} K={K} N={N}")


@pytest.mark.parametrize("offset", [0, 1])
def test_gemm_ring_shape_with_offset_scales(orc, offset):
    """Scales and zeros as views starting `offset` halves into a larger
    buffer: 16-byte aligned (offset 0) keeps the ring kernel, 2-byte aligned
    (offset 1, which the format allows) must fall back to the staged kernel;
    both match the oracle."""
    M, K, N = 300, 2048, 8200
    W, X = workloads.single_gemm(M, K, N, seed=offset)
    p = qg.qg_pack(W.cuda(), 4)
    op = orc.pack(W.numpy(), 4)
    views = []
    for t in (p.scales, p.zeros):
        buf = torch.zeros(t.numel() + 8, dtype=torch.float16, device="cuda")
        buf[offset:offset + t.numel()] = t.reshape(-1)
        views.append(buf[offset:offset + t.numel()].view(t.shape))
    shifted = qg.PackedWeight(4, K, N, p.codes, views[0], views[1])
    Y = qg.qg_gemm_int4(X.cuda(), shifted).float().cpu().numpy()
    rows = [0, 127, 128, 255, 256, 299]
    assert_close(Y[rows], orc.gemm(X.numpy()[rows], op), f"offset={offset}")


def _packed_from_codes(orc, bits, q, s, z):
    q = np.asarray(q, np.int64)
    N, K = q.shape
    per = 32 // bits
    words = np.zeros((N, K // per), np.uint64)
    for j in range(per):
        words |= q[:, j::per].astype(np.uint64) << np.uint64(16 * (j % 2) + bits * (j // 2))
    return orc.Packed(bits, K, N, words.astype(np.uint32),
                      orc.half_bits(np.asarray(s, np.float64).reshape(N, K // 128)),
                      orc.half_bits(np.asarray(z, np.float64).reshape(N, K // 128)))


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M", [1, 5, 16, 40])
def test_gemm_integer_exact(orc, bits, M):
    rng = np.random.default_rng(100 + M)
    K, N = 2048, 48
    q = rng.integers(0, 1 << bits, size=(N, K))
    z = rng.integers(0, 1 << bits, size=(N, K // 128))
    op = _packed_from_codes(orc, bits, q, np.full(N * K // 128, 2.0 ** -4), z)
    X = np.zeros((M, K), np.float16)
    for m in range(M):
        idx = rng.choice(K, 8, replace=False)
        X[m, idx] = rng.choice([-1, 1], 8)
    ref = orc.gemm(X, op)
    Y = GEMM[bits](torch.from_numpy(X).cuda(), to_gpu(op, qg))
    assert np.array_equal(f16_bits(Y), orc.half_bits(ref))


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M", [1, 16, 64])
def test_gemm_one_hot_rows(orc, bits, M):
    W, _ = workloads.single_gemm(1, 2048, 136, seed=5)
    p = qg.qg_pack(W.cuda(), bits)
    op = orc.pack(W.numpy(), bits)
    ks = (np.arange(M) * 97) % 2048
    X = np.zeros((M, 2048), np.float16)
    X[np.arange(M), ks] = 1.0
    Y = f16_bits(GEMM[bits](torch.from_numpy(X).cuda(), p))
    dq = orc.dequant(op)                       # [N][K]
    assert np.array_equal(Y, orc.half_bits(dq[:, ks].T))


@pytest.mark.parametrize("M", [1, 16, 32])
def test_gemm_cancellation(orc, M):
    """Partial sums reach 4096*7.5 code units while the exact result is -0.5:
    an FP16 accumulator would lose it, FP32 accumulation keeps it exact."""
    K, N = 8192, 16
    half = K // 2
    q = np.full((N, K), 15, np.int64)
    q[:, half - 1] = 14
    op = _packed_from_codes(orc, 4, q, np.full(N * K // 128, 0.5), np.zeros(N * K // 128))
    X = np.ones((M, K), np.float16)
    X[:, half:] = -1
    Y = qg.qg_gemm_int4(torch.from_numpy(X).cuda(), to_gpu(op, qg)).float().cpu().numpy()
    assert np.all(Y == -0.5)
    assert np.all(orc.gemm(X[:1], op) == -0.5)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M", [1, 16, 512])
def test_gemm_deterministic(bits, M):
    W, X = workloads.single_gemm(M, 2048, 2048, seed=3)
    p = qg.qg_pack(W.cuda(), bits)
    Xd = X.cuda()
    Ys = [f16_bits(GEMM[bits](Xd, p)) for _ in range(3)]
    assert np.array_equal(Ys[0], Ys[1]) and np.array_equal(Ys[0], Ys[2])


def test_gemm_m0_is_noop():
    W, _ = workloads.single_gemm(1, 256, 64, seed=1)
    p = qg.qg_pack(W.cuda(), 4)
    Y = qg.qg_gemm_int4(torch.zeros(0, 256, dtype=torch.float16, device="cuda"), p)
    assert Y.shape == (0, 64)


def test_gemm_rejects_mismatched_bits():
    W, X = workloads.single_gemm(1, 256, 64, seed=1)
    p = qg.qg_pack(W.cuda(), 4)
    with pytest.raises(qg.QGValueError):
        qg.qg_gemm_int2(X.cuda(), p)


@pytest.mark.parametrize("M", [1, 16, 64])
def test_gemm_captured_in_graph_replays(M):
    """GEMM launches recorded in a caller's graph (as the bench does) replay to
    the eager result every time, with eager work between replays."""
    W, X = workloads.single_gemm(M, 2048, 512, seed=4)
    p = qg.qg_pack(W.cuda(), 4)
    Xd = X.cuda()
    ref = f16_bits(qg.qg_gemm_int4(Xd, p))
    Y = torch.empty(M, 512, dtype=torch.float16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.qg_gemm_int4(Xd, p, Y=Y)
    for r in range(3):
        Y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(f16_bits(Y), ref), f"replay {r}"
        qg.qg_gemm_int4(Xd[:1], p)
        torch.cuda.synchronize()


def _strided(p, pad_words):
    """The same weight with its code rows pad_words (a multiple of 4) apart
    past K*bits/32, the padding filled with a pattern no row should read."""
    words = p.K * p.bits // 32
    buf = torch.full((p.N, words + pad_words), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    buf[:, :words] = p.codes
    return qg.PackedWeight(p.bits, p.K, p.N, buf, p.scales, p.zeros, p.group)


# Every kernel route with code rows at a larger stride (ldc): the GEMV, the
# skinny kernel (with K parts), the 32-, 64- and 128-row ring tiles (with a K
# split), the staged kernel (K of 10 groups) -- bit for bit against the same
# weight with compact rows.
STRIDED = [(1, 2048, 304), (1, 8192, 64), (9, 6144, 40), (40, 2048, 520), (300, 2048, 2104),
           (2048, 8192, 2048), (200, 1280, 296), (64, 8192, 256)]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,K,N", STRIDED)
def test_gemm_code_row_stride(orc, bits, M, K, N):
    W, X = workloads.single_gemm(M, K, N, seed=M + K + N + 5)
    p = qg.qg_pack(W.cuda(), bits)
    Xd = X.cuda()
    ref = f16_bits(GEMM[bits](Xd, p))
    for pad in (4, K * bits // 32):  # one extra 16-byte chunk; INT4-stride INT2 rows
        got = f16_bits(GEMM[bits](Xd, _strided(p, pad)))
        assert np.array_equal(got, ref), f"bits={bits} M={M} K={K} N={N} pad={pad}"


@pytest.mark.parametrize("bits", [4, 2])
def test_unpack_and_dequant_code_row_stride(bits):
    W, _ = workloads.single_gemm(1, 512, 33, seed=77)
    p = qg.qg_pack(W.cuda(), bits)
    s = _strided(p, 8)
    assert torch.equal(qg.qg_unpack(s), qg.qg_unpack(p))
    assert torch.equal(qg.qg_dequant(s), qg.qg_dequant(p))
    assert torch.equal(qg.qg_dequant(s, fp16=True).view(torch.int16),
                       qg.qg_dequant(p, fp16=True).view(torch.int16))
