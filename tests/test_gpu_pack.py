"""GPU parity of qg_pack, qg_unpack and qg_dequant against the oracle: bit-exact
codes, scales and zeros; bit-exact unpacked codes; FP32 dequant equal to the
oracle's exact value and FP16 dequant equal to its round-to-nearest-even."""
import numpy as np
import pytest
import torch

import workloads
from helpers import f16_bits, to_gpu

qg = pytest.importorskip("int2_quantized_gemm_amd")
pytestmark = pytest.mark.gpu


def _pack_both(orc, W: np.ndarray, bits: int):
    p = qg.qg_pack(torch.from_numpy(W).cuda(), bits)
    op = orc.pack(W, bits)
    return p, op


def _assert_pack_equal(p, op):
    assert np.array_equal(p.codes.cpu().numpy().view(np.uint32), op.codes)
    assert np.array_equal(f16_bits(p.scales), op.scales)
    assert np.array_equal(f16_bits(p.zeros), op.zeros)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("K,N", [(128, 1), (256, 37), (384, 300), (2048, 2048), (8192, 64)])
def test_pack_bit_exact(orc, bits, K, N):
    W, _ = workloads.single_gemm(1, K, N, seed=K + N)
    _assert_pack_equal(*_pack_both(orc, W.numpy(), bits))


@pytest.mark.parametrize("bits", [4, 2])
def test_pack_full_block_bit_exact(orc, bits):
    """The loop block's four weights at D=2048, F=8192 (the measured shapes)."""
    inp = workloads.block(1, seed=0)
    for name, W in inp.W.items():
        _assert_pack_equal(*_pack_both(orc, W.numpy(), bits))


@pytest.mark.parametrize("bits", [4, 2])
def test_pack_special_groups(orc, bits):
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((512, 40)) * 0.02).astype(np.float32)
    W[:128, 0] = 0.0                                   # all-zero group
    W[128:256, 1] = np.abs(W[128:256, 1])              # all positive
    W[256:384, 2] = -np.abs(W[256:384, 2])             # all negative
    W[5, :] = 0.0                                      # exact zeros
    W[:128, 3] = 1e-9                                  # scale rounds to 0 -> 1
    W[:128, 4] = 65504.0 * ((1 << bits) - 1)           # largest finite scale
    W[:, 5] = np.where(np.arange(512) % 2 == 0, 1.0, -1.0)  # alternating +-1
    W[:, 6] = np.ldexp(1.0, -20)                       # subnormal-range scale
    _assert_pack_equal(*_pack_both(orc, W, bits))


def test_pack_ldw_larger_than_n(orc):
    W, _ = workloads.single_gemm(1, 256, 72, seed=9)
    Wd = torch.zeros(256, 80, dtype=torch.float32)
    Wd[:, :72] = W
    p = qg.qg_pack(Wd.cuda()[:, :72], 4)
    _assert_pack_equal(p, orc.pack(W.numpy(), 4))


@pytest.mark.parametrize("bad", [np.nan, np.inf, 3e38])
def test_pack_rejects_non_finite_and_overflow(bad):
    W = np.zeros((128, 8), np.float32)
    W[7, 3] = bad
    with pytest.raises(qg.QGValueError):
        qg.qg_pack(torch.from_numpy(W).cuda(), 4)


def test_status_word_reports_each_call_alone(orc):
    """Pack and re-quantisation share one status word per device that is
    never cleared between calls: a failure must fail its own call only, and
    consecutive failures must each be reported."""
    good, _ = workloads.single_gemm(1, 256, 16, seed=5)
    bad = good.clone()
    bad[7, 3] = float("nan")
    for _ in range(2):
        with pytest.raises(qg.QGValueError):
            qg.qg_pack(bad.cuda(), 4)
        p = qg.qg_pack(good.cuda(), 4)
    _assert_pack_equal(p, orc.pack(good.numpy(), 4))
    broken = qg.qg_pack(good.cuda(), 4)
    broken.scales.view(torch.int16)[3, 1] = 0x7C00  # +inf
    with pytest.raises(qg.QGValueError):
        qg.qg_requant_4to2(broken)
    qg.qg_requant_4to2(p)
    with pytest.raises(qg.QGValueError):
        qg.qg_pack(bad.cuda(), 2)
    qg.qg_release_cache()  # the word is freed and allocated again
    _assert_pack_equal(qg.qg_pack(good.cuda(), 2), orc.pack(good.numpy(), 2))


def test_pack_and_requant_refused_under_capture(orc):
    """qg_pack and qg_requant_4to2 synchronise their stream, so on a stream
    under graph capture they are refused before anything is enqueued: the
    capture stays valid (a GEMM captured beside them replays to the eager
    result) and both calls work again once the capture has ended."""
    W, X = workloads.single_gemm(4, 256, 64, seed=6)
    Wd, Xd = W.cuda(), X.cuda()
    p = qg.qg_pack(Wd, 4)
    ref = f16_bits(qg.qg_gemm_int4(Xd, p))
    Y = torch.empty(4, 64, dtype=torch.float16, device="cuda")
    out4 = qg.PackedWeight.empty(256, 64, 4, Wd.device)
    out2 = qg.PackedWeight.empty(256, 64, 2, Wd.device)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        with pytest.raises(qg.QGValueError, match="captured"):
            qg.qg_pack(Wd, 4, out=out4)
        with pytest.raises(qg.QGValueError, match="captured"):
            qg.qg_requant_4to2(p, out=out2)
        qg.qg_gemm_int4(Xd, p, Y=Y)
    for r in range(2):
        Y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(f16_bits(Y), ref), f"replay {r}"
    op = orc.pack(W.numpy(), 4)
    _assert_pack_equal(qg.qg_pack(Wd, 4, out=out4), op)
    qg.qg_requant_4to2(p, out=out2)
    _assert_pack_equal(out2, orc.requant_4to2(op))


@pytest.mark.parametrize("bits", [4, 2])
def test_unpack_and_dequant_bit_exact(orc, bits):
    W, _ = workloads.single_gemm(1, 1024, 96, seed=bits)
    p, op = _pack_both(orc, W.numpy(), bits)
    assert np.array_equal(qg.qg_unpack(p).cpu().numpy(), orc.unpack(op))
    ref = orc.dequant(op)
    d32 = qg.qg_dequant(p, fp16=False).cpu().numpy().astype(np.float64)
    assert np.array_equal(d32, ref)
    d16 = f16_bits(qg.qg_dequant(p, fp16=True))
    assert np.array_equal(d16, orc.half_bits(ref))


def test_unpack_hand_built_words(orc):
    from conftest import golden
    for case in golden("bit_order.json")["cases"]:
        bits, per = case["bits"], 32 // case["bits"]
        codes = np.full((1, 128 // per), int(case["word"], 16), dtype=np.uint32)
        op = orc.Packed(bits, 128, 1, codes, np.full((1, 1), 0x3C00, np.uint16),
                        np.zeros((1, 1), np.uint16))
        q = qg.qg_unpack(to_gpu(op, qg)).cpu().numpy()[0]
        assert list(q[:per]) == case["codes"]


def _same_bits(a, b):
    """Bit-for-bit equality (NaN patterns included) of two tensors."""
    return torch.equal(a.view(torch.int16) if a.dtype == torch.float16 else a,
                       b.view(torch.int16) if b.dtype == torch.float16 else b)


def _canary_weight(K, N, bits, group=128):
    """A packed-weight buffer set whose every byte holds a canary pattern."""
    p = qg.PackedWeight.empty(K, N, bits, "cuda", group)
    p.codes.fill_(0x5A5A5A5A)
    p.scales.view(torch.int16).fill_(0x7BAD)
    p.zeros.view(torch.int16).fill_(0x7BAD)
    return p, [t.clone() for t in (p.codes, p.scales, p.zeros)]


@pytest.mark.parametrize("bits,group", [(4, 128), (2, 128), (4, 256)])
@pytest.mark.parametrize("bad", [np.nan, -np.inf, 3e38])
def test_rejected_pack_leaves_outputs_untouched(bits, group, bad):
    """A rejected qg_pack writes nothing: the validation pass runs first and
    the packing pass is never enqueued, so canary-filled codes, scales and
    zeros come back unchanged (also the groups of the call that were fine)."""
    W = np.random.default_rng(3).standard_normal((256, 40)).astype(np.float32) * 0.02
    W[200, 17] = bad
    p, before = _canary_weight(256, 40, bits, group)
    with pytest.raises(qg.QGValueError):
        qg.qg_pack(torch.from_numpy(W).cuda(), bits, group=group, out=p)
    torch.cuda.synchronize()
    for a, b in zip((p.codes, p.scales, p.zeros), before):
        assert _same_bits(a, b)


@pytest.mark.parametrize("in_place", [False, True])
def test_rejected_requant_leaves_outputs_untouched(in_place):
    """A rejected qg_requant_4to2 writes nothing: out of place the canary
    INT2 buffers, in place the INT4 weight itself, come back unchanged."""
    W, _ = workloads.single_gemm(1, 512, 48, seed=9)
    p4 = qg.qg_pack(W.cuda(), 4)
    p4.scales.view(torch.int16)[30, 2] = 0x7E00  # NaN
    torch.cuda.synchronize()
    if in_place:
        before = [t.clone() for t in (p4.codes, p4.scales, p4.zeros)]
        with pytest.raises(qg.QGValueError, match="non-finite"):
            qg.qg_requant_4to2(p4, in_place=True)
        torch.cuda.synchronize()
        for a, b in zip((p4.codes, p4.scales, p4.zeros), before):
            assert _same_bits(a, b)
    else:
        p2, before = _canary_weight(512, 48, 2)
        with pytest.raises(qg.QGValueError, match="non-finite"):
            qg.qg_requant_4to2(p4, out=p2)
        torch.cuda.synchronize()
        for a, b in zip((p2.codes, p2.scales, p2.zeros), before):
            assert _same_bits(a, b)
