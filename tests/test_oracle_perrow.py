"""Pins of the oracle's per-row groups (group size G = K: one scale and one
zero per output channel).

The pages meet per-row quantisation in the INT4 -> INT2 re-packing of the loop
block ("β-Informed Deployment Features" page, CTX-TIER Phase 2b: a per-row
weight has group_size = K = 2048).  The reading: the same quantiser as for
groups of 128 (range with 0 included, s = fp16((hi - lo) / (2^b - 1)),
integer zero point, round-half-even), applied to the whole row.

Pins: a row worked by hand (INT2 and INT4) whose per-row and per-128 packs
differ; the exact-rational brute force of scale, zero and codes (including
all-positive, all-negative and all-zero rows) and of the GEMM; the error bound
|w^ - w| <= s/2; the pages' re-quantisation recipe on per-row weights; the
format check.
"""
import numpy as np
import pytest

from oracle import brute


def _hand_row(K=256):
    """One output channel: zero except w[0] = -1.5 and w[200] = 3."""
    W = np.zeros((K, 1), np.float32)
    W[0, 0] = -1.5
    W[200, 0] = 3.0
    return W


def test_hand_worked_row_int2(orc):
    # Whole row: lo = -1.5, hi = 3, s = 4.5 / 3 = 1.5 (FP16 0x3E00),
    # z = rne(1.5 / 1.5) = 1; q = rne(w / 1.5) + 1: -1.5 -> 0, 3 -> 3, 0 -> 1.
    p = orc.pack(_hand_row(), 2, group=256)
    assert p.scales.shape == (1, 1) and p.zeros.shape == (1, 1)
    assert int(p.scales[0, 0]) == 0x3E00 and int(p.zeros[0, 0]) == 0x3C00
    q = orc.unpack(p)[0]
    assert q[0] == 0 and q[200] == 3
    assert np.all(np.delete(q, [0, 200]) == 1)
    w = orc.dequant(p)[0]
    assert w[0] == -1.5 and w[200] == 3.0 and np.all(np.delete(w, [0, 200]) == 0.0)
    # Groups of 128 differ: group 0 has lo = -1.5, hi = 0 (s = 0.5, z = 3),
    # group 1 lo = 0, hi = 3 (s = 1, z = 0; stored as -0, the negation of lo).
    g = orc.pack(_hand_row(), 2)
    assert [int(v) for v in g.scales[0]] == [0x3800, 0x3C00]
    assert [orc.half_to_double(v) for v in g.zeros[0]] == [3.0, 0.0]


def test_hand_worked_row_int4(orc):
    # Whole row: s = fp16(4.5 / 15 = 0.3) = 1229 / 4096 (FP16 0x34CD: 0.3 =
    # 1.2 * 2^-2, fraction 0.2 * 1024 = 204.8 rounds to 205); z = rne(1.5 / s)
    # = rne(4.9992) = 5; -1.5 -> rne(-4.9992) + 5 = 0, 3 -> rne(9.9984) + 5 = 15,
    # 0 -> 5; 3 dequantises to 10 s = 3.00048828125.
    p = orc.pack(_hand_row(), 4, group=256)
    assert int(p.scales[0, 0]) == 0x34CD and int(p.zeros[0, 0]) == 0x4500
    q = orc.unpack(p)[0]
    assert q[0] == 0 and q[200] == 15 and np.all(np.delete(q, [0, 200]) == 5)
    w = orc.dequant(p)[0]
    assert w[0] == -5 * 1229 / 4096 and w[200] == 3.00048828125


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("seed", [0, 1])
def test_perrow_pack_matches_exact_rational_brute_force(orc, bits, seed):
    rng = np.random.default_rng(100 + seed)
    K, N = 384, 5
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    W[:, 1] = np.abs(W[:, 1])    # all positive
    W[:, 2] = -np.abs(W[:, 2])   # all negative
    W[:, 3] = 0.0                # all zero
    p = orc.pack(W, bits, group=K)
    S, Z, Q = brute.pack(W.tolist(), bits, group=K)
    assert p.scales.shape == (N, 1)
    for n in range(N):
        assert orc.half_to_double(p.scales[n, 0]) == float(S[n][0])
        assert orc.half_to_double(p.zeros[n, 0]) == float(Z[n][0])
        assert [int(w) for w in p.codes[n]] == brute.words(Q[n], bits)


@pytest.mark.parametrize("bits", [2, 4])
def test_perrow_gemm_matches_exact_rational_brute_force(orc, bits):
    rng = np.random.default_rng(7 + bits)
    M, K, N = 3, 256, 4
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    X = rng.standard_normal((M, K)).astype(np.float16)
    p = orc.pack(W, bits, group=K)
    S, Z, Q = brute.pack(W.tolist(), bits, group=K)
    exact = brute.gemm(X.tolist(), S, Z, Q, group=K)
    Y = orc.gemm(X, p)
    for m in range(M):
        for n in range(N):
            assert abs(Y[m, n] - float(exact[m][n])) <= 1e-12 * (1 + abs(float(exact[m][n])))


@pytest.mark.parametrize("bits", [2, 4])
def test_perrow_error_bound(orc, bits):
    rng = np.random.default_rng(3)
    K, N = 2048, 32
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    p = orc.pack(W, bits, group=K)
    s = orc.halves_to_double(p.scales)[:, 0]                    # [N]
    err = np.abs(orc.dequant(p) - W.T.astype(np.float64))      # [N][K]
    assert np.all(err <= s[:, None] / 2 * (1 + 1e-12))
    # a whole row's range is wider than a group's: per-row error is larger
    g = orc.pack(W, bits)
    assert np.mean(err ** 2) > np.mean((orc.dequant(g) - W.T) ** 2)


def test_perrow_requant_recipe(orc):
    """The pages' re-quantisation test (N = 64, K = 256, Gaussian weights) on
    per-row weights: error of INT4 -> INT2 against packing straight to INT2
    within 2x; the INT2 weight stays per-row."""
    rng = np.random.default_rng(11)
    K, N = 256, 64
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    p2 = orc.requant_4to2(orc.pack(W, 4, group=K))
    direct = orc.pack(W, 2, group=K)
    assert p2.group == K and p2.scales.shape == (N, 1)
    rms = lambda a: float(np.sqrt(np.mean(a ** 2)))
    ratio = rms(orc.dequant(p2).T - W) / rms(orc.dequant(direct).T - W)
    assert ratio <= 2.0, ratio


def test_perrow_format_check(orc):
    W = np.zeros((512, 4), np.float32)
    with pytest.raises(orc.OracleError):
        orc.pack(W, 4, group=256)        # neither 128 nor K
    with pytest.raises(orc.OracleError):
        orc.pack(np.zeros((200, 4), np.float32), 4, group=200)   # K not a multiple of 128
