"""Pins for the oracle's unpack, dequant and GEMM.

Pinned against hand-built words (bit order), a hand-worked GEMM, an
exact-rational brute force, one-hot rows, integer-exact cases, a cancellation
case whose partial sums are large but whose result is small, and the all-ones
closed form.
"""
import numpy as np
import pytest

from conftest import golden
from oracle import brute


def _packed(orc, bits, codes_nk, scales, zeros):
    """Build a Packed from explicit codes [N][K] and per-group s/z values."""
    codes_nk = np.asarray(codes_nk, dtype=np.int64)
    N, K = codes_nk.shape
    per = 32 // bits
    words = np.zeros((N, K // per), dtype=np.uint64)
    for j in range(per):
        words |= (codes_nk[:, j::per].astype(np.uint64) << np.uint64(16 * (j % 2) + bits * (j // 2)))
    s = np.asarray(scales, dtype=np.float64).reshape(N, K // 128)
    z = np.asarray(zeros, dtype=np.float64).reshape(N, K // 128)
    return orc.Packed(bits, K, N, words.astype(np.uint32), orc.half_bits(s), orc.half_bits(z))


def test_unpack_bit_order_hand_built(orc):
    for case in golden("bit_order.json")["cases"]:
        bits = case["bits"]
        per = 32 // bits
        word = int(case["word"], 16)
        codes = np.full((1, 128 // per), word, dtype=np.uint32)
        p = orc.Packed(bits, 128, 1, codes, np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16))
        q = orc.unpack(p)[0]
        assert list(q[:per]) == case["codes"]


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_unpack_round_trip_of_codes(orc, bits):
    rng = np.random.default_rng(5)
    q = rng.integers(0, 1 << bits, size=(6, 256))
    p = _packed(orc, bits, q, np.full(12, 0.5), np.zeros(12))
    assert np.array_equal(orc.unpack(p), q.astype(np.uint8))
    # same words as the exact brute-force packer
    for n in range(6):
        assert [int(w) for w in p.codes[n]] == brute.words(list(q[n]), bits)


def test_gemm_hand_worked_closed_form(orc):
    gd = golden("gemm_closed_form.json")
    k = np.arange(128)
    codes = np.stack([k % 16, np.where(k < 64, 15, 0)])
    p = _packed(orc, 4, codes, [gd["col0"]["scale"], gd["col1"]["scale"]],
                [gd["col0"]["zero"], gd["col1"]["zero"]])
    Y = orc.gemm(np.ones((1, 128), np.float16), p)
    assert list(Y[0]) == gd["Y"]


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("K", [128, 256])
def test_gemm_matches_exact_rational_brute_force(orc, bits, K):
    rng = np.random.default_rng(K + bits)
    M, N = 3, 5
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    X = rng.standard_normal((M, K)).astype(np.float16)
    p = orc.pack(W, bits)
    Y = orc.gemm(X, p)
    S, Z, Q = brute.pack(W.tolist(), bits)
    Yx = brute.gemm(X.tolist(), S, Z, Q)
    for m in range(M):
        for n in range(N):
            ex = float(Yx[m][n])
            assert abs(Y[m, n] - ex) <= 1e-12 * max(1.0, abs(ex))


@pytest.mark.parametrize("bits", [2, 4])
def test_gemm_one_hot_rows_give_dequantised_rows(orc, bits):
    rng = np.random.default_rng(9)
    K, N = 384, 24
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    p = orc.pack(W, bits)
    ks = [0, 1, 127, 128, 200, 383]
    X = np.zeros((len(ks), K), np.float16)
    for m, k in enumerate(ks):
        X[m, k] = 1.0
    Y = orc.gemm(X, p)
    dq = orc.dequant(p)
    for m, k in enumerate(ks):
        assert np.array_equal(Y[m], dq[:, k])


@pytest.mark.parametrize("bits", [2, 4])
def test_gemm_integer_exact(orc, bits):
    """s = 2^-4, X in {-1, 0, 1} with at most 8 nonzeros: Y is an exact
    multiple of 2^-4 computed by integer arithmetic."""
    rng = np.random.default_rng(13)
    K, N, M = 512, 16, 4
    q = rng.integers(0, 1 << bits, size=(N, K))
    z = rng.integers(0, 1 << bits, size=(N, K // 128))
    p = _packed(orc, bits, q, np.full(N * K // 128, 2.0 ** -4), z)
    X = np.zeros((M, K), np.int64)
    for m in range(M):
        idx = rng.choice(K, 8, replace=False)
        X[m, idx] = rng.choice([-1, 1], 8)
    Yint = X @ (q - np.repeat(z, 128, axis=1)).T        # exact integers
    Y = orc.gemm(X.astype(np.float16), p)
    assert np.array_equal(Y, Yint * 2.0 ** -4)


def test_gemm_cancellation(orc):
    """+1 on the first half of K and -1 on the second half with mirrored codes:
    partial sums reach thousands of units but the exact result is tiny."""
    K, N = 8192, 4
    half = K // 2
    q = np.zeros((N, K), np.int64)
    q[:, :half] = 15
    q[:, half:] = 15
    q[:, half - 1] = 14    # breaks the symmetry by exactly one code step
    p = _packed(orc, 4, q, np.full(N * K // 128, 0.5), np.zeros(N * K // 128))
    X = np.ones((1, K), np.float16)
    X[0, half:] = -1
    Y = orc.gemm(X, p)
    assert np.all(Y == -0.5)


@pytest.mark.parametrize("bits", [2, 4])
def test_gemm_all_ones_closed_form(orc, bits):
    rng = np.random.default_rng(17)
    K, N = 1024, 32
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    p = orc.pack(W, bits)
    Y = orc.gemm(np.ones((1, K), np.float16), p)[0]
    q = orc.unpack(p).astype(np.int64).reshape(N, K // 128, 128)
    s = orc.halves_to_double(p.scales)
    z = orc.halves_to_double(p.zeros)
    closed = (s * (q.sum(axis=2) - 128 * z)).sum(axis=1)
    assert np.allclose(Y, closed, rtol=1e-13, atol=1e-15)
