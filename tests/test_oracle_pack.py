"""Pins for the oracle's quantiser/packer (qg_pack's definition).

Pinned against: hand-worked groups (tests/golden/int*_ramp_group.json), an
exact-rational re-derivation (oracle/brute.py) on small random inputs, the
quantisation error bound |w^ - w| <= s/2, the uniform-noise law
MSE = s^2/12, the pages' byte counts for the loop block, and the degenerate
groups whose answer is fixed by the definition.
"""
import numpy as np
import pytest

from conftest import golden
from oracle import brute


def _ramp():
    k = np.arange(128, dtype=np.float64)
    return ((k - 32) / 64).astype(np.float32).reshape(128, 1)


def test_int2_ramp_group_hand_worked(orc):
    gd = golden("int2_ramp_group.json")
    p = orc.pack(_ramp(), 2)
    assert int(p.scales[0, 0]) == gd["scale_bits"]
    assert orc.half_to_double(p.scales[0, 0]) == gd["scale_value"]
    assert int(p.zeros[0, 0]) == gd["zero_bits"]
    assert [int(w) for w in p.codes[0]] == gd["words"]
    q = orc.unpack(p)[0]
    for lo, hi, code in gd["code_ranges"]:
        assert np.all(q[lo:hi + 1] == code)
    dq = orc.dequant(p)[0]
    for k in range(128):
        assert dq[k] == gd["dequant_by_code"][str(int(q[k]))]


def test_int4_ramp_group_hand_worked(orc):
    gd = golden("int4_ramp_group.json")
    p = orc.pack(_ramp(), 4)
    assert int(p.scales[0, 0]) == gd["scale_bits"]
    assert int(p.zeros[0, 0]) == gd["zero_bits"]
    q = orc.unpack(p)[0]
    for k, code in gd["sample_codes"].items():
        assert int(q[int(k)]) == code, k


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pack_matches_exact_rational_brute_force(orc, bits, seed):
    rng = np.random.default_rng(seed)
    K, N = 256, 3
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    if seed == 2:  # one all-positive and one all-negative group
        W[:128, 0] = np.abs(W[:128, 0])
        W[128:, 1] = -np.abs(W[128:, 1])
    p = orc.pack(W, bits)
    S, Z, Q = brute.pack(W.tolist(), bits)
    for n in range(N):
        for g in range(K // 128):
            assert orc.half_to_double(p.scales[n, g]) == float(S[n][g])
            assert orc.half_to_double(p.zeros[n, g]) == float(Z[n][g])
        assert [int(w) for w in p.codes[n]] == brute.words(Q[n], bits)


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_error_bound_and_ranges(orc, bits):
    rng = np.random.default_rng(7)
    K, N = 1024, 64
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    p = orc.pack(W, bits)
    qmax = (1 << bits) - 1
    q = orc.unpack(p).astype(np.int64)
    s = orc.halves_to_double(p.scales)            # [N][G]
    z = orc.halves_to_double(p.zeros)
    assert q.min() >= 0 and q.max() <= qmax
    assert z.min() >= 0 and z.max() <= qmax and np.all(z == np.round(z))
    dq = orc.dequant(p)                           # [N][K]
    err = np.abs(dq - W.T.astype(np.float64))
    s_k = np.repeat(s, 128, axis=1)
    # Away from the group's clamped extremes the error is at most s/2.
    inner = (q > 0) & (q < qmax)
    assert np.all(err[inner] <= s_k[inner] / 2 * (1 + 1e-12))
    # At the extremes the excess comes only from rounding s to FP16.
    lo = W.T.reshape(N, -1, 128).min(axis=2).clip(max=0)
    hi = W.T.reshape(N, -1, 128).max(axis=2).clip(min=0)
    s_exact = np.repeat((hi - lo) / qmax, 128, axis=1)
    bound = s_k / 2 + qmax * np.abs(s_k - s_exact) + 1e-12
    assert np.all(err <= bound)


def test_pack_noise_law(orc):
    """Uniform rounding noise: mean squared error ~ mean(s^2)/12."""
    rng = np.random.default_rng(11)
    K, N = 2048, 512
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    for bits in (2, 4):
        p = orc.pack(W, bits)
        dq = orc.dequant(p)
        q = orc.unpack(p)
        qmax = (1 << bits) - 1
        inner = (q > 0) & (q < qmax)
        err2 = (dq - W.T.astype(np.float64)) ** 2
        s2 = np.repeat(orc.halves_to_double(p.scales) ** 2, 128, axis=1)
        ratio = err2[inner].mean() / (s2[inner].mean() / 12)
        assert 0.95 <= ratio <= 1.05, (bits, ratio)


def test_exact_zero_weight_dequantises_to_plus_zero(orc):
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((256, 8)) * 0.02).astype(np.float32)
    W[5, :] = 0.0
    W[200, 3] = 0.0
    for bits in (2, 4):
        p = orc.pack(W, bits)
        q = orc.unpack(p)
        z = orc.halves_to_double(p.zeros)
        dq = orc.dequant(p)
        assert np.all(q[:, 5] == z[:, 0])
        assert q[3, 200] == z[3, 1]
        assert np.all(dq[:, 5] == 0) and not np.any(np.signbit(dq[:, 5]))
        assert dq[3, 200] == 0 and not np.signbit(dq[3, 200])


def test_degenerate_groups(orc):
    W = np.zeros((256, 3), dtype=np.float32)
    W[128:, 1] = np.linspace(0.1, 0.3, 128)      # all positive: z = 0
    W[128:, 2] = -np.linspace(0.1, 0.3, 128)     # all negative: z = qmax
    for bits in (2, 4):
        qmax = (1 << bits) - 1
        p = orc.pack(W, bits)
        q = orc.unpack(p)
        s = orc.halves_to_double(p.scales)
        z = orc.halves_to_double(p.zeros)
        # all-zero group: s = 1, z = 0, q = 0, dequant exactly 0
        assert s[0, 0] == 1.0 and z[0, 0] == 0 and np.all(q[0, :128] == 0)
        assert np.all(orc.dequant(p)[:, :128] == 0)
        assert z[1, 1] == 0 and q[1, 255] == qmax
        assert z[2, 1] == qmax and q[2, 255] == 0


def test_pack_rejects_non_finite_and_overflow(orc):
    W = np.zeros((128, 2), dtype=np.float32)
    W[3, 1] = np.nan
    with pytest.raises(orc.OracleError):
        orc.pack(W, 4)
    W[3, 1] = np.inf
    with pytest.raises(orc.OracleError):
        orc.pack(W, 4)
    W[3, 1] = 3e38   # scale (3e38)/15 overflows FP16
    with pytest.raises(orc.OracleError):
        orc.pack(W, 4)
    W[3, 1] = 65504.0 * 3   # INT2: range/3 = 65504 fits exactly
    p = orc.pack(W, 2)
    assert orc.half_to_double(p.scales[1, 0]) == 65504.0


def test_loop_block_code_bytes_match_the_pages(orc):
    """The oracle's pack of the five-weight loop block (seeded N(0, 0.02)
    weights of the page's shapes) gives exactly the page's 32 MB of INT4 codes
    and 16 MB after the INT2 re-pack, i.e. K/2-byte INT4 and K/4-byte INT2
    rows, and its re-quantisation frees the page's 16 MB."""
    import workloads
    gd = golden("loop_block_bytes.json")
    g = workloads.generator(0)
    totals = {4: 0, 2: 0}
    requant = 0
    for K, N in gd["five_weights_KN"]:
        W = workloads.weight(K, N, g).numpy()
        p4 = orc.pack(W, 4)
        p2 = orc.pack(W, 2)
        assert p4.codes.shape == (N, K // 8) and p4.codes.dtype == np.uint32   # K/2 bytes a row
        assert p2.codes.shape == (N, K // 16) and p2.codes.dtype == np.uint32  # K/4 bytes a row
        totals[4] += p4.codes.nbytes
        totals[2] += p2.codes.nbytes
        requant += orc.requant_4to2(p4).codes.nbytes
    assert totals[4] == gd["int4_code_bytes_five"]
    assert totals[2] == gd["int2_code_bytes_five"] == requant
    assert totals[4] - requant == gd["freed_bytes"]
