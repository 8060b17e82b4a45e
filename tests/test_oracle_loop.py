"""Pins for the oracle's LayerNorm stand-in and loop driver.

The loop's glue (LayerNorm, self-only attention, identity FFN activation) is
this library's reading, not a passage of the pages; these tests pin the oracle
to that written reading with closed forms: LayerNorm of constructed rows,
zero weights (residual unchanged), and diagonal weights, for which each
iteration reduces to h += a*b*LN(h) followed by h += 2*c*d*LN(h).
"""
import numpy as np
import pytest


def test_layernorm_closed_forms(orc):
    D = 256
    c, mu = 0.75, 3.0
    h = np.where(np.arange(D) % 2 == 0, mu + c, mu - c)[None, :]
    x = orc.layernorm(h)
    want = c / np.sqrt(c * c + 1e-5)
    assert np.array_equal(x[0], orc.round_half(np.where(np.arange(D) % 2 == 0, want, -want)))
    # ramp 0..D-1: mean (D-1)/2, population variance (D^2 - 1)/12
    h = np.arange(D, dtype=np.float64)[None, :]
    x = orc.layernorm(h)
    want = (np.arange(D) - (D - 1) / 2) / np.sqrt((D * D - 1) / 12 + 1e-5)
    assert np.array_equal(x[0], orc.round_half(want))


def _diag_packed(orc, K, N, value, pairs, bits=4):
    """Packed weight whose dequant is `value` at (k, n) in pairs, 0 elsewhere."""
    q = np.zeros((N, K), np.int64)
    for k, n in pairs:
        q[n, k] = 1
    per = 32 // bits
    words = np.zeros((N, K // per), dtype=np.uint64)
    for j in range(per):
        words |= q[:, j::per].astype(np.uint64) << np.uint64(16 * (j % 2) + bits * (j // 2))
    G = K // 128
    return orc.Packed(bits, K, N, words.astype(np.uint32),
                      orc.half_bits(np.full((N, G), value)), orc.half_bits(np.zeros((N, G))))


def _random_packed(orc, K, N, bits, seed):
    rng = np.random.default_rng(seed)
    return orc.pack((rng.standard_normal((K, N)) * 0.02).astype(np.float32), bits)


def _np_ln(h):
    mu = h.mean(axis=1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=1, keepdims=True)
    return ((h - mu) / np.sqrt(var + 1e-5)).astype(np.float16).astype(np.float64)


@pytest.mark.parametrize("bits", [2, 4])
def test_loop_with_diagonal_weights_reduces_to_closed_form(orc, bits):
    D, F, M = 128, 256, 3
    a, b, c, d = 0.5, 2.0, 0.25, 1.0
    qk = _random_packed(orc, D, 3 * D, bits, 1)
    v = _diag_packed(orc, D, 3 * D, a, [(k, 2 * D + k) for k in range(D)], bits)
    # Q/K columns random (must not reach h), V columns a*I
    qkv = orc.Packed(bits, D, 3 * D, qk.codes.copy(), qk.scales.copy(), qk.zeros.copy())
    qkv.codes[2 * D:] = v.codes[2 * D:]
    qkv.scales[2 * D:] = v.scales[2 * D:]
    qkv.zeros[2 * D:] = v.zeros[2 * D:]
    out = _diag_packed(orc, D, D, b, [(k, k) for k in range(D)], bits)
    up = _diag_packed(orc, D, F, c, [(k, k) for k in range(D)] + [(k, k + D) for k in range(D)], bits)
    down = _diag_packed(orc, F, D, d, [(n, n) for n in range(D)] + [(n + D, n) for n in range(D)], bits)
    blk = orc.Block(D, F, qkv, out, up, down)
    rng = np.random.default_rng(0)
    h0 = rng.standard_normal((M, D)).astype(np.float16).astype(np.float64)
    h, last = orc.loop_range(blk, h0, 0, 3)
    want = h0.copy()
    for _ in range(3):
        want = want + a * b * _np_ln(want)
        x2 = _np_ln(want)
        want = want + 2 * c * d * x2
    assert np.allclose(h, want, rtol=0, atol=1e-12)
    assert np.array_equal(last["norm"], x2)
    assert np.array_equal(last["u"], np.concatenate([c * x2, c * x2], axis=1))
    assert np.array_equal(last["y"], 2 * c * d * x2)
    # Q/K columns of the last qkv are the random weights applied to LN(h)
    assert np.any(last["qkv"][:, :2 * D] != 0)


def test_loop_zero_weights_leave_residual_unchanged(orc):
    D, F, M = 128, 384, 2
    z = [_diag_packed(orc, K, N, 0.5, []) for K, N in ((D, 3 * D), (D, D), (D, F), (F, D))]
    blk = orc.Block(D, F, *z)
    h0 = np.random.default_rng(1).standard_normal((M, D))
    h, _ = orc.loop_range(blk, h0, 0, 5)
    assert np.array_equal(h, h0)


def test_loop_empty_range_is_noop_and_split_composes(orc):
    D, F, M = 128, 256, 2
    blk = orc.Block(D, F, _random_packed(orc, D, 3 * D, 4, 2), _random_packed(orc, D, D, 4, 3),
                    _random_packed(orc, D, F, 4, 4), _random_packed(orc, F, D, 4, 5))
    h0 = np.random.default_rng(2).standard_normal((M, D)).astype(np.float16).astype(np.float64)
    h, _ = orc.loop_range(blk, h0, 4, 4)
    assert np.array_equal(h, h0)
    h_full, _ = orc.loop_range(blk, h0, 0, 4)
    h_a, _ = orc.loop_range(blk, h0, 0, 1)
    h_b, _ = orc.loop_range(blk, h_a, 1, 4)
    assert np.array_equal(h_full, h_b)
    assert not np.array_equal(h_full, h0)


def test_loop_rejects_bad_ranges(orc):
    D, F = 128, 256
    blk = orc.Block(D, F, _random_packed(orc, D, 3 * D, 4, 2), _random_packed(orc, D, D, 4, 3),
                    _random_packed(orc, D, F, 4, 4), _random_packed(orc, F, D, 4, 5))
    with pytest.raises(orc.OracleError):
        orc.loop_range(blk, np.zeros((1, D)), 3, 2)
    with pytest.raises(orc.OracleError):
        orc.loop_range(blk, np.zeros((1, D)), -1, 2)
