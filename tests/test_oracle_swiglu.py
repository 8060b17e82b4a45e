"""Pins of the oracle's SwiGLU FFN (a block with a gate weight).

The pages name the loop block's five weights (attn_qkv, attn_out, mlp_gate,
mlp_up, mlp_down; "β-Informed Deployment Features", CTX-TIER Phase 2) and
define ffn_dim as the width of the gate and up projections for SwiGLU
("Model" page, Parameters).  The reading: a = fp16(silu(g) * u) with
g = fp16(x . Wgate), u = fp16(x . Wup), silu(z) = z / (1 + e^-z).

Pins: silu's special values and its odd-part identity; a zero gate makes the
FFN contribute exactly nothing; a diagonal block whose weights are exact in
INT4 reduces one iteration to an element-wise formula, evaluated here with
numpy's float16 casts and scipy's logistic function (asymmetric gate and up
scales, so swapped operands or a sign error in the exponent fail).
"""
import math

import numpy as np
import pytest
from scipy.special import expit


def test_silu_special_values(orc):
    assert orc.silu(0.0) == 0.0
    assert orc.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    for z in (0.1, 1.0, 2.5, 7.0, 30.0):
        assert orc.silu(z) - orc.silu(-z) == pytest.approx(z, rel=1e-14)
    assert orc.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(orc.silu(-40.0)) < 1e-15


def _block_weights(D, F, seed):
    rng = np.random.default_rng(seed)
    return {k: (rng.standard_normal(s) * 0.02).astype(np.float32)
            for k, s in (("qkv", (D, 3 * D)), ("out", (D, D)), ("gate", (D, F)),
                         ("up", (D, F)), ("down", (F, D)))}


def test_zero_gate_contributes_nothing(orc):
    D, F, M = 128, 256, 3
    W = _block_weights(D, F, 1)
    W["gate"][:] = 0.0
    gated = orc.pack_block(W, 4, D, F)
    Wn = dict(W)
    Wn["down"] = np.zeros_like(W["down"])
    plain = orc.pack_block({k: Wn[k] for k in ("qkv", "out", "up", "down")}, 4, D, F)
    h0 = np.random.default_rng(2).standard_normal((M, D))
    hg, last = orc.loop_range(gated, h0, 0, 2)
    hp, _ = orc.loop_range(plain, h0, 0, 2)
    assert np.array_equal(hg, hp)
    assert np.all(last["u"] == 0.0)


@pytest.mark.parametrize("a,b,c", [(15 / 16, 15 / 32, 15 / 64), (15 / 64, 15 / 16, 15 / 8)])
def test_diagonal_block_closed_form(orc, a, b, c):
    """Wqkv = Wout = 0 (attention adds nothing), Wgate = a I, Wup = b I,
    Wdown = c I with a/15, b/15, c/15 powers of two (exact INT4 weights):
    h' = h + fp16(c * fp16(silu(fp16(a x)) * fp16(b x))), x = fp16(LN(h))."""
    D = F = 128
    M = 5
    W = {"qkv": np.zeros((D, 3 * D), np.float32), "out": np.zeros((D, D), np.float32),
         "gate": (a * np.eye(D)).astype(np.float32), "up": (b * np.eye(D)).astype(np.float32),
         "down": (c * np.eye(D)).astype(np.float32)}
    blk = orc.pack_block(W, 4, D, F)
    h0 = np.random.default_rng(3).standard_normal((M, D)) * 2.0
    got, last = orc.loop_range(blk, h0, 0, 1)

    f16 = lambda v: np.asarray(v, np.float64).astype(np.float16).astype(np.float64)
    mu = h0.mean(axis=1, keepdims=True)
    var = ((h0 - mu) ** 2).mean(axis=1, keepdims=True)
    x = f16((h0 - mu) / np.sqrt(var + 1e-5))
    g = f16(a * x)
    u = f16(b * x)
    act = f16(g * expit(g) * u)
    want = h0 + f16(c * act)
    np.testing.assert_allclose(got, want, rtol=1e-3, atol=1e-6)
    np.testing.assert_allclose(last["g"], g, rtol=1e-3, atol=1e-6)
    np.testing.assert_allclose(last["u"], act, rtol=1e-3, atol=1e-6)
    # the gate really matters here: silu applied to u instead would differ
    wrong = h0 + f16(c * f16(u * expit(u) * g))
    assert np.max(np.abs(wrong - want)) > 1e-2
