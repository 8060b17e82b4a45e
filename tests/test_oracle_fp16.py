"""Pins for the oracle's FP16 conversions against numpy's IEEE binary16.

numpy converts float64 -> float16 in one correctly rounded step (ties to
even) and float16 -> float64 exactly; the oracle's conversions are written
independently from the binary16 definition, so agreement on every bit
pattern and on targeted rounding cases pins them.
"""
import numpy as np
import pytest

from conftest import golden  # noqa: F401


def test_half_to_double_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.halves_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_round_half_matches_ieee_on_random_values(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000),
        rng.standard_normal(100000) * 1e-5,     # subnormal range
        rng.standard_normal(100000) * 3e4,      # near overflow
        rng.uniform(-1, 1, 100000) * 2.0 ** rng.integers(-30, 17, 100000),
    ])
    ours = orc.round_half(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(ours, ref)
    with np.errstate(over="ignore"):
        ref_bits = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.half_bits(x), ref_bits)


@pytest.mark.parametrize("x,expect", [
    (1.0 + 2.0 ** -11, 1.0),                  # tie between 1 and 1+2^-10 -> even (1.0)
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2 * 2.0 ** -10),  # tie -> even mantissa 2
    (65504.0, 65504.0),
    (65519.99, 65504.0),
    (65520.0, np.inf),                         # tie between 65504 and 2^16 -> inf
    (2.0 ** -24, 2.0 ** -24),                  # smallest subnormal
    (2.0 ** -25, 0.0),                         # tie with 0 -> even (0)
    (3 * 2.0 ** -25, 2.0 ** -23),              # tie between 1 and 2 subnormal units -> 2
    (-(1.0 + 2.0 ** -11), -1.0),
])
def test_round_half_special_cases(orc, x, expect):
    assert orc.round_half(np.array([x]))[0] == expect
