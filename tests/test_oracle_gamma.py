"""Pins for the oracle's gamma (mean |W|, correctly rounded to binary32).

Pinned against: numpy's correctly rounded float64 -> float32 conversion, a
brute-force nearest-neighbour search with exact fractions, exact Fraction sums,
and closed forms (constant-magnitude matrices, power-of-two scaling).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sbl_inputs import f32_to_bf16_bits, weight


def _f32_neighbours(f):
    f = np.float32(f)
    return float(np.nextafter(f, np.float32(-np.inf))), float(np.nextafter(f, np.float32(np.inf)))


def test_round_rational_matches_numpy_on_exact_doubles():
    # Any float64 v is num/den exactly; numpy's float64->float32 cast rounds once, to nearest-even.
    g = np.random.default_rng(1)
    vals = np.concatenate([
        g.standard_normal(4000) * 10.0 ** g.integers(-40, 38, 4000),
        np.abs(g.standard_normal(500)) * 2.0 ** -140,   # binary32 subnormal range
        np.abs(g.standard_normal(500)) * 2.0 ** -127,
    ])
    vals = np.abs(vals)
    # exact ties: a binary32 value plus half an ulp
    base = np.abs(g.standard_normal(500)).astype(np.float32)
    nxt = np.nextafter(base, np.float32(np.inf))
    ties = (base.astype(np.float64) + nxt.astype(np.float64)) / 2.0
    vals = np.concatenate([vals, ties])
    for v in vals:
        if v > 3.0e38:
            continue
        num, den = float(v).as_integer_ratio()
        assert oracle.round_rational_to_f32(num, den) == float(np.float32(v)), v


def test_round_rational_brute_force_nearest_even():
    g = np.random.default_rng(2)
    for _ in range(3000):
        den = int(g.integers(1, 10 ** 12))
        num = int(g.integers(0, 10 ** 12)) * int(2 ** int(g.integers(0, 40)))
        if g.random() < 0.3:
            den *= 2 ** int(g.integers(100, 170))   # push into the subnormal range
        x = Fraction(num, den)
        f = oracle.round_rational_to_f32(num, den)
        if float(x) > 3.0e38:
            continue
        lo, hi = _f32_neighbours(f)
        d = abs(x - Fraction(f))
        assert d <= abs(x - Fraction(lo)) and d <= abs(x - Fraction(hi))
        if d == abs(x - Fraction(hi)) or (lo >= 0 and d == abs(x - Fraction(lo))):
            # tie: the significand of f must be even
            bits = int(np.float32(f).view(np.uint32))
            assert bits & 1 == 0


def test_abs_sum_exact_matches_fraction_sum():
    g = np.random.default_rng(3)
    bits = g.integers(0, 0x7F80, size=(13, 24), dtype=np.uint16)   # every finite magnitude incl. subnormals
    bits |= (g.integers(0, 2, size=bits.shape).astype(np.uint16) << 15)
    total = sum(abs(Fraction(float(v))) for v in oracle.bf16_to_f64(bits).ravel())
    assert Fraction(oracle.abs_sum_exact(bits), 2 ** 133) == total


def test_gamma_constant_magnitude():
    # mean of a constant-magnitude matrix is that magnitude, exactly
    for v in (0.0234375, 1.0, 3.0e-20, 2.0 ** -130):
        b = f32_to_bf16_bits(np.full((7, 16), v, dtype=np.float32))
        b[::2] |= 0x8000
        expect = float(oracle.bf16_to_f64(b[0, 0:1])[0])
        assert float(oracle.gamma_f32(b)) == abs(expect)


def test_gamma_scales_by_powers_of_two():
    W = weight(0, 0, 64, 256)
    g0 = float(oracle.gamma_f32(W))
    for k in (-5, 3, 11):
        Wk = f32_to_bf16_bits(oracle.bf16_to_f64(W).astype(np.float32) * np.float32(2.0 ** k))
        assert float(oracle.gamma_f32(Wk)) == math.ldexp(g0, k)


def test_gamma_zero_matrix():
    assert float(oracle.gamma_f32(np.zeros((4, 8), np.uint16))) == 0.0
    assert float(oracle.gamma_f32(np.full((4, 8), 0x8000, np.uint16))) == 0.0   # -0.0


def test_gamma_explainer_values():
    # The 8 weights of the explainer page's worked N:M example, rounded to bf16:
    # 0.80078125 + 0.30078125 + 0.5 + 1.203125 + 0.69921875 + 0.2001953125
    # + 0.8984375 + 0.400390625 = 5.0029296875, and 5.0029296875 / 8 is exact in binary32.
    W = f32_to_bf16_bits(np.array([[0.8, -0.3, 0.5, 1.2, -0.7, 0.2, 0.9, -0.4]], np.float32))
    assert float(oracle.gamma_f32(W)) == 0.6253662109375


def test_gamma_rounding_is_not_naive_float_sum():
    # gamma is independent of summation order: permuting W leaves it bit-identical
    W = weight(0, 1, 37, 64)
    perm = np.random.default_rng(5).permutation(W.size)
    assert oracle.gamma_f32(W) == oracle.gamma_f32(W.ravel()[perm].reshape(W.shape))


@pytest.mark.parametrize("shape", [(1, 8), (3, 8), (256, 256)])
def test_gamma_equals_fraction_mean(shape):
    W = weight(9, shape[0], *shape)
    mean = sum(abs(Fraction(float(v))) for v in oracle.bf16_to_f64(W).ravel()) / W.size
    f = float(oracle.gamma_f32(W))
    lo, hi = _f32_neighbours(f)
    assert abs(mean - Fraction(f)) <= abs(mean - Fraction(lo))
    assert abs(mean - Fraction(f)) <= abs(mean - Fraction(hi))
