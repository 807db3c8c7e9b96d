"""Pins for ternary quantization, quant-then-mask and the packed planes.

Pinned against: RoundClip(w/gamma, -1, 1) in exact rational arithmetic over
every finite bf16 value, constructed exact-boundary rows, the closed-form zero
fraction for Gaussian weights, and hand-built packing examples.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sbl_inputs import boundary_row_weight, f32_to_bf16_bits, weight

ALL_FINITE_BF16 = np.array([b for b in range(1 << 16) if ((b >> 7) & 0xFF) != 0xFF], dtype=np.uint16)


def _roundclip_exact(w: Fraction, gamma: Fraction) -> int:
    """RoundClip(w / gamma, -1, 1) with round-half-even, in exact arithmetic."""
    if gamma == 0:
        return 0
    return max(-1, min(1, round(w / gamma)))   # Fraction.__round__ is half-even


@pytest.mark.parametrize("gamma", [0.0234375, 0.6253662109375, 1.0, 2.0 ** -130, 3.0e-3])
def test_ternary_exhaustive_against_roundclip(gamma):
    got = oracle.ternary(ALL_FINITE_BF16, np.float32(gamma))
    vals = oracle.bf16_to_f64(ALL_FINITE_BF16)
    G = Fraction(float(np.float32(gamma)))
    # RoundClip only differs from 0 above |w| >= gamma/2; check every value, but use a
    # cheap exact shortcut far from the threshold to keep the test fast
    for b, v, q in zip(ALL_FINITE_BF16, vals, got):
        if abs(v) < float(G) / 4 or abs(v) > float(G) * 4:
            want = 0 if abs(v) < float(G) / 4 else (1 if v > 0 else -1)
        else:
            want = _roundclip_exact(Fraction(float(v)), G)
        assert q == want, (hex(int(b)), v, q, want)


def test_ternary_boundary_rows():
    W = boundary_row_weight(4, 16)      # |w| alternates 0.5, 1.5 -> gamma = 1 exactly
    g = oracle.gamma_f32(W)
    assert float(g) == 1.0
    q = oracle.ternary(W, g)
    sign = np.sign(oracle.bf16_to_f64(W))
    expect = np.tile(np.array([0, 1] * 8), (4, 1)) * sign
    assert np.array_equal(q, expect)


def test_dense_8of8_is_plain_absmean_ternary():
    W = weight(0, 3, 48, 128)
    w_eff, mask, g = oracle.effective_weight(W, 8)
    assert mask.all()
    assert np.array_equal(w_eff, oracle.ternary(W, g))


def test_quant_then_mask_uses_full_matrix_gamma():
    W = weight(0, 4, 32, 64)
    for n in (2, 4, 6):
        w_eff, mask, g = oracle.effective_weight(W, n)
        assert g == oracle.gamma_f32(W)                # gamma never sees the mask
        q = oracle.ternary(W, g)
        assert np.all(w_eff[~mask] == 0)
        assert np.array_equal(w_eff[mask], q[mask])
        assert set(np.unique(w_eff)).issubset({-1, 0, 1})
        # at most N non-zeros per group (kept slots may quantize to 0)
        assert np.all((w_eff != 0).reshape(32, 8, 8).sum(-1) <= n)


def test_pack_codes_bit_layout():
    w = np.array([[1, 0, -1, 0, 0, 0, 0, 1, -1, -1, -1, -1, -1, -1, -1, -1]], np.int8)
    c = oracle.pack_codes(w)
    assert c.shape == (1, 2)
    assert int(c[0, 0]) == (0b01 << 0) | (0b11 << 4) | (0b01 << 14)
    assert int(c[0, 1]) == 0xFFFF
    assert np.array_equal(oracle.unpack_codes(c), w)
    m = oracle.pack_mask(np.array([[1, 0, 1, 1, 1, 0, 1, 1] * 2], bool))
    assert m.tolist() == [[0b11011101, 0b11011101]]


def test_pack_roundtrip_random():
    W = weight(0, 5, 40, 96)
    w_eff, mask, g = oracle.effective_weight(W, 6)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(w_eff)), w_eff)
    codes = oracle.pack_codes(w_eff)
    for j in range(8):
        assert not np.any(((codes >> (2 * j)) & 3) == 0b10)


def _masked_zero_fraction(n_keep: int, p0: float) -> float:
    """E[max(K, 8 - N)] / 8 with K ~ Binomial(8, p0): zeros in a group are the masked
    8 - N smallest plus any kept entries that still fall under the ternary threshold."""
    drop = 8 - n_keep
    return sum(math.comb(8, k) * p0 ** k * (1 - p0) ** (8 - k) * max(k, drop) for k in range(9)) / 8


def test_gaussian_zero_fraction_closed_form():
    # For i.i.d. N(0, s^2) weights, E|w| = s*sqrt(2/pi), so a weight quantizes to 0 with
    # probability P(|z| <= sqrt(2/pi)/2) = erf(1/(2*sqrt(pi))) = 0.310064...
    p0 = math.erf(1.0 / (2.0 * math.sqrt(math.pi)))
    assert abs(p0 - 0.310064) < 1e-6
    W = weight(77, 0, 1024, 2048)
    n = W.size
    for n_keep, closed in ((8, 0.310064), (6, 0.345973), (4, 0.510162), (2, 0.750211)):
        assert abs(_masked_zero_fraction(n_keep, p0) - closed) < 1e-6
        w_eff, _, _ = oracle.effective_weight(W, n_keep)
        frac = float(np.mean(w_eff == 0))
        sigma = math.sqrt(closed * (1 - closed) / n)
        assert abs(frac - closed) < 6 * sigma + 2e-4, (n_keep, frac, closed)
        # the two signs are equally likely
        plus, minus = np.mean(w_eff == 1), np.mean(w_eff == -1)
        assert abs(plus - minus) < 6 * math.sqrt((1 - closed) / 2 / n) + 2e-4


def test_ternary_zero_gamma():
    assert not oracle.ternary(np.zeros((2, 8), np.uint16), np.float32(0.0)).any()
