"""Pins for the oracle's RMSNorm + activation quantization (the Q_a(Norm(x)) of
[SUM] 方法步骤详情 step (3)).

The definition: ms = RN32(exact mean of x^2), r = RN32(1 / sqrt(RN32(ms + eps))),
y = bf16(RN32(RN32(x r) g)).  Pinned here by

* exact rational arithmetic (``fractions``) with a nearest-value search over the
  binary32 neighbours, for the mean square and for the reciprocal square root
  (a different route from the oracle's integer-square-root rounding);
* hand-worked rows whose mean square is exactly a binary32 midpoint, or a
  midpoint plus a tiny term, where any rounded partial sum goes wrong;
* invariance of every output bit under a permutation of the row;
* closed forms: one-hot and constant rows, subnormal and overflowing rows;
* float64 RMSNorm within the bf16 rounding of the output.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sbl_inputs import activation, f32_to_bf16_bits

F32_MAX = Fraction(float(np.finfo(np.float32).max))


def _bits(vals):
    return f32_to_bf16_bits(np.asarray(vals, np.float32).reshape(1, -1))


def _nearest_f32_by_search(value: Fraction) -> np.float32:
    """Binary32 nearest to a non-negative rational: start from float64's guess and
    step over the neighbours while one is nearer (ties: even significand)."""
    if value > F32_MAX + Fraction(2) ** 103:     # beyond the overflow threshold
        return np.float32(np.inf)
    c = np.float32(float(value)) if float(value) < 3.4e38 else np.float32(np.finfo(np.float32).max)
    best = c
    for _ in range(4):
        for cand in (np.nextafter(best, np.float32(0)), np.nextafter(best, np.float32(np.inf))):
            if not np.isfinite(cand):
                continue
            db = abs(Fraction(float(best)) - value)
            dc = abs(Fraction(float(cand)) - value)
            if dc < db or (dc == db and (int(np.float32(cand).view(np.uint32)) & 1) == 0):
                best = np.float32(cand)
    return best


def _exact_mean_square(row_bits) -> Fraction:
    xs = [Fraction(float(v)) for v in oracle.bf16_to_f64(np.asarray(row_bits, np.uint16))]
    return sum((v * v for v in xs), Fraction(0)) / len(xs)


@pytest.mark.parametrize("seed", range(4))
def test_mean_square_against_fractions(seed):
    g = np.random.default_rng(seed)
    d = int(g.choice([8, 24, 64, 200]))
    # values spread over many binades, signs mixed, some zeros and subnormals
    mag = np.exp2(g.uniform(-140, 60, size=(6, d))) * g.choice([-1, 1], size=(6, d))
    mag[g.random((6, d)) < 0.1] = 0.0
    x = f32_to_bf16_bits(mag.astype(np.float32))
    got = oracle.mean_square_f32(x)
    for t in range(x.shape[0]):
        ref = _nearest_f32_by_search(_exact_mean_square(x[t]))
        assert got[t].view(np.uint32) == ref.view(np.uint32), (t, float(got[t]), float(ref))


def test_mean_square_midpoint_rows():
    """Hand-worked: six ones and 2^-11 over d = 8 give a mean square of exactly
    3/4 + 2^-25, the midpoint between 3/4 and the next binary32 (spacing 2^-24 on
    [1/2, 1)); ties go to the even 3/4.  A 2^-100 in the eighth slot adds 2^-203
    and the mean rounds up to 3/4 + 2^-24.  A float32 running sum loses the 2^-22
    (it is half an ulp of 6) and gives 3/4 for both."""
    tie = _bits([1, 1, 1, 1, 1, 1, 2.0 ** -11, 0])
    above = _bits([1, 1, 1, 1, 1, 1, 2.0 ** -11, 2.0 ** -100])
    assert oracle.mean_square_f32(tie)[0] == np.float32(0.75)
    assert oracle.mean_square_f32(above)[0] == np.float32(0.75 + 2.0 ** -24)
    # the same rows in another order give the same bits
    assert oracle.mean_square_f32(above[:, ::-1].copy())[0] == np.float32(0.75 + 2.0 ** -24)


def test_mean_square_closed_forms():
    # constant rows: the square of a bf16 is exact in binary32
    for c in (1.5, -0.01171875, 3.0e-20, 1.0e18):
        cb = f32_to_bf16_bits(np.float32(c).reshape(1))
        cv = float(oracle.bf16_to_f64(cb)[0])
        row = np.repeat(cb, 40).reshape(1, 40)
        assert oracle.mean_square_f32(row)[0] == np.float32(cv * cv)
    # the smallest subnormal squared is 2^-266: rounds to zero
    assert oracle.mean_square_f32(np.full((1, 16), 1, np.uint16))[0] == 0.0
    # the largest bf16 squared overflows binary32
    assert np.isinf(oracle.mean_square_f32(np.full((1, 16), 0x7F7F, np.uint16))[0])


def _is_nearest_rsqrt(v: np.float32, r: np.float32) -> bool:
    """r is the binary32 nearest to 1/sqrt(v) iff both neighbouring midpoints m
    bracket it: m_lo^2 v < 1 < m_hi^2 v (exact rationals)."""
    fv, fr = Fraction(float(v)), Fraction(float(r))
    lo = (fr + Fraction(float(np.nextafter(r, np.float32(0))))) / 2
    hi = (fr + Fraction(float(np.nextafter(r, np.float32(np.inf))))) / 2
    return lo * lo * fv < 1 < hi * hi * fv


def test_rsqrt_nearest_by_fractions():
    g = np.random.default_rng(7)
    vs = np.concatenate([
        np.exp2(g.uniform(-149, 127.9, 600)).astype(np.float32),
        g.uniform(0.5, 4.0, 400).astype(np.float32),
        np.array([np.finfo(np.float32).tiny, np.finfo(np.float32).max, 1.4e-45, 2.0, 3.0, 0.75], np.float32),
    ])
    vs = vs[vs > 0]
    for v in vs:
        assert _is_nearest_rsqrt(v, oracle.rsqrt_rn32(v)), float(v)


def test_rsqrt_closed_forms():
    for k in range(-74, 64):
        assert oracle.rsqrt_rn32(np.float32(4.0 ** k)) == np.float32(2.0 ** -k)
    assert oracle.rsqrt_rn32(np.float32(np.inf)) == 0.0


@pytest.mark.parametrize("d", [64, 2048, 11008])
def test_rmsnorm_within_bf16_rounding_of_float64(d):
    x = activation(5, d, 6, d, dist="student_t4")
    g = f32_to_bf16_bits(np.random.default_rng(d).uniform(0.5, 1.5, d).astype(np.float32))
    eps = 1e-6
    y = oracle.bf16_to_f64(oracle.rmsnorm_bf16(x, g, eps))
    xf = oracle.bf16_to_f64(x)
    ref = xf / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + eps) * oracle.bf16_to_f64(g)
    assert np.all(np.abs(y - ref) <= (2.0 ** -8 + 2.0 ** -20) * np.abs(ref))


def test_rmsnorm_permutation_invariant():
    d = 512
    x = activation(8, 1, 5, d, dist="student_t4")
    g = f32_to_bf16_bits(np.random.default_rng(3).uniform(0.5, 1.5, d).astype(np.float32))
    perm = np.random.default_rng(4).permutation(d)
    y = oracle.rmsnorm_bf16(x, g, 1e-6)
    yp = oracle.rmsnorm_bf16(x[:, perm].copy(), g[perm].copy(), 1e-6)
    assert np.array_equal(yp, y[:, perm])
    assert np.array_equal(oracle.rmsnorm_rstd(x[:, perm].copy(), 1e-6), oracle.rmsnorm_rstd(x, 1e-6))


def test_rmsnorm_one_hot_rows():
    """One non-zero v in a row of d: ms = v^2 / d, and with eps below half an ulp
    of ms, r = RN32(sqrt(d) / |v|); for v = +-1 and d = 2048 the output is
    bf16(RN32(2^5.5)) = 45.25 at the non-zero and 0 elsewhere."""
    d = 2048
    for v in (1.0, -1.0):
        x = np.zeros((4, d), np.float32)
        x[np.arange(4), [0, 7, 100, d - 1]] = v
        y = oracle.bf16_to_f64(oracle.rmsnorm_bf16(f32_to_bf16_bits(x), None, 2.0 ** -149))
        nz = y[np.arange(4), [0, 7, 100, d - 1]]
        assert np.all(nz == v * 45.25)
        assert np.count_nonzero(y) == 4


def test_rmsnorm_constant_rows_rstd():
    # x = c: ms = c^2 exactly, r = RN32(1 / sqrt(RN32(c^2 + eps)))
    for c, eps in ((2.0, 2.0 ** -30), (0.25, 1e-6), (3.0, 1e-5)):
        row = f32_to_bf16_bits(np.full((1, 64), c, np.float32))
        r = oracle.rmsnorm_rstd(row, eps)[0]
        v = np.float32(np.float32(c * c) + np.float32(eps))
        assert _is_nearest_rsqrt(v, r)


def test_rmsnorm_zero_row_and_weight_scaling():
    d = 256
    x = activation(6, 0, 3, d)
    x[1] = 0
    y1 = oracle.rmsnorm_bf16(x, None, 1e-5)
    assert not np.any(oracle.bf16_to_f64(y1[1]))
    xq, a = oracle.rmsnorm_act_quant(x, None, 1e-5)
    assert a[1] == 0 and not np.any(xq[1])
    # a weight of 2 (exact power of two) doubles every output bit for bit
    g2 = f32_to_bf16_bits(np.full(d, 2.0, np.float32))
    y2 = oracle.rmsnorm_bf16(x, g2, 1e-5)
    assert np.array_equal(oracle.bf16_to_f64(y2), 2.0 * oracle.bf16_to_f64(y1))
    # x_q of a scaled-by-2 norm output equals that of the unscaled one (absmax scales too)
    xq2, a2 = oracle.act_quant(y2)
    assert np.array_equal(xq2, xq) and np.array_equal(a2, 2 * a)


def test_rmsnorm_overflowing_row_gives_zeros():
    # the largest bf16 squared overflows: ms = inf, r = 0, y = 0
    x = np.full((1, 16), 0x7F7F, np.uint16)
    assert oracle.rmsnorm_rstd(x, 1e-6)[0] == 0.0
    assert not np.any(oracle.bf16_to_f64(oracle.rmsnorm_bf16(x, None, 1e-6)))
