"""Pins for per-token absmax int8 activation quantization.

Pinned against: exact rational round-half-even of 127*x/a over every finite
bf16 x for a range of row maxima a, the IEEE binary32 evaluation order
fl(fl(127*x)/a) (the precision a GPU kernel decides codes in), and invariances.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sbl_inputs import activation, bf16_bits_to_f32, f32_to_bf16_bits

FINITE = np.array([b for b in range(1 << 16) if ((b >> 7) & 0xFF) != 0xFF], dtype=np.uint16)
# a = 127 * 2^k makes 127*x/a = x * 2^-k, so many x land exactly on half-integers (ties)
ABSMAX_CASES = [1.0, 1.984375, 127.0, 3.140625, 0.0078125 * 3, 2.0 ** -130 * 7, 65280.0, 1.7e38, 0.99609375]


def _rows_for(a):
    """One token row per chunk: [a, x_1 .. x_k] for every finite bf16 x with |x| <= a."""
    a_bits = f32_to_bf16_bits(np.array([a], np.float32))[0]
    av = float(bf16_bits_to_f32(np.array([a_bits]))[0])
    xs = FINITE[np.abs(bf16_bits_to_f32(FINITE).astype(np.float64)) <= av]
    k = 255
    pad = (-len(xs)) % k
    xs = np.concatenate([xs, np.zeros(pad, np.uint16)])
    rows = xs.reshape(-1, k)
    return np.concatenate([np.full((rows.shape[0], 1), a_bits, np.uint16), rows], axis=1), av


@pytest.mark.parametrize("a", ABSMAX_CASES)
def test_act_quant_exact_rational(a):
    rows, av = _rows_for(a)
    q, amax = oracle.act_quant(rows)
    assert np.all(amax == np.float32(av))
    xv = oracle.bf16_to_f64(rows)
    A = Fraction(av)
    # exact check near half-integers, cheap exact check elsewhere
    z = 127.0 * xv / av
    frac = np.abs(z - np.floor(z) - 0.5)
    near = frac < 1e-3
    for (r, c) in zip(*np.nonzero(near)):
        want = round(Fraction(127) * Fraction(float(xv[r, c])) / A)   # half-even
        assert q[r, c] == want
    far = ~near
    assert np.array_equal(q[far], np.floor(z[far] + 0.5).astype(np.int8))


@pytest.mark.parametrize("a", ABSMAX_CASES)
def test_act_quant_binary32_sequence_agrees(a):
    # Binary32 evaluation: scale x and a by the same exact power of two so that
    # a lands in [1, 2) (this keeps 127*x finite for |x| near FLT_MAX and a out of the
    # subnormal range), then rint(fl32(fl32(127*x') / a')).  Agreement with the exact
    # result is what lets a binary32 kernel be bit-exact.
    rows, av = _rows_for(a)
    q, _ = oracle.act_quant(rows)
    x32 = bf16_bits_to_f32(rows)
    a32 = np.max(np.abs(x32), axis=1, keepdims=True)
    k = (1 - np.frexp(a32)[1]).astype(np.int32)
    xs, as_ = np.ldexp(x32, k).astype(np.float32), np.ldexp(a32, k).astype(np.float32)
    assert np.all((as_ >= 1) & (as_ < 2))
    q32 = np.rint((np.float32(127.0) * xs) / as_).astype(np.int8)
    assert np.array_equal(q, q32)


@pytest.mark.parametrize("a", ABSMAX_CASES)
def test_act_quant_reciprocal_fast_path_agrees(a):
    # A GPU kernel may replace the division by a multiplication with fl32(127 / a'):
    # qf = fl32(x' * fl32(127 / a')) is within |q| 2^-23 <= 2^-16 of the exact quotient, so
    # rint(qf) is exact whenever qf is more than 2^-14 away from a half-integer; the other
    # elements (ties among them) fall back to the division.  Exhaustive over every bf16 x.
    rows, av = _rows_for(a)
    q, _ = oracle.act_quant(rows)
    x32 = bf16_bits_to_f32(rows)
    a32 = np.max(np.abs(x32), axis=1, keepdims=True)
    k = (1 - np.frexp(a32)[1]).astype(np.int32)
    xs, as_ = np.ldexp(x32, k).astype(np.float32), np.ldexp(a32, k).astype(np.float32)
    c = (np.float32(127.0) / as_).astype(np.float32)
    qf = (xs * c).astype(np.float32)
    r = np.rint(qf)
    slow = np.abs(qf - r) > np.float32(0.5 - 2.0 ** -14)
    r[slow] = np.rint((np.float32(127.0) * xs[slow]) / np.broadcast_to(as_, xs.shape)[slow])
    assert np.array_equal(q, r.astype(np.int8))
    assert slow.mean() < 0.01


def test_act_quant_properties():
    x = activation(0, 0, 64, 256, dist="student_t4")
    q, a = oracle.act_quant(x)
    xv = oracle.bf16_to_f64(x)
    assert np.all(np.abs(q) <= 127)
    arg = np.argmax(np.abs(xv), axis=1)
    assert np.all(np.abs(q[np.arange(64), arg]) == 127)
    assert np.all(np.sign(q) * np.sign(xv) >= 0)
    for t in range(4):                       # monotone within a row
        o = np.argsort(xv[t], kind="stable")
        assert np.all(np.diff(q[t, o].astype(int)) >= 0)
    # scaling a token by 2^k leaves x_q unchanged and scales a_t by 2^k
    xs = f32_to_bf16_bits(bf16_bits_to_f32(x) * np.float32(8.0))
    q2, a2 = oracle.act_quant(xs)
    assert np.array_equal(q2, q) and np.array_equal(a2, a * np.float32(8.0))


def test_act_quant_zero_row_and_empty():
    x = np.zeros((3, 16), np.uint16)
    x[1, 5] = 0x3F80           # 1.0
    x[2, :] = 0x8000           # -0.0 everywhere
    q, a = oracle.act_quant(x)
    assert a.tolist() == [0.0, 1.0, 0.0]
    assert not q[0].any() and not q[2].any()
    assert q[1, 5] == 127 and q[1].sum() == 127
    q, a = oracle.act_quant(np.zeros((0, 16), np.uint16))
    assert q.shape == (0, 16) and a.shape == (0,)
