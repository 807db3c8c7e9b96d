"""Pins for the oracle's RMSNorm + activation quantization (the Q_a(Norm(x)) of
[SUM] 方法步骤详情 step (3)): the float64 RMSNorm within the bf16 rounding of the
output, one-hot rows (every element is summed exactly once, closed form
y = sign(v) sqrt(d)), an all-zero row, and the weight vector scaling.

The binary32 summation order is fixed by the oracle's docstring; it is checked
here only through these bounds and cases, not value by value."""
import numpy as np
import pytest

import oracle
from sbl_inputs import activation, f32_to_bf16_bits


@pytest.mark.parametrize("d", [64, 2048, 11008])
def test_rmsnorm_within_bf16_rounding_of_float64(d):
    x = activation(5, d, 6, d, dist="student_t4")
    g = f32_to_bf16_bits(np.random.default_rng(d).uniform(0.5, 1.5, d).astype(np.float32))
    eps = 1e-6
    y = oracle.bf16_to_f64(oracle.rmsnorm_bf16(x, g, eps))
    xf = oracle.bf16_to_f64(x)
    ref = xf / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + eps) * oracle.bf16_to_f64(g)
    assert np.all(np.abs(y - ref) <= (2.0 ** -8 + 2.0 ** -20) * np.abs(ref))


def test_rmsnorm_one_hot_rows():
    d = 2048
    for v in (1.0, -3.0, 0.015625):
        x = np.zeros((d, d), np.float32)
        np.fill_diagonal(x, v)
        y = oracle.bf16_to_f64(oracle.rmsnorm_bf16(f32_to_bf16_bits(x), None, 0.0))
        diag = np.diag(y)
        assert np.all(diag == np.sign(v) * np.sqrt(d)) or np.all(np.abs(diag - np.sign(v) * np.sqrt(d)) <= 2.0 ** -8 * np.sqrt(d))
        assert np.count_nonzero(y - np.diag(diag)) == 0


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
