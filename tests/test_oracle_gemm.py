"""Pins for the forward product, its dequantization and the Dual-STE backward.

Pinned against: exact int64 matrix products, PyTorch CPU float64 autograd of
the straight-through-estimator expression (an independent formulation of the
backward), the dense 8:8 special case, and the Dual-STE invariant that masked
weights receive the dense gradient (versus the stop-gradient ablation).
"""
import numpy as np
import pytest
import torch

import oracle
from sbl_inputs import activation, grad_out, weight


def _case(n_keep=6, T=48, d_out=40, d_in=64, seed=0, dist="normal"):
    W = weight(50 + seed, 0, d_out, d_in)
    x = activation(50 + seed, 0, T, d_in, dist=dist)
    dY = grad_out(50 + seed, 0, T, d_out)
    return W, x, dY, oracle.sparse_bitlinear_step(W, x, dY, n_keep)


@pytest.mark.parametrize("n_keep", [8, 6, 4, 2])
def test_acc_equals_int64_product(n_keep):
    W, x, dY, r = _case(n_keep)
    exact = r["x_q"].astype(np.int64) @ r["w_eff"].astype(np.int64).T     # numpy integer matmul
    assert np.array_equal(r["acc"], exact)


def test_dense_case_is_dense_ternary_gemm():
    W, x, dY, r = _case(8)
    q = oracle.ternary(W, r["gamma"]).astype(np.int64)
    assert np.array_equal(r["acc"], r["x_q"].astype(np.int64) @ q.T)


def _torch_ste(W, x, dY, n_keep):
    """PyTorch float64 autograd of the STE expression, written independently of the oracle's
    backward: x~ = x + (deq(Q_a(x)) - x).detach(), W~ = W + (gamma W_eff - W).detach(),
    y = x~ W~^T, loss = <y, dY>."""
    w_eff, mask, g = oracle.effective_weight(W, n_keep)
    x_q, a = oracle.act_quant(x)
    Wt = torch.tensor(oracle.bf16_to_f64(W), dtype=torch.float64, requires_grad=True)
    xt = torch.tensor(oracle.bf16_to_f64(x), dtype=torch.float64, requires_grad=True)
    deq_x = torch.tensor(x_q.astype(np.float64)) * torch.tensor(a.astype(np.float64))[:, None] / 127.0
    weff = torch.tensor(w_eff.astype(np.float64)) * float(g)
    x_ste = xt + (deq_x - xt).detach()
    W_ste = Wt + (weff - Wt).detach()
    y = x_ste @ W_ste.T
    (y * torch.tensor(oracle.bf16_to_f64(dY))).sum().backward()
    return y.detach().numpy(), xt.grad.numpy(), Wt.grad.numpy()


@pytest.mark.parametrize("n_keep", [6, 4, 2, 8])
def test_forward_and_backward_match_torch_ste(n_keep):
    W, x, dY, r = _case(n_keep, dist="student_t4")
    y, dX, dW = _torch_ste(W, x, dY, n_keep)
    np.testing.assert_allclose(r["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
    np.testing.assert_allclose(r["dX"], dX, rtol=1e-12, atol=1e-12 * np.abs(dX).max())
    np.testing.assert_allclose(r["dW"], dW, rtol=1e-12, atol=1e-12 * np.abs(dW).max())


def test_dual_ste_masked_weights_get_dense_gradient():
    W, x, dY, r = _case(6, T=64)
    mask = r["mask"]
    assert (~mask).sum() > 0
    # masked positions receive a non-zero gradient (the STE test above shows it is the dense one)
    assert np.all(np.abs(r["dW"][~mask]) > 0)
    # the stop-gradient ablation zeroes exactly those positions
    _, dW_sg = oracle.backward_stop_gradient(dY, r["w_eff"], r["gamma"], r["x_q"], r["absmax"], mask)
    assert np.all(dW_sg[~mask] == 0) and np.array_equal(dW_sg[mask], r["dW"][mask])


def test_dx_ignores_masked_weights():
    W, x, dY, r = _case(4, T=16, d_out=24, d_in=32)
    w_eff = r["w_eff"].copy()
    dX1, _ = oracle.backward(dY, w_eff, r["gamma"], r["x_q"], r["absmax"])
    # zeroing an already-masked entry cannot change anything
    w_eff[~r["mask"]] = 0
    dX2, _ = oracle.backward(dY, w_eff, r["gamma"], r["x_q"], r["absmax"])
    assert np.array_equal(dX1, dX2)
    # flipping a kept non-zero code changes exactly one column of dX
    o, i = np.argwhere(r["w_eff"] != 0)[0]
    w_eff[o, i] = -w_eff[o, i]
    dX3, _ = oracle.backward(dY, w_eff, r["gamma"], r["x_q"], r["absmax"])
    changed = np.nonzero(np.any(dX3 != dX1, axis=0))[0]
    assert changed.tolist() == [i]


def test_y_zero_where_acc_zero_and_empty_tokens():
    W, x, dY, r = _case(2)
    assert np.all(r["y"][r["acc"] == 0] == 0)
    empty = oracle.sparse_bitlinear_step(W, x[:0], dY[:0], 6)
    assert empty["y"].shape == (0, W.shape[0]) and empty["dX"].shape == (0, W.shape[1])
    assert np.all(empty["dW"] == 0)
