"""Pins for the oracle's optimizer step + repack (the reading of [SUM]
方法步骤详情 step (8) with the optimizer's hyper-parameters): AdamW against torch.optim.AdamW in float64 (a library
routine), its closed form at the first step, the exact float64 -> bf16 rounding
against the float32 route and hand-derived double-rounding cases, and the flip
count against a loop."""
import numpy as np
import pytest
import torch

import oracle
from sbl_inputs import f32_to_bf16_bits, weight


def test_bf16_rounding_matches_float32_route_on_float32_values():
    g = np.random.default_rng(3)
    x = np.concatenate([g.standard_normal(4000) * 10.0 ** g.integers(-40, 38, 4000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.39e38, 2.0 ** -133, 2.0 ** -126])])
    x = x.astype(np.float32)
    x = x[np.isfinite(x)]
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(x.astype(np.float64)), f32_to_bf16_bits(x))


def test_bf16_rounding_no_double_rounding():
    # worked by hand: 1 + 2^-8 is the tie between 1.0 (0x3f80) and 1.0078125 (0x3f81);
    # a hair above it must round up, a hair below down (a float32 step first would tie to even)
    cases = [(1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81), (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),
             (1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82), (-(2.0 + 2.0 ** -7 + 2.0 ** -45), 0xC001),
             (2.0 ** -133 * 0.5 + 2.0 ** -160, 0x0001), (2.0 ** -133 * 0.5, 0x0000), (3.4e38, 0x7F80)]
    for x, want in cases:
        assert int(oracle.f64_to_bf16_bits(np.array([x]))[0]) == want, (x, hex(want))


def _torch_adamw(W64, g, m, v, step, lr, beta1, beta2, eps, wd):
    p = torch.nn.Parameter(torch.from_numpy(W64.copy()))
    opt = torch.optim.AdamW([p], lr=lr, betas=(beta1, beta2), eps=eps, weight_decay=wd)
    p.grad = torch.from_numpy(g.copy())
    opt.step()  # initialises the state with step 1
    st = opt.state[p]
    if step > 1 or np.any(m) or np.any(v):
        # redo the step from the given state
        with torch.no_grad():
            p.copy_(torch.from_numpy(W64))
        st["exp_avg"].copy_(torch.from_numpy(m.astype(np.float64)))
        st["exp_avg_sq"].copy_(torch.from_numpy(v.astype(np.float64)))
        st["step"].fill_(step - 1)
        opt.step()
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("step", [1, 2, 50])
def test_adamw_matches_torch(step):
    g_ = np.random.default_rng(step)
    W = weight(41, step, 24, 40)
    grad = g_.standard_normal(W.shape) * 1e-3
    m = g_.standard_normal(W.shape) * 1e-4 if step > 1 else np.zeros(W.shape)
    v = g_.random(W.shape) * 1e-6 if step > 1 else np.zeros(W.shape)
    hp = dict(beta1=0.9, beta2=0.95, eps=1e-5, weight_decay=0.1)
    W1, W1_bits, m1, v1 = oracle.adamw_update(W, grad, m, v, step, 3e-4, **hp)
    tW, tm, tv = _torch_adamw(oracle.bf16_to_f64(W), grad, m, v, step, 3e-4, 0.9, 0.95, 1e-5, 0.1)
    np.testing.assert_allclose(W1, tW, rtol=1e-13, atol=1e-18)
    np.testing.assert_allclose(m1, tm, rtol=1e-13, atol=1e-20)
    np.testing.assert_allclose(v1, tv, rtol=1e-13, atol=1e-24)
    np.testing.assert_array_equal(W1_bits, oracle.f64_to_bf16_bits(W1))


def test_adamw_first_step_closed_form():
    # from zero state the bias-corrected moments are g and g^2, so the step is
    # lr * g / (|g| + eps) on top of the decay; with grad_scale the same for s * g
    W = weight(42, 0, 16, 32)
    grad = np.random.default_rng(9).standard_normal(W.shape)
    z = np.zeros(W.shape)
    lr, wd, eps, s = 1e-2, 0.1, 1e-5, 0.25
    W1, _, m1, v1 = oracle.adamw_update(W, grad, z, z, 1, lr, eps=eps, weight_decay=wd, grad_scale=s)
    gs = s * grad
    want = oracle.bf16_to_f64(W) * (1 - lr * wd) - lr * gs / (np.abs(gs) + eps)
    np.testing.assert_allclose(W1, want, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m1, 0.1 * gs, rtol=1e-12)
    np.testing.assert_allclose(v1, 0.05 * gs * gs, rtol=1e-12)


def test_mask_flips_and_repack_composition():
    W = weight(43, 1, 32, 64)
    g_ = np.random.default_rng(4)
    grad = g_.standard_normal(W.shape) * 0.05
    z = np.zeros(W.shape)
    _, mprev, _ = oracle.quant_mask_pack(W, 6)
    W1, m1, v1, codes, mplane, gam, flips = oracle.adamw_repack(W, grad, z, z, 1, 1e-2, 6, mask_prev=mprev)
    c2, m2, g2 = oracle.quant_mask_pack(W1, 6)
    assert np.array_equal(codes, c2) and np.array_equal(mplane, m2) and gam == g2
    a, b = oracle.unpack_mask(mprev), oracle.unpack_mask(mplane)
    loop = sum(1 for i in range(a.shape[0]) for j in range(a.shape[1]) if a[i, j] != b[i, j])
    assert flips == loop and flips > 0
    assert np.array_equal(oracle.pack_mask(oracle.unpack_mask(mplane)), mplane)
