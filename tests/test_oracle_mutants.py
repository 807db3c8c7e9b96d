"""The pins must catch plausible mistakes: plant each mistake in the oracle (on the
CPU, via monkeypatch) and check that at least one pin test fails on it."""
import math

import numpy as np
import pytest

import oracle
import oracle.sparse_bitlinear as sb

import test_oracle_act as t_act
import test_oracle_gamma as t_gamma
import test_oracle_gemm as t_gemm
import test_oracle_mask as t_mask
import test_oracle_ternary as t_tern
import test_oracle_norm as t_norm
import test_oracle_optimizer as t_opt
import test_oracle_pairs as t_pairs
import test_oracle_sparse24 as t_sp
import test_oracle_variants as t_var


def _ties_to_higher_index(W_bits, n_keep, m=8):
    W = sb.bf16_to_f64(W_bits)
    d_out, d_in = W.shape
    mag = np.abs(W).reshape(d_out, d_in // m, m)[..., ::-1]
    order = np.argsort(-mag, axis=-1, kind="stable")
    keep = np.zeros_like(mag, dtype=bool)
    np.put_along_axis(keep, order[..., :n_keep], True, axis=-1)
    return keep[..., ::-1].reshape(d_out, d_in)


def _ternary_ge(W_bits, gamma):
    W = sb.bf16_to_f64(W_bits)
    return (np.sign(W) * (np.abs(W) >= float(gamma) / 2.0)).astype(np.int8)


def _gamma_after_mask(W_bits, n_keep, m=8):
    mask = sb.nm_mask(W_bits, n_keep, m)
    Wm = np.where(mask, W_bits, np.uint16(0)).astype(np.uint16)
    g = sb.gamma_f32(Wm)
    return (sb.ternary(W_bits, g) * mask).astype(np.int8), mask, g


def _act_quant_128(x_bits):
    x = sb.bf16_to_f64(x_bits)
    a = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0])
    safe = np.where(a > 0, a, 1.0)
    q = np.clip(np.rint(128.0 * x / safe[:, None]), -128, 127)
    q[a == 0] = 0
    return q.astype(np.int8), a.astype(np.float32)


def _act_quant_half_away(x_bits):
    x = sb.bf16_to_f64(x_bits)
    a = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0])
    safe = np.where(a > 0, a, 1.0)
    z = 127.0 * x / safe[:, None]
    q = np.sign(z) * np.floor(np.abs(z) + 0.5)
    q[a == 0] = 0
    return q.astype(np.int8), a.astype(np.float32)


def _backward_no_gamma(dY_bits, w_eff, gamma, x_q, absmax):
    dY = sb.bf16_to_f64(dY_bits)
    return dY @ w_eff.astype(np.float64), dY.T @ sb.dequant_act(x_q, absmax)


def _backward_raw_x(dY_bits, w_eff, gamma, x_q, absmax):
    dY = sb.bf16_to_f64(dY_bits)
    return float(gamma) * (dY @ w_eff.astype(np.float64)), dY.T @ x_q.astype(np.float64)


def _backward_weff_transposed_dw(dY_bits, w_eff, gamma, x_q, absmax):
    dY = sb.bf16_to_f64(dY_bits)
    dW = dY.T @ sb.dequant_act(x_q, absmax)
    return float(gamma) * (dY @ w_eff.astype(np.float64)), dW * (w_eff != 0)


def _forward_y_no_127(acc, gamma, absmax):
    return acc.astype(np.float64) * (float(gamma) * absmax.astype(np.float64)[:, None])


def _qmask_ties_to_higher_index(w_q, n_keep, m=8):
    d_out, d_in = w_q.shape
    key = np.abs(w_q.astype(np.int64)).reshape(d_out, d_in // m, m)[..., ::-1]
    order = np.argsort(-key, axis=-1, kind="stable")
    keep = np.zeros(key.shape, dtype=bool)
    np.put_along_axis(keep, order[..., :n_keep], True, axis=-1)
    return keep[..., ::-1].reshape(d_out, d_in)


def _mask_grad_multiply(dW, mask):
    return dW * mask


_ORIG_EFF = sb.effective_weight


def _effective_weight_ignores_m(W_bits, n_keep, m=8):
    return _ORIG_EFF(W_bits, n_keep, 8)


def _adamw_coupled_decay(W_bits, g, m, v, step, lr, beta1=0.9, beta2=0.95, eps=1e-5, weight_decay=0.1,
                         grad_scale=1.0):
    W = sb.bf16_to_f64(W_bits)
    gs = np.asarray(g, np.float64) * grad_scale + weight_decay * W     # L2 in the gradient, not decoupled
    m1 = beta1 * np.asarray(m, np.float64) + (1 - beta1) * gs
    v1 = beta2 * np.asarray(v, np.float64) + (1 - beta2) * gs * gs
    W1 = W - lr * (m1 / (1 - beta1 ** step)) / (np.sqrt(v1 / (1 - beta2 ** step)) + eps)
    return W1, sb.f64_to_bf16_bits(W1), m1, v1


def _adamw_no_bias_correction(W_bits, g, m, v, step, lr, beta1=0.9, beta2=0.95, eps=1e-5, weight_decay=0.1,
                              grad_scale=1.0):
    W = sb.bf16_to_f64(W_bits)
    gs = np.asarray(g, np.float64) * grad_scale
    m1 = beta1 * np.asarray(m, np.float64) + (1 - beta1) * gs
    v1 = beta2 * np.asarray(v, np.float64) + (1 - beta2) * gs * gs
    W1 = W * (1 - lr * weight_decay) - lr * m1 / (np.sqrt(v1) + eps)
    return W1, sb.f64_to_bf16_bits(W1), m1, v1


def _bf16_via_float32(x):
    from sbl_inputs import f32_to_bf16_bits
    return f32_to_bf16_bits(np.asarray(x, np.float64).astype(np.float32))


_ORIG_RMS = sb.rmsnorm_bf16


def _rmsnorm_sum_not_mean(x_bits, g_bits, eps):
    x = sb.bf16_to_f64(x_bits)
    d = x.shape[1]
    return _ORIG_RMS(x_bits, g_bits, eps * d) if d == 1 else sb.f64_to_bf16_bits(
        x / np.sqrt((x ** 2).sum(axis=1, keepdims=True) + eps) *
        (1.0 if g_bits is None else sb.bf16_to_f64(np.asarray(g_bits))))


def _mean_square_float32_sum(x_bits):
    x = sb.bf16_to_f64(x_bits).astype(np.float32)
    s = np.zeros(x.shape[0], np.float32)
    for j in range(x.shape[1]):
        s = s + x[:, j] * x[:, j]
    return (s / np.float32(x.shape[1])).astype(np.float32)


def _rsqrt_double_rounded(v):
    v32 = np.float32(v)
    if np.isinf(v32):
        return np.float32(0.0)
    return np.float32(np.float32(1.0) / np.sqrt(v32))


def _pack_pairs_digits_swapped(w_eff):
    p = sb.unpack_pairs  # noqa: F841  (the inverse is left as it is)
    w = np.asarray(w_eff, np.int8)
    out = np.zeros((w.shape[0], w.shape[1] // 8), np.uint8)
    digit = {0: 0, 1: 1, -1: 2}
    for o in range(w.shape[0]):
        for g in range(w.shape[1] // 8):
            grp = [int(v) for v in w[o, 8 * g:8 * g + 8]]
            nz = [j for j in range(8) if grp[j]]
            p0, p1 = (nz + [j for j in range(8) if j not in nz])[:2] if len(nz) < 2 else nz
            p0, p1 = min(p0, p1), max(p0, p1)
            out[o, g] = 9 * sb.pair_index(p0, p1) + 3 * digit[grp[p1]] + digit[grp[p0]]
    return out


_ORIG_SP = sb.pack_sparse24


def _sparse24_halves_swapped(w_eff):
    p = _ORIG_SP(w_eff).copy()
    p[..., 0:4], p[..., 4:8] = p[..., 4:8].copy(), p[..., 0:4].copy()
    return p


_ORIG_PACK = sb.pack_codes


def _pack_minus_as_10(w_eff):
    out = _ORIG_PACK(np.where(w_eff == -1, 0, w_eff).astype(np.int8))
    d_out, d_in = w_eff.shape
    neg = (w_eff == -1).reshape(d_out, d_in // 8, 8)
    for j in range(8):
        out |= (neg[..., j].astype(np.uint16) << (2 * j + 1)).astype(np.uint16)
    return out


def _round_ties_up(num, den):
    E = num.bit_length() - den.bit_length()
    if (num << max(0, -E)) < (den << max(0, E)):
        E -= 1
    q_exp = max(E, -126) - 23
    n2, d2 = (num, den << q_exp) if q_exp >= 0 else (num << -q_exp, den)
    q, r = divmod(n2, d2)
    if 2 * r >= d2:
        q += 1
    return math.ldexp(q, q_exp)


MUTANTS = [
    ("mask ties to higher index", "nm_mask", _ties_to_higher_index, [t_mask.test_mask_signed_zero_and_sign_ties]),
    ("ternary tie goes to +-1", "ternary", _ternary_ge, [t_tern.test_ternary_boundary_rows]),
    ("gamma from masked weights", "effective_weight", _gamma_after_mask, [t_tern.test_quant_then_mask_uses_full_matrix_gamma]),
    ("activation scale 128", "act_quant", _act_quant_128, [t_act.test_act_quant_properties]),
    ("activation rounding half away from zero", "act_quant", _act_quant_half_away,
     [lambda: t_act.test_act_quant_exact_rational(1.984375)]),
    ("dX without gamma", "backward", _backward_no_gamma,
     [lambda: t_gemm.test_forward_and_backward_match_torch_ste(6)]),
    ("dW from raw x_q", "backward", _backward_raw_x,
     [lambda: t_gemm.test_forward_and_backward_match_torch_ste(6)]),
    ("dW stop-gradient through the mask", "backward", _backward_weff_transposed_dw,
     [t_gemm.test_dual_ste_masked_weights_get_dense_gradient]),
    ("y without the /127", "forward_y", _forward_y_no_127,
     [lambda: t_gemm.test_forward_and_backward_match_torch_ste(4)]),
    ("-1 packed as 10", "pack_codes", _pack_minus_as_10, [t_tern.test_pack_codes_bit_layout]),
    ("rational rounding ties up", "round_rational_to_f32", _round_ties_up,
     [t_gamma.test_round_rational_matches_numpy_on_exact_doubles]),
    ("quantized-weight mask ties to higher index", "mask_from_quantized", _qmask_ties_to_higher_index,
     [t_var.test_mask_from_quantized_worked_groups]),
    ("masked gradient as dW * M (signed zeros)", "mask_grad", _mask_grad_multiply,
     [t_var.test_mask_grad_zeroes_masked_slots_only]),
    ("N:4 packed as N:8 groups", "effective_weight", _effective_weight_ignores_m,
     [lambda: t_var.test_pack_n_of_4_planes(2)]),
    ("AdamW with coupled weight decay", "adamw_update", _adamw_coupled_decay,
     [lambda: t_opt.test_adamw_matches_torch(2)]),
    ("AdamW without bias correction", "adamw_update", _adamw_no_bias_correction,
     [t_opt.test_adamw_first_step_closed_form]),
    ("bf16 rounding through float32 (double rounding)", "f64_to_bf16_bits", _bf16_via_float32,
     [t_opt.test_bf16_rounding_no_double_rounding]),
    ("RMSNorm with the sum of squares instead of the mean", "rmsnorm_bf16", _rmsnorm_sum_not_mean,
     [lambda: t_norm.test_rmsnorm_within_bf16_rounding_of_float64(64)]),
    ("RMSNorm mean square from a float32 running sum", "mean_square_f32", _mean_square_float32_sum,
     [t_norm.test_mean_square_midpoint_rows]),
    ("RMSNorm reciprocal square root rounded twice", "rsqrt_rn32", _rsqrt_double_rounded,
     [t_norm.test_rsqrt_nearest_by_fractions]),
    ("kept-only plane with the two halves' codes swapped", "pack_sparse24", _sparse24_halves_swapped,
     [t_sp.test_worked_groups]),
    ("pair byte with the two digits swapped", "pack_pairs", _pack_pairs_digits_swapped,
     [t_pairs.test_worked_groups]),
]


@pytest.mark.parametrize("name,attr,fn,tests", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, attr, fn, tests):
    monkeypatch.setattr(sb, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    caught = False
    for t in tests:
        try:
            t()
        except AssertionError:
            caught = True
    assert caught, f"no pin caught the planted mistake: {name}"
