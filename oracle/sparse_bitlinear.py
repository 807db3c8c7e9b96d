"""CPU oracle for the Sparse-BitLinear operator (Sparse-BitNet).

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously-correct
definition of what the operator computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the HIP library and its Python binding) never
calls it and shares no code with it.

Sources (the pages this follows; cited by page and section):

* [SUM]  "Sparse-BitNet：1.58-bit 大模型天然兼容半结构化稀疏 / Sparse-BitNet:
  1.58-bit LLMs are Naturally Friendly to Semi-Structured Sparsity", the
  structured summary of arXiv 2603.05168 at paper.rainbus.top.
  Sections used: 前置知识 (prerequisites) > "1.58-bit BitNet 量化",
  "半结构化 N:M 稀疏", "Straight-Through Estimator (STE)"; 核心方法 (core
  method); 方法步骤详情 (method steps, the Algorithm 1 walk-through).
* [GIST] the gist.science summary of arXiv 2603.05168, section
  "2.2 Sparse-BitNet 框架" (Quant-then-Mask, mask from master weights, Dual STE).
* [EXPL] "什麼是 Sparse-BitNet？核心概念一次搞懂" (openclaw-pages article),
  sections "1.58 位元量化的技術原理" (threshold form of ternary rounding) and
  "N:M 半結構化稀疏性的運作機制" (the worked 2:4 example).

Arithmetic: every bf16 input is decoded exactly to float64.  The mask, the
ternary codes, gamma, the int8 activations and the int32 accumulators are
exact (integers or exactly-rounded values).  y, dX and dW are float64.

Readings of points the pages leave open (each is repeated where it is used):

* gamma is the correctly rounded (nearest-even) binary32 value of the exact
  mean of |W| over the full, unmasked matrix.
* RoundClip(W/gamma, -1, 1) ties go to 0: a weight is non-zero iff
  |w| > gamma/2 (the threshold form on [EXPL]).
* Top-N ties prefer the lower index; magnitude is compared on the bf16 value,
  so +x and -x tie and +0/-0 are both 0.
* Groups are M consecutive positions along d_in.
* Activations: a_t = max_i |x[t,i]|; x_q = round-half-even(127 * x / a_t),
  and a zero row quantizes to zeros.
* Forward scale s = gamma * a_t / 127.
* Backward (Dual STE, identity through quantizers and the mask):
  dX = gamma * dY @ W_eff; dW = dY^T @ x~ with x~ = x_q * a_t / 127, dense over
  every master weight, masked ones included.
* Ablations ([GIST] 4.3 消融实验): "mask from quantized weight" ranks |W_q| in {0, 1}
  with the main mask's tie rule (lower index first); "mask without grad" sets
  the gradient of masked slots to +0.
* N:4 patterns (2:4) use groups of 4 inside the same 8-slot packed words.

Parity pins live in ``tests/test_oracle_*.py``; none of them re-types these
formulas.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

FLT_MAX = float(np.finfo(np.float32).max)

# ----------------------------------------------------------------------------
# bf16 decoding
# ----------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64, exactly.  Asserts finiteness."""
    bits = np.asarray(bits, dtype=np.uint16)
    exp = (bits >> 7) & 0xFF
    assert not np.any(exp == 0xFF), "non-finite bf16 input"
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# gamma = mean |W|        [SUM] 前置知识 > 1.58-bit BitNet 量化:
#                          gamma = ||W||_1 / (d_out * d_in)
# ----------------------------------------------------------------------------

BF16_QUANTUM_LOG2 = -133  # smallest bf16 subnormal is 2^-133


def abs_sum_exact(W_bits: np.ndarray) -> int:
    """Exact sum of |W| as a Python integer in units of 2^-133.

    Every bf16 magnitude is an integer significand times a power of two:
    normal (biased exponent e >= 1): (128 + fraction) * 2^(e - 134);
    subnormal (e = 0): fraction * 2^-133.  Both equal sig * 2^(max(e,1) - 1)
    in units of 2^-133.  Significands are summed per exponent (exactly: the
    per-exponent sums stay far below 2^53) and then combined as big integers.
    """
    b = np.asarray(W_bits, dtype=np.uint16).astype(np.int64) & 0x7FFF
    e = b >> 7
    assert not np.any(e == 0xFF), "non-finite bf16 input"
    frac = b & 0x7F
    sig = np.where(e > 0, frac | 0x80, frac)
    shift = np.maximum(e, 1) - 1
    assert sig.size * 255 < 2 ** 53
    per_exp = np.bincount(shift.ravel(), weights=sig.ravel().astype(np.float64), minlength=255)
    total = 0
    for s, v in enumerate(per_exp):
        if v:
            total += int(v) << s
    return total


def round_rational_to_f32(num: int, den: int) -> float:
    """binary32 value nearest to num/den (ties to even), for num >= 0, den > 0.

    Returned as a Python float holding an exactly representable binary32 value.
    Handles the subnormal range (quantum 2^-149); overflow returns +inf.
    """
    assert num >= 0 and den > 0
    if num == 0:
        return 0.0
    # exponent E with 2^E <= num/den < 2^(E+1)
    E = num.bit_length() - den.bit_length()
    if (num << max(0, -E)) < (den << max(0, E)):
        E -= 1
    q_exp = max(E, -126) - 23          # exponent of one unit in the last place
    if q_exp >= 0:
        n2, d2 = num, den << q_exp
    else:
        n2, d2 = num << (-q_exp), den
    q, r = divmod(n2, d2)
    if 2 * r > d2 or (2 * r == d2 and (q & 1)):
        q += 1
    val = math.ldexp(q, q_exp)
    if val > FLT_MAX:
        return math.inf
    return val


def gamma_f32(W_bits: np.ndarray) -> np.float32:
    """gamma = RN_binary32( sum|W| / (d_out * d_in) ), over the full unmasked W.

    [SUM] 前置知识 > 1.58-bit BitNet 量化 defines gamma as the mean absolute
    value; [SUM] 核心方法 computes quantization and mask side by side on the
    master weight, so gamma never sees the mask.  The pages do not fix the
    arithmetic; the reading taken is the correctly rounded binary32 of the
    exact mean, which does not depend on summation order.
    """
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    n = W_bits.size
    assert n > 0
    S = abs_sum_exact(W_bits)
    return np.float32(round_rational_to_f32(S, n << 133))


# ----------------------------------------------------------------------------
# N:M top-N mask       [SUM] 前置知识 > 半结构化 N:M 稀疏 (||M_group||_0 = N
#                      over every M consecutive positions); [SUM] 核心方法 (i)
#                      M = Pi_{N:M}(|W|) on the continuous master weight;
#                      [GIST] 2.2 (mask from master weights, not ternary ones)
# ----------------------------------------------------------------------------


def nm_mask(W_bits: np.ndarray, n_keep: int, m: int = 8) -> np.ndarray:
    """Boolean keep-mask [d_out, d_in]: in every group of ``m`` consecutive
    d_in positions keep the ``n_keep`` entries of largest |W|.

    Ties: a stable sort by decreasing magnitude, so equal magnitudes keep the
    lower index first.  Exactly ``n_keep`` slots are kept per group.
    """
    W = bf16_to_f64(W_bits)
    d_out, d_in = W.shape
    assert d_in % m == 0 and 1 <= n_keep <= m
    mag = np.abs(W).reshape(d_out, d_in // m, m)
    order = np.argsort(-mag, axis=-1, kind="stable")
    keep = np.zeros_like(mag, dtype=bool)
    np.put_along_axis(keep, order[..., :n_keep], True, axis=-1)
    return keep.reshape(d_out, d_in)


# ----------------------------------------------------------------------------
# Ternary quantization  [SUM] 前置知识 > 1.58-bit BitNet 量化:
#                       W_q = RoundClip(W / gamma, -1, +1);
#                       [EXPL] 1.58 位元量化的技術原理: 0 when |w| <= gamma/2
# ----------------------------------------------------------------------------


def ternary(W_bits: np.ndarray, gamma: float) -> np.ndarray:
    """W_q in {-1, 0, +1} (int8): sign(w) where |w| > gamma/2, else 0.

    This is RoundClip(w/gamma, -1, 1) with the tie |w/gamma| = 1/2 going to 0,
    evaluated as an exact float64 comparison (gamma/2 is exact).  gamma = 0
    (an all-zero matrix) gives all zeros.
    """
    W = bf16_to_f64(W_bits)
    half = float(gamma) / 2.0
    return (np.sign(W) * (np.abs(W) > half)).astype(np.int8)


def effective_weight(W_bits: np.ndarray, n_keep: int, m: int = 8
                     ) -> Tuple[np.ndarray, np.ndarray, np.float32]:
    """Quant-then-mask: W_eff = Q_t(W) * Pi_{N:M}(|W|).  Returns (W_eff int8, mask bool, gamma).

    [SUM] 核心方法 (iii) and 方法步骤详情 steps (2), (4), (5); [GIST] 2.2.
    """
    g = gamma_f32(W_bits)
    mask = nm_mask(W_bits, n_keep, m)
    w_eff = ternary(W_bits, g) * mask.astype(np.int8)
    return w_eff.astype(np.int8), mask, g


# ----------------------------------------------------------------------------
# Packed planes (the library's storage format, M = 8)
# ----------------------------------------------------------------------------

CODE_ZERO, CODE_PLUS, CODE_MINUS = 0b00, 0b01, 0b11


def pack_codes(w_eff: np.ndarray) -> np.ndarray:
    """Code plane uint16 [d_out, d_in/8]: slot j of group g at bits 2j..2j+1;
    00 = 0, 01 = +1, 11 = -1 (10 never occurs)."""
    d_out, d_in = w_eff.shape
    assert d_in % 8 == 0
    c = np.zeros(w_eff.shape, dtype=np.uint16)
    c[w_eff == 1] = CODE_PLUS
    c[w_eff == -1] = CODE_MINUS
    c = c.reshape(d_out, d_in // 8, 8)
    out = np.zeros((d_out, d_in // 8), dtype=np.uint16)
    for j in range(8):
        out |= (c[..., j] << (2 * j)).astype(np.uint16)
    return out


def pack_mask(mask: np.ndarray) -> np.ndarray:
    """Mask plane uint8 [d_out, d_in/8]: bit j set iff slot j of the group is kept."""
    d_out, d_in = mask.shape
    assert d_in % 8 == 0
    k = mask.reshape(d_out, d_in // 8, 8).astype(np.uint8)
    out = np.zeros((d_out, d_in // 8), dtype=np.uint8)
    for j in range(8):
        out |= (k[..., j] << j).astype(np.uint8)
    return out


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_codes``: int8 W_eff [d_out, 8 * groups]."""
    codes = np.asarray(codes, dtype=np.uint16)
    d_out, G = codes.shape
    out = np.zeros((d_out, G, 8), dtype=np.int8)
    for j in range(8):
        f = (codes >> (2 * j)) & 3
        assert not np.any(f == 0b10), "invalid code 10"
        out[..., j] = np.where(f == CODE_PLUS, 1, np.where(f == CODE_MINUS, -1, 0))
    return out.reshape(d_out, G * 8)


def quant_mask_pack(W_bits: np.ndarray, n_keep: int, m: int = 8, from_quantized: bool = False):
    """The packing step as the library exposes it: (codes, mask plane, gamma).

    m is the group size of the mask (8, or 4 for N:4 such as 2:4: two mask
    groups per 8-slot word of the planes).  from_quantized selects the
    ablation mask of ``mask_from_quantized`` instead of Pi_{N:M}(|W|).
    """
    if from_quantized:
        g = gamma_f32(W_bits)
        wq = ternary(W_bits, g)
        mask = mask_from_quantized(wq, n_keep, m)
        w_eff = (wq * mask.astype(np.int8)).astype(np.int8)
    else:
        w_eff, mask, g = effective_weight(W_bits, n_keep, m)
    return pack_codes(w_eff), pack_mask(mask), g


# ----------------------------------------------------------------------------
# Ablations  [SUM] 核心方法 (the two design points the variants remove) and
#            [GIST] 4.3 消融实验: "mask from quantized weight" and "mask without grad"
# ----------------------------------------------------------------------------


def mask_from_quantized(w_q: np.ndarray, n_keep: int, m: int = 8) -> np.ndarray:
    """Ablation mask Pi_{N:M}(|W_q|): top-n_keep of |W_q| in {0, 1} per group of m.

    The pages give no tie rule for this variant, whose keys are nearly all tied
    (they name the ties as the reason it fails); the main mask's rule is used:
    equal keys keep the lower index.  So a group keeps its non-zero slots in
    index order, then zero slots in index order, n_keep in all.
    """
    d_out, d_in = w_q.shape
    assert d_in % m == 0 and 1 <= n_keep <= m
    key = np.abs(w_q.astype(np.int64)).reshape(d_out, d_in // m, m)
    order = np.argsort(-key, axis=-1, kind="stable")
    keep = np.zeros(key.shape, dtype=bool)
    np.put_along_axis(keep, order[..., :n_keep], True, axis=-1)
    return keep.reshape(d_out, d_in)


def mask_grad(dW: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Ablation "mask without grad": the masked slots get no gradient (dW * M)."""
    return np.where(mask, dW, 0.0)


# ----------------------------------------------------------------------------
# Activation quantization  [SUM] 前置知识 > 1.58-bit BitNet 量化 (absmax to
#                          8-bit integers); [SUM] 方法步骤详情 step (3)
# ----------------------------------------------------------------------------


def act_quant(x_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token absmax int8 quantization: (x_q int8 [T, d_in], absmax float32 [T]).

    a_t = max_i |x[t, i]|;  x_q = round-half-even(127 * x / a_t), a zero row
    gives zeros.  The pages name absmax 8-bit quantization but not the
    granularity, range or rounding; the reading is per token, scale 127
    (so -128 never occurs) and ties to even.

    Evaluated in float64: 127*x is exact, and the one rounding of the
    quotient cannot move it across or onto a half-integer (for bf16 x and a_t
    the exact quotient is either a half-integer or at least 2^-17 relative
    away from one), so rint gives the exactly rounded value.  A test checks
    this against exact rational arithmetic.
    """
    x = bf16_to_f64(x_bits)
    assert x.ndim == 2
    a = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0])
    safe = np.where(a > 0, a, 1.0)
    q = np.rint(127.0 * x / safe[:, None])
    q[a == 0] = 0.0
    assert np.all(np.abs(q) <= 127)
    return q.astype(np.int8), a.astype(np.float32)


def dequant_act(x_q: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """x~ = x_q * a_t / 127 in float64 (the activation that enters the product)."""
    return x_q.astype(np.float64) * (absmax.astype(np.float64)[:, None] / 127.0)


# ----------------------------------------------------------------------------
# Forward  [SUM] 前置知识 > 半结构化 N:M 稀疏 (y = (W (.) M) x);
#          [SUM] 方法步骤详情 step (6): y ~= s * W_eff x~, s absorbs the scales
# ----------------------------------------------------------------------------


def forward_acc(w_eff: np.ndarray, x_q: np.ndarray) -> np.ndarray:
    """Exact integer accumulators acc[t, o] = sum_i x_q[t, i] * W_eff[o, i] (int64).

    The product is taken in float64: every term and every partial sum is an
    integer of magnitude <= 127 * d_in < 2^53, so any summation order is exact.
    """
    d_in = x_q.shape[1]
    assert 127 * d_in < 2 ** 53
    acc = x_q.astype(np.float64) @ w_eff.astype(np.float64).T
    out = acc.astype(np.int64)
    assert np.all(np.abs(out) < 2 ** 31)
    return out


def forward_y(acc: np.ndarray, gamma: float, absmax: np.ndarray) -> np.ndarray:
    """y[t, o] = acc[t, o] * gamma * a_t / 127, float64 (gamma, a_t widened exactly)."""
    return acc.astype(np.float64) * (float(gamma) * absmax.astype(np.float64)[:, None] / 127.0)


# ----------------------------------------------------------------------------
# Backward (Dual STE)  [SUM] 前置知识 > Straight-Through Estimator (STE);
#                      [SUM] 核心方法 (dense gradient to every master weight);
#                      [SUM] 方法步骤详情 step (7); [GIST] 2.2
# ----------------------------------------------------------------------------


def backward(dY_bits: np.ndarray, w_eff: np.ndarray, gamma: float,
             x_q: np.ndarray, absmax: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(dX [T, d_in], dW [d_out, d_in]) in float64.

    The straight-through estimator replaces both Q_t and Pi_{N:M} by the
    identity, so the forward y = x~ (gamma W_eff)^T gives
    dX = dY @ (gamma W_eff)   and   dW = dY^T @ x~   for every (o, i),
    including masked positions.  The activation quantizer is also passed
    straight through, so dX is the gradient w.r.t. the layer input.
    """
    dY = bf16_to_f64(dY_bits)
    xt = dequant_act(x_q, absmax)
    dX = float(gamma) * (dY @ w_eff.astype(np.float64))
    dW = dY.T @ xt
    return dX, dW


def backward_stop_gradient(dY_bits, w_eff, gamma, x_q, absmax, mask):
    """Ablation from [SUM] 前置知识 > STE ("mask without grad"): dW multiplied by the mask."""
    dX, dW = backward(dY_bits, w_eff, gamma, x_q, absmax)
    return dX, mask_grad(dW, mask)


# ----------------------------------------------------------------------------
# Kept-only 2:4 operand plane (2:8 and 2:4 patterns)  [SUM] 前置知识 > 半结构化
# N:M 稀疏 (2:4 as the hardware pattern; at most N non-zeros per group)
# ----------------------------------------------------------------------------


def pack_sparse24(w_eff: np.ndarray) -> np.ndarray:
    """Kept-only plane uint8 [d_out, d_in / 64, 16] of a ternary W_eff whose every
    group of 4 consecutive d_in positions holds at most 2 non-zeros (always true
    for 2:8 and 2:4 masks).

    Per row and 64-wide step s, for each half h (positions 64 s + 32 h .. + 31,
    8 groups of 4): a 32-bit word of 16 two-bit codes (00 = 0, 01 = +1, 11 = -1),
    slot 2 g + i being the i-th stored value of group g, and a 32-bit word of
    positions, bits 4 g .. 4 g + 1 and 4 g + 2 .. 4 g + 3 holding the positions
    (0..3, first < second) of those two values in their group.  Stored values:
    the group's non-zeros in position order, padded with zeros at the next free
    positions (one non-zero at a: (a, a + 1), or (2, 3) for a = 3; none: (0, 1)).
    Bytes 0-3: codes of h = 0, 4-7: codes of h = 1, 8-11: positions of h = 0,
    12-15: positions of h = 1 (little endian).  Same size as the code plane.
    """
    w = np.asarray(w_eff, np.int8)
    d_out, d_in = w.shape
    assert d_in % 64 == 0
    out = np.zeros((d_out, d_in // 64, 16), np.uint8)
    code_of = {0: 0, 1: CODE_PLUS, -1: CODE_MINUS}
    for o in range(d_out):
        for st in range(d_in // 64):
            for h in range(2):
                cw = 0
                iw = 0
                for g in range(8):
                    k0 = 64 * st + 32 * h + 4 * g
                    grp = [int(v) for v in w[o, k0:k0 + 4]]
                    nz = [i for i in range(4) if grp[i] != 0]
                    assert len(nz) <= 2, "more than 2 non-zeros in a group of 4"
                    if len(nz) == 2:
                        i0, i1 = nz
                    elif len(nz) == 1:
                        i0, i1 = (nz[0], nz[0] + 1) if nz[0] < 3 else (2, 3)
                    else:
                        i0, i1 = 0, 1
                    cw |= code_of[grp[i0]] << (2 * (2 * g)) | code_of[grp[i1]] << (2 * (2 * g + 1))
                    iw |= (i0 | (i1 << 2)) << (4 * g)
                out[o, st, 4 * h:4 * h + 4] = np.frombuffer(np.uint32(cw).tobytes(), np.uint8)
                out[o, st, 8 + 4 * h:12 + 4 * h] = np.frombuffer(np.uint32(iw).tobytes(), np.uint8)
    return out


def unpack_sparse24(plane: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_sparse24``: int8 W_eff [d_out, 64 * steps]."""
    plane = np.asarray(plane, np.uint8)
    d_out, steps, _ = plane.shape
    w = np.zeros((d_out, steps * 64), np.int8)
    val = {0: 0, CODE_PLUS: 1, CODE_MINUS: -1}
    for o in range(d_out):
        for st in range(steps):
            for h in range(2):
                cw = int(np.frombuffer(plane[o, st, 4 * h:4 * h + 4].tobytes(), np.uint32)[0])
                iw = int(np.frombuffer(plane[o, st, 8 + 4 * h:12 + 4 * h].tobytes(), np.uint32)[0])
                for g in range(8):
                    i0, i1 = (iw >> (4 * g)) & 3, (iw >> (4 * g + 2)) & 3
                    assert i0 < i1, "positions out of order"
                    c0, c1 = (cw >> (4 * g)) & 3, (cw >> (4 * g + 2)) & 3
                    assert c0 != 0b10 and c1 != 0b10, "invalid code 10"
                    k0 = 64 * st + 32 * h + 4 * g
                    w[o, k0 + i0] = val[c0]
                    w[o, k0 + i1] = val[c1]
    return w


# ----------------------------------------------------------------------------
# Pair plane: one byte per group of 8 for masks keeping at most 2 of 8 (2:8,
# 1:8)  [SUM] 前置知识 > 半结构化 N:M 稀疏 (at most N non-zeros per group of M);
# the packed weight format of inference decoding is precomputed once
# ----------------------------------------------------------------------------

PAIR_CODES = 252  # 28 position pairs x 3 x 3 ternary values


def pair_index(p0: int, p1: int) -> int:
    """Rank of the position pair (p0, p1), 0 <= p0 < p1 <= 7, in lexicographic order (0 .. 27)."""
    assert 0 <= p0 < p1 <= 7
    return sum(7 - a for a in range(p0)) + (p1 - p0 - 1)


def pack_pairs(w_eff: np.ndarray) -> np.ndarray:
    """Pair plane uint8 [d_out, d_in / 8] of a ternary W_eff whose every group of 8
    consecutive d_in positions holds at most 2 non-zeros.

    Each group is two stored slots at positions p0 < p1 with ternary values
    v0, v1 (digits 0, 1, 2 for 0, +1, -1), and its byte is
    9 * pair_index(p0, p1) + 3 * digit(v0) + digit(v1), always below 252.
    The stored slots are the group's non-zeros; a group with fewer than two
    pads with zero values at the lowest free positions (one non-zero at a:
    (0, a), or (0, 1) when a = 0; none: (0, 1)), so each group has one byte.
    1 bit per weight: the information content of a 2:8 group (28 x 9 cases
    need log2(252) bits).
    """
    w = np.asarray(w_eff, np.int8)
    d_out, d_in = w.shape
    assert d_in % 8 == 0
    digit = {0: 0, 1: 1, -1: 2}
    out = np.zeros((d_out, d_in // 8), np.uint8)
    for o in range(d_out):
        for g in range(d_in // 8):
            grp = [int(v) for v in w[o, 8 * g:8 * g + 8]]
            nz = [j for j in range(8) if grp[j] != 0]
            assert len(nz) <= 2, "more than 2 non-zeros in a group of 8"
            if len(nz) == 2:
                p0, p1 = nz
            elif len(nz) == 1:
                p0, p1 = (0, 1) if nz[0] == 0 else (0, nz[0])
            else:
                p0, p1 = 0, 1
            out[o, g] = 9 * pair_index(p0, p1) + 3 * digit[grp[p0]] + digit[grp[p1]]
    return out


def unpack_pairs(plane: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_pairs``: int8 W_eff [d_out, 8 * groups]."""
    plane = np.asarray(plane, np.uint8)
    d_out, G = plane.shape
    pairs = [(a, b) for a in range(8) for b in range(a + 1, 8)]
    value = (0, 1, -1)
    w = np.zeros((d_out, 8 * G), np.int8)
    for o in range(d_out):
        for g in range(G):
            b = int(plane[o, g])
            assert b < PAIR_CODES, "pair byte out of range"
            p0, p1 = pairs[b // 9]
            w[o, 8 * g + p0] = value[(b % 9) // 3]
            w[o, 8 * g + p1] = value[b % 3]
    return w


# ----------------------------------------------------------------------------
# Norm + activation quantization  [SUM] 方法步骤详情 step (3): x~ = Q_a(Norm(x))
# ----------------------------------------------------------------------------

BF16_SQUARE_QUANTUM_LOG2 = -266  # (2^-133)^2: every square of a bf16 is a multiple of it


def square_sum_exact(x_bits: np.ndarray) -> list:
    """Exact sum of x^2 over each row, as Python integers in units of 2^-266.

    A bf16 magnitude is sig * 2^(s - 133) with s = max(e, 1) - 1 (see
    ``abs_sum_exact``), so its square is sig^2 * 2^(2 s) units of 2^-266.
    Squared significands are summed per exponent (exact: below 2^53) and then
    combined as big integers.
    """
    b = np.asarray(x_bits, dtype=np.uint16)
    assert b.ndim == 2
    T, d = b.shape
    m = b.astype(np.int64) & 0x7FFF
    e = m >> 7
    assert not np.any(e == 0xFF), "non-finite bf16 input"
    frac = m & 0x7F
    sig = np.where(e > 0, frac | 0x80, frac)
    shift = np.maximum(e, 1) - 1
    assert d * 255 * 255 < 2 ** 53
    rows = np.repeat(np.arange(T, dtype=np.int64), d)
    bins = np.bincount(rows * 254 + shift.ravel(), weights=(sig * sig).ravel().astype(np.float64),
                       minlength=T * 254).reshape(T, 254)
    out = []
    for t in range(T):
        total = 0
        for s_, v in zip(np.flatnonzero(bins[t]), bins[t][bins[t] != 0]):
            total += int(v) << (2 * int(s_))
        out.append(total)
    return out


def mean_square_f32(x_bits: np.ndarray) -> np.ndarray:
    """Per row, the correctly rounded binary32 value of the exact mean of x^2.

    Rounding the exact mean once makes the value independent of any summation
    order, as for gamma; it overflows to +inf only beyond the binary32 range.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, d = x_bits.shape
    assert d > 0
    sums = square_sum_exact(x_bits)
    return np.array([round_rational_to_f32(S, d << -BF16_SQUARE_QUANTUM_LOG2) for S in sums],
                    dtype=np.float32)


def rsqrt_rn32(v) -> np.float32:
    """The binary32 value nearest to 1 / sqrt(v), for a binary32 v > 0 (+inf gives 0).

    Exact integer arithmetic: with 2^E <= 1/sqrt(v) < 2^(E+1), the result is
    round(z) 2^(E - 23) for z = 2^(23 - E) / sqrt(v) in [2^23, 2^24), and
    floor(z) = isqrt(floor(z^2)).  1/sqrt(v) is never a midpoint of the
    binary32 grid (a midpoint's square is not the reciprocal of a dyadic
    rational), so there is no tie; for binary32 v the result is always normal.
    """
    v = float(np.float32(v))
    if math.isinf(v):
        return np.float32(0.0)
    assert v > 0.0
    B, A = v.as_integer_ratio()          # v = B / A, so 1/v = A / B
    E = (A.bit_length() - B.bit_length()) // 2 + 1
    while (A << max(0, -2 * E)) < (B << max(0, 2 * E)):      # 1/v < 4^E
        E -= 1
    while (A << max(0, -2 * (E + 1))) >= (B << max(0, 2 * (E + 1))):  # 1/v >= 4^(E+1)
        E += 1
    k = 46 - 2 * E                        # z^2 = (A / B) 2^k
    num, den = (A << k, B) if k >= 0 else (A, B << -k)
    z = math.isqrt(num // den)
    if 4 * num >= (2 * z + 1) ** 2 * den:
        z += 1
    return np.float32(math.ldexp(z, E - 23))


def rmsnorm_rstd(x_bits: np.ndarray, eps: float) -> np.ndarray:
    """r = RN32(1 / sqrt(RN32(ms + eps))) per row, ms = ``mean_square_f32``; eps a
    binary32 value > 0 (the addition is one binary32 operation)."""
    eps32 = np.float32(eps)
    assert np.isfinite(eps32) and eps32 > 0
    ms = mean_square_f32(x_bits)
    return np.array([rsqrt_rn32(np.float32(m) + eps32) for m in ms], dtype=np.float32)


def rmsnorm_bf16(x_bits: np.ndarray, g_bits, eps: float) -> np.ndarray:
    """RMSNorm of each row, rounded to bf16: y = bf16(RN32(RN32(x r) g)) with
    r = ``rmsnorm_rstd`` (the correctly rounded reciprocal square root of the
    binary32 sum of the exact mean square and eps).

    The pages name Norm(x) but not its kind; RMSNorm with a bf16 weight g (None:
    ones) is the reading (the Qwen2.5 models they train use it), in binary32
    with the output in bf16, the activation dtype of the model.  Since the
    result feeds an integer decision (x_q), every step is one correctly rounded
    operation on exact inputs: the mean square of the row is rounded once from
    its exact value, the same for any order of the sum.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, d = x_bits.shape
    x = bf16_to_f64(x_bits).astype(np.float32)
    gv = np.ones(d, np.float32) if g_bits is None else bf16_to_f64(np.asarray(g_bits)).astype(np.float32)
    r = rmsnorm_rstd(x_bits, eps)
    y = (x * r[:, None]) * gv[None, :]       # two binary32 products per element
    return f64_to_bf16_bits(y.astype(np.float64))


def rmsnorm_act_quant(x_bits: np.ndarray, g_bits, eps: float):
    """Q_a(Norm(x)): (x_q int8, absmax float32) of the bf16 RMSNorm output."""
    return act_quant(rmsnorm_bf16(x_bits, g_bits, eps))


# ----------------------------------------------------------------------------
# Optimizer step + repack  [SUM] 方法步骤详情 step (8) (AdamW updates W; its
#                          hyper-parameters beta = (0.9, 0.95), eps = 1e-5,
#                          weight decay 0.1, grad clip 1.0) and step (2) of the
#                          next step (the mask is recomputed from the new W)
# ----------------------------------------------------------------------------


def adamw_update(W_bits: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, step: int, lr: float,
                 beta1: float = 0.9, beta2: float = 0.95, eps: float = 1e-5, weight_decay: float = 0.1,
                 grad_scale: float = 1.0):
    """One AdamW step on the bf16 master weight, in float64.

    AdamW with decoupled weight decay: the gradient is first multiplied by
    grad_scale (the caller's global-norm clipping factor, min(1, clip / ||g||),
    which spans every parameter of the model and so lies outside the
    operator), then
        m' = beta1 m + (1 - beta1) g,   v' = beta2 v + (1 - beta2) g^2,
        W' = W (1 - lr wd) - lr (m' / (1 - beta1^t)) / (sqrt(v' / (1 - beta2^t)) + eps).
    Returns (W' float64, W' rounded to bf16 bits, m' float64, v' float64).
    The pages fix the hyper-parameters but not the state precision; float32
    states are the reading (the library stores m', v' as float32).
    """
    assert step >= 1
    W = bf16_to_f64(W_bits)
    gs = np.asarray(g, np.float64) * float(grad_scale)
    m1 = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * gs
    v1 = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * gs * gs
    mhat = m1 / (1.0 - beta1 ** step)
    vhat = v1 / (1.0 - beta2 ** step)
    W1 = W * (1.0 - lr * weight_decay) - lr * mhat / (np.sqrt(vhat) + eps)
    return W1, f64_to_bf16_bits(W1), m1, v1


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), as bit patterns.

    Exact: the value is split into its binary64 fields and rounded on the
    integer significand (no intermediate float32 rounding).  Values beyond the
    bf16 range become +-inf; subnormal results round on the subnormal grid.
    """
    x = np.asarray(x, np.float64)
    bits = x.view(np.uint64)
    sign = (bits >> np.uint64(63)).astype(np.uint64)
    e = ((bits >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    frac = (bits & np.uint64((1 << 52) - 1)).astype(np.uint64)
    out = np.zeros(x.shape, np.uint64)
    for idx in np.ndindex(x.shape):
        ei, fi = int(e[idx]), int(frac[idx])
        if ei == 0 and fi == 0:
            out[idx] = 0
            continue
        assert ei != 0x7FF, "non-finite value"
        # value = sig * 2^(exp2) with sig an integer of 53 bits (normal binary64)
        sig = (fi | (1 << 52)) if ei else fi
        exp2 = (ei if ei else 1) - 1075
        # bf16 normal: 8-bit significand, exponent field 1..254; grid 2^(E - 7)
        top = sig.bit_length() - 1 + exp2           # floor(log2 |x|)
        q = max(top, -126) - 7                       # grid exponent (subnormals: 2^-133)
        shift = q - exp2
        if shift <= 0:
            r = sig << (-shift)
        else:
            r, rem = sig >> shift, sig & ((1 << shift) - 1)
            half = 1 << (shift - 1)
            if rem > half or (rem == half and (r & 1)):
                r += 1
        # r * 2^q with r <= 256; a carry to 256 moves to the next binade
        if r == 256:
            r, q = 128, q + 1
        if r == 0:
            b = 0
        else:
            top_r = r.bit_length() - 1 + q
            if top_r > 127:
                b = 0x7F80                           # overflow to infinity
            elif top_r < -126:
                b = r << (q + 133)                   # subnormal: 2^-133 units
            else:                                    # r has 8 bits: hidden one + 7-bit mantissa
                b = ((top_r + 127) << 7) | (r & 0x7F)
        out[idx] = b
    return (out | (sign << np.uint64(15))).astype(np.uint16)


def mask_flips(mask_prev: np.ndarray, mask_new: np.ndarray) -> int:
    """Mask flip count: slots whose keep bit changed between two steps (the
    training diagnostic of [SUM] 核心方法, masks recomputed every step)."""
    return int(np.count_nonzero(np.asarray(mask_prev, bool) != np.asarray(mask_new, bool)))


def adamw_repack(W_bits, g, m, v, step, lr, n_keep, m_group=8, mask_prev=None, **hp):
    """Optimizer step followed by the next step's packing: (W' bf16 bits, m', v', codes, mask plane,
    gamma, flips or None)."""
    _, W1_bits, m1, v1 = adamw_update(W_bits, g, m, v, step, lr, **hp)
    codes, mplane, gam = quant_mask_pack(W1_bits, n_keep, m_group)
    flips = None
    if mask_prev is not None:
        flips = mask_flips(unpack_mask(mask_prev), unpack_mask(mplane))
    return W1_bits, m1, v1, codes, mplane, gam, flips


def unpack_mask(mplane: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_mask``: bool [d_out, 8 * groups]."""
    mplane = np.asarray(mplane, np.uint8)
    d_out, G = mplane.shape
    out = np.zeros((d_out, G, 8), bool)
    for j in range(8):
        out[..., j] = (mplane >> j) & 1
    return out.reshape(d_out, G * 8)


# ----------------------------------------------------------------------------
# Whole step
# ----------------------------------------------------------------------------


def sparse_bitlinear_step(W_bits, x_bits, dY_bits, n_keep: int):
    """One forward + backward pass of a Sparse-BitLinear layer.  Returns a dict."""
    w_eff, mask, g = effective_weight(W_bits, n_keep, 8)
    x_q, a = act_quant(x_bits)
    acc = forward_acc(w_eff, x_q)
    y = forward_y(acc, g, a)
    out = dict(gamma=g, mask=mask, w_eff=w_eff, codes=pack_codes(w_eff), mask_plane=pack_mask(mask),
               x_q=x_q, absmax=a, acc=acc, y=y)
    if dY_bits is not None:
        dX, dW = backward(dY_bits, w_eff, g, x_q, a)
        out.update(dX=dX, dW=dW)
    return out
