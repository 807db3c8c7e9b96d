"""GPU parity of every step against the CPU oracle, on seeded inputs.

Bit-exact: gamma bits, code plane, mask plane, x_q, absmax bits, int32
accumulators.  Float: y within 1e-5 relative; dX and dW within 2e-2 of the
float64 oracle (per-row L2 and elementwise against max|ref|).
"""
import numpy as np
import pytest
import torch

import oracle
from sbl_inputs import (activation, boundary_row_weight, f32_to_bf16_bits, grad_out, sample_rows,
                        tie_heavy_weight, weight)

from gpu_util import (ERR_MODEL_BF16, ERR_MODEL_F32, assert_grad_close, assert_y_close, bf16_to_f64, bits16,
                      f32_bits, to_dev_bf16)

pytestmark = pytest.mark.gpu

try:
    import sparsity_sparse_bitlinear_amd as sbl
except ImportError:
    if torch.cuda.is_available():  # a GPU without the library is a failure, not a skip
        raise
    pytest.skip("no GPU and no libsbl.so", allow_module_level=True)


def gpu_pack(W_bits, n):
    codes, mask, gamma = sbl.quant_mask_pack(to_dev_bf16(W_bits), n)
    torch.cuda.synchronize()
    return bits16(codes), mask.cpu().numpy(), gamma.cpu().numpy()[0]


def check_pack(W_bits, n):
    codes, mask, g = gpu_pack(W_bits, n)
    rc, rm, rg = oracle.quant_mask_pack(W_bits, n)
    assert f32_bits(g) == f32_bits(rg), (float(g), float(rg))
    np.testing.assert_array_equal(mask, rm)
    np.testing.assert_array_equal(codes, rc)


# ---------------------------------------------------------------------------
# quant / mask / pack
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [2, 4, 6, 8])
@pytest.mark.parametrize("shape", [(256, 256), (1, 8), (3, 24), (40, 64), (333, 72), (517, 1032)])
def test_pack_parity_gaussian(shape, n):
    check_pack(weight(11, shape[0] * 7 + shape[1], *shape), n)


@pytest.mark.parametrize("n", [2, 4, 6, 8])
def test_pack_parity_tie_heavy(n):
    check_pack(tie_heavy_weight(1, 96, 256), n)
    check_pack(tie_heavy_weight(2, 64, 64, alphabet=(-1, 1), scale=0.5), n)


# N:M variants and the mask-from-quantized-weight ablation: every N of N:8,
# N:4 (2:4) inside the 8-slot planes, bit-exact planes and gamma.
def check_pack_nm(W_bits, n, m, fq):
    codes, mask, gamma = sbl.quant_mask_pack(to_dev_bf16(W_bits), n, m=m, from_quantized=fq)
    torch.cuda.synchronize()
    rc, rm, rg = oracle.quant_mask_pack(W_bits, n, m, from_quantized=fq)
    assert f32_bits(gamma.cpu().numpy()[0]) == f32_bits(rg)
    np.testing.assert_array_equal(mask.cpu().numpy(), rm)
    np.testing.assert_array_equal(bits16(codes), rc)


@pytest.mark.parametrize("fq", [False, True])
@pytest.mark.parametrize("n,m", [(n, 8) for n in range(1, 9)] + [(n, 4) for n in range(1, 5)])
def test_pack_parity_nm_patterns(n, m, fq):
    check_pack_nm(weight(13, 10 * n + m, 333, 1032), n, m, fq)
    check_pack_nm(tie_heavy_weight(3, 64, 128), n, m, fq)
    check_pack_nm(boundary_row_weight(24, 64), n, m, fq)


@pytest.mark.parametrize("n,m,fq", [(6, 8, False), (2, 4, False), (6, 8, True), (8, 8, False)])
def test_pack_batch_matches_single_calls(n, m, fq):
    # one batched call over a layer's worth of shapes (tiny, ragged, large) equals the single calls
    shapes = [(256, 2048), (1, 8), (333, 1032), (11008, 2048), (3, 24), (2048, 11008), (40, 64)]
    Ws = [to_dev_bf16(weight(17, i, d_o, d_i)) for i, (d_o, d_i) in enumerate(shapes)]
    Ws[4] = to_dev_bf16(tie_heavy_weight(5, 3, 24))
    cb, mb, gb = sbl.quant_mask_pack_batch(Ws, n, m=m, from_quantized=fq)
    for i, W in enumerate(Ws):
        c1, m1, g1 = sbl.quant_mask_pack(W, n, m=m, from_quantized=fq)
        torch.cuda.synchronize()
        assert torch.equal(cb[i], c1) and torch.equal(mb[i], m1), i
        assert f32_bits(gb[i].cpu().numpy()[0]) == f32_bits(g1.cpu().numpy()[0]), i
    # and the small ones against the oracle
    for i in (0, 1, 2, 4, 6):
        rc, rm, rg = oracle.quant_mask_pack(bits16(Ws[i]), n, m, from_quantized=fq)
        np.testing.assert_array_equal(bits16(cb[i]), rc)
        np.testing.assert_array_equal(mb[i].cpu().numpy(), rm)
        assert f32_bits(gb[i].cpu().numpy()[0]) == f32_bits(rg)


def test_pack_graph_capture_matches_eager():
    # the packing (three kernels, no memset) captured in a HIP graph: every replay, with
    # eager work between the replays, equals the eager result bit for bit, single and batched
    shapes = [(1000, 1032), (11008, 2048), (3, 24)]
    Ws = [to_dev_bf16(weight(19, i, d_o, d_i)) for i, (d_o, d_i) in enumerate(shapes)]
    want = [sbl.quant_mask_pack(W, 6) for W in Ws]
    torch.cuda.synchronize()
    one = [torch.empty_like(t) for t in want[0]]
    bat = [[torch.empty_like(t) for t in w] for w in want]
    ws1 = torch.empty((sbl.quant_workspace_size(*shapes[0]),), dtype=torch.uint8, device="cuda")
    wsb = torch.empty((sbl.quant_batch_workspace_size(shapes),), dtype=torch.uint8, device="cuda")

    def run():
        sbl.quant_mask_pack(Ws[0], 6, codes=one[0], mask=one[1], gamma=one[2], workspace=ws1)
        sbl.quant_mask_pack_batch(Ws, 6, codes=[b[0] for b in bat], masks=[b[1] for b in bat],
                                  gammas=[b[2] for b in bat], workspace=wsb)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        for t in one + [t for b in bat for t in b]:
            t.zero_()
        other = sbl.quant_mask_pack(Ws[2], 2)           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in [(one, want[0])] + list(zip(bat, want)):
            assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), f"replay {i}"
            assert torch.equal(got[2].view(torch.int32), ref[2].view(torch.int32)), f"replay {i}"
        assert other[0].shape == (3, 3)


# Kept-only 2:4 plane and the forward on the sparse matrix instruction: the
# plane bit-exact against the oracle, and the int32 sums (so every output)
# identical to the dense path's.  (4096, 4096, 128) is a grid of 256 blocks of
# 256 x 256 (the 8-wave kernel); the smaller grids run the 4-wave one.
@pytest.mark.parametrize("n,m", [(2, 8), (2, 4), (1, 4)])
@pytest.mark.parametrize("T,d_out,d_in", [(300, 200, 256), (77, 1000, 1152), (513, 256, 2048), (33, 40, 11008),
                                          (4096, 4096, 128)])
def test_sparse24_parity(T, d_out, d_in, n, m):
    W = weight(67, n + m + d_in, d_out, d_in)
    x = activation(67, d_out + T, T, d_in, dist="student_t4")
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), n, m=m)
    plane, bad = sbl.pack_sparse24(codes)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    w_eff, _, _ = oracle.effective_weight(W, n, m)
    if d_out * d_in <= 300_000:
        np.testing.assert_array_equal(plane.cpu().numpy(), oracle.pack_sparse24(w_eff))
    xq, a = sbl.act_quant(to_dev_bf16(x))
    for dt in (sbl.I32, sbl.F32, sbl.BF16):
        y_d = sbl.forward(codes, gamma, xq, a, out_dtype=dt)
        y_s = sbl.forward_sparse24(plane, gamma, xq, a, out_dtype=dt)
        torch.cuda.synchronize()
        view = torch.int16 if dt == sbl.BF16 else torch.int32
        assert torch.equal(y_s.view(view), y_d.view(view)), dt
    acc_ref = oracle.forward_acc(w_eff, oracle.act_quant(x)[0])
    np.testing.assert_array_equal(sbl.forward_sparse24(plane, gamma, xq, a, out_dtype=sbl.I32).cpu().numpy(), acc_ref)


def test_sparse24_counts_unrepresentable_groups():
    # a 6:8 code plane has groups of 4 with 3 or 4 non-zeros; their count is reported
    W = weight(68, 0, 64, 256)
    codes, _, _ = sbl.quant_mask_pack(to_dev_bf16(W), 6)
    _, bad = sbl.pack_sparse24(codes)
    torch.cuda.synchronize()
    w_eff = oracle.unpack_codes(bits16(codes))
    want = int(np.count_nonzero(np.count_nonzero(w_eff.reshape(64, -1, 4), axis=-1) > 2))
    assert want > 0 and int(bad.item()) == want


@pytest.mark.parametrize("n,m", [(3, 8), (5, 8), (7, 8), (2, 4), (1, 4)])
def test_step_parity_nm_patterns(n, m):
    # the forward and backward kernels take the planes of any pattern as they are
    T, d_out, d_in = 77, 200, 328
    W = weight(53, n + m, d_out, d_in)
    x = activation(53, n + m + 1, T, d_in, dist="student_t4")
    dY = grad_out(53, n + m + 2, T, d_out)
    w_eff, mask, g = oracle.effective_weight(W, n, m)
    xq_r, a_r = oracle.act_quant(x)
    acc_ref = oracle.forward_acc(w_eff, xq_r)
    dX_r, dW_r = oracle.backward(dY, w_eff, g, xq_r, a_r)
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), n, m=m)
    xq, a = sbl.act_quant(to_dev_bf16(x))
    acc = sbl.forward(codes, gamma, xq, a, out_dtype=sbl.I32)
    dX, dW = sbl.backward(codes, gamma, xq, a, to_dev_bf16(dY))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    assert_grad_close(bf16_to_f64(dX), dX_r)
    assert_grad_close(dW.cpu().numpy(), dW_r)
    assert_grad_close(bf16_to_f64(dX), dX_r, tol=ERR_MODEL_BF16)
    assert_grad_close(dW.cpu().numpy(), dW_r, tol=ERR_MODEL_BF16)


@pytest.mark.parametrize("d_out,d_in", [(200, 328), (11008, 2048)])
def test_mask_grad_parity(d_out, d_in):
    # mask-without-grad ablation: masked slots +0, kept slots bit for bit, and the
    # result against the oracle's stop-gradient backward
    T = 64
    W = weight(57, d_out, d_out, d_in)
    x = activation(57, d_in, T, d_in, dist="student_t4")
    dY = grad_out(57, T, T, d_out)
    codes, mask, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6)
    xq, a = sbl.act_quant(to_dev_bf16(x))
    _, dW = sbl.backward(codes, gamma, xq, a, to_dev_bf16(dY))
    full = dW.clone()
    sbl.mask_grad(dW, mask)
    torch.cuda.synchronize()
    keep = oracle.nm_mask(W, 6)
    got = dW.cpu().numpy()
    np.testing.assert_array_equal(got.view(np.int32), oracle.mask_grad(full.cpu().numpy(), keep).view(np.int32))
    if d_out <= 256:
        r = oracle.sparse_bitlinear_step(W, x, dY, 6)
        _, dW_sg = oracle.backward_stop_gradient(dY, r["w_eff"], r["gamma"], r["x_q"], r["absmax"], r["mask"])
        assert_grad_close(got, dW_sg)


# Optimizer step + repack (AdamW on the bf16 master weight, then the next
# step's gamma, mask, codes and the mask flip count).  W' within one bf16 step
# of the float64 oracle (the kernel computes in float32), m' and v' to float32
# accuracy; the packing of the W' the kernel wrote is bit-exact.
@pytest.mark.parametrize("step", [1, 7])
@pytest.mark.parametrize("n,m_group,d_out,d_in", [(6, 8, 200, 328), (2, 4, 333, 1032), (6, 8, 2048, 2048)])
def test_adamw_repack_parity(step, n, m_group, d_out, d_in):
    W = weight(81, step + d_in, d_out, d_in)
    g_ = np.random.default_rng(step + d_out)
    grad = (g_.standard_normal(W.shape) * 1e-3).astype(np.float32)
    m0 = (g_.standard_normal(W.shape) * 1e-4).astype(np.float32) if step > 1 else np.zeros(W.shape, np.float32)
    v0 = (g_.random(W.shape) * 1e-6).astype(np.float32) if step > 1 else np.zeros(W.shape, np.float32)
    hp = dict(beta1=0.9, beta2=0.95, eps=1e-5, weight_decay=0.1, grad_scale=0.5)
    lr = 2e-3
    Wd = to_dev_bf16(W)
    _, mprev, _ = sbl.quant_mask_pack(Wd, n, m=m_group)
    md, vd = torch.from_numpy(m0).cuda(), torch.from_numpy(v0).cuda()
    codes, mask, gamma, flips = sbl.adamw_repack(Wd, torch.from_numpy(grad).cuda(), md, vd, step=step, lr=lr,
                                                 n_keep=n, m_group=m_group, mask_prev=mprev, **hp)
    torch.cuda.synchronize()
    W1_ref, _, m1_ref, v1_ref = oracle.adamw_update(W, grad, m0, v0, step, lr, **hp)
    W1 = oracle.bf16_to_f64(bits16(Wd))
    # within one bf16 step of the exact value, plus the float32 error of the two terms
    # (where they cancel near zero the float32 error exceeds a bf16 step), and nearly
    # always the nearest bf16 value
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(W1_ref), 2.0 ** -126))).astype(int) - 7)
    W0 = oracle.bf16_to_f64(W)
    decayed = W0 * (1 - lr * hp["weight_decay"])
    terms = np.abs(decayed) + np.abs(W1_ref - decayed)
    assert np.all(np.abs(W1 - W1_ref) < ulp + 2.0 ** -21 * terms)
    exact = bits16(Wd) == oracle.f64_to_bf16_bits(W1_ref)
    assert exact.mean() > 0.999, exact.mean()
    # float32 error bound of a two-term update, relative to its terms (they may cancel)
    gs = grad.astype(np.float64) * hp["grad_scale"]
    m_terms = 0.9 * np.abs(m0) + 0.1 * np.abs(gs)
    v_terms = 0.95 * np.abs(v0) + 0.05 * gs * gs
    assert np.all(np.abs(md.cpu().numpy() - m1_ref) <= 2.0 ** -21 * m_terms + 1e-30)
    assert np.all(np.abs(vd.cpu().numpy() - v1_ref) <= 2.0 ** -21 * v_terms + 1e-30)
    rc, rm, rg = oracle.quant_mask_pack(bits16(Wd), n, m_group)
    assert f32_bits(gamma.cpu().numpy()[0]) == f32_bits(rg)
    np.testing.assert_array_equal(mask.cpu().numpy(), rm)
    np.testing.assert_array_equal(bits16(codes), rc)
    want_flips = oracle.mask_flips(oracle.unpack_mask(mprev.cpu().numpy()), oracle.unpack_mask(rm))
    assert int(flips.item()) == want_flips


def test_adamw_repack_in_place_mask_and_no_flips():
    # mask_prev == mask (in place), and without mask_prev no flip count
    W = weight(82, 0, 64, 256)
    grad = torch.from_numpy((np.random.default_rng(1).standard_normal(W.shape) * 1e-2).astype(np.float32)).cuda()
    Wa, Wb = to_dev_bf16(W), to_dev_bf16(W)
    _, mk, _ = sbl.quant_mask_pack(Wa, 6)
    prev = mk.clone()
    ma, va = torch.zeros(W.shape, device="cuda"), torch.zeros(W.shape, device="cuda")
    mb, vb = torch.zeros(W.shape, device="cuda"), torch.zeros(W.shape, device="cuda")
    ca, _, ga, fa = sbl.adamw_repack(Wa, grad, ma, va, step=1, lr=1e-2, mask_prev=mk, mask=mk)
    cb, mkb, gb, fb = sbl.adamw_repack(Wb, grad, mb, vb, step=1, lr=1e-2)
    torch.cuda.synchronize()
    assert fb is None
    assert torch.equal(ca, cb) and torch.equal(mk, mkb) and torch.equal(ga, gb)
    assert int(fa.item()) == oracle.mask_flips(oracle.unpack_mask(prev.cpu().numpy()),
                                               oracle.unpack_mask(mkb.cpu().numpy()))


def test_pack_boundary_rows():
    W = boundary_row_weight(24, 64)     # gamma = 1 exactly; |w| = 0.5 sits on the threshold
    check_pack(W, 8)
    check_pack(W, 6)


def test_pack_all_zero_and_signed_zero():
    W = np.zeros((16, 64), np.uint16)
    W[::2, 1::3] = 0x8000
    check_pack(W, 6)
    check_pack(W, 8)


def test_pack_extreme_magnitudes():
    # huge (>= 1024) and tiny (< 2^-47) values and bf16 subnormals take the exact
    # per-exponent path of the gamma reduction
    g = np.random.default_rng(5)
    base = g.standard_normal((64, 256)).astype(np.float32) * 0.02
    base[g.random(base.shape) < 0.01] *= 1e30
    base[g.random(base.shape) < 0.01] *= 1e-30
    W = f32_to_bf16_bits(base)
    sub = g.random(W.shape) < 0.01
    W[sub] = g.integers(1, 0x80, size=int(sub.sum())).astype(np.uint16)  # bf16 subnormals
    for n in (2, 6, 8):
        check_pack(W, n)
    tiny = f32_to_bf16_bits(np.full((8, 64), 3e-38, np.float32))      # gamma in the subnormal-adjacent range
    check_pack(tiny, 6)
    maxv = np.full((4, 64), 0x7F7F, np.uint16)                          # largest finite bf16
    check_pack(maxv, 6)


def test_pack_large_matrix():
    check_pack(weight(3, 4, 11008, 2048), 6)


# ---------------------------------------------------------------------------
# activation quantization
# ---------------------------------------------------------------------------

def check_act(x_bits):
    xq, a = sbl.act_quant(to_dev_bf16(x_bits))
    torch.cuda.synchronize()
    rq, ra = oracle.act_quant(x_bits)
    np.testing.assert_array_equal(f32_bits(a.cpu().numpy()), f32_bits(ra))
    np.testing.assert_array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize("shape,dist,outl", [((64, 256), "normal", 0.0), ((513, 896), "normal", 0.001),
                                             ((7, 8), "normal", 0.0), ((3, 11008), "student_t4", 0.0),
                                             ((300, 2048), "student_t4", 0.0), ((5, 16392), "normal", 0.0),
                                             ((2, 40008), "normal", 0.0)])
def test_act_parity(shape, dist, outl):
    check_act(activation(21, shape[1], *shape, dist=dist, outlier_frac=outl))


# Q_a(Norm(x)) fused: bit-exact x_q, absmax and rstd against the oracle's
# RMSNorm (the exact mean square rounded once, a correctly rounded reciprocal
# square root) followed by the exact act quant.
def check_rmsnorm(x, g, eps):
    xq, a, r = sbl.rmsnorm_act_quant(to_dev_bf16(x), to_dev_bf16(g) if g is not None else None, eps,
                                     with_rstd=True)
    torch.cuda.synchronize()
    rq, ra = oracle.rmsnorm_act_quant(x, g, eps)
    np.testing.assert_array_equal(r.cpu().numpy().view(np.uint32), oracle.rmsnorm_rstd(x, eps).view(np.uint32))
    np.testing.assert_array_equal(a.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    np.testing.assert_array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize("with_g", [False, True])
@pytest.mark.parametrize("T,d_in", [(64, 2048), (33, 11008), (7, 64), (5, 4104), (2, 16384), (300, 896),
                                    (6, 4096), (3, 8)])
def test_rmsnorm_act_quant_parity(T, d_in, with_g):
    x = activation(91, d_in + T, T, d_in, dist="student_t4", outlier_frac=0.001)
    g = f32_to_bf16_bits(np.random.default_rng(d_in).uniform(0.25, 2.0, d_in).astype(np.float32)) if with_g else None
    x[0] = 0  # a zero row
    check_rmsnorm(x, g, 1e-6)


def _midpoint_rows(d, n, seed):
    """Rows whose mean square is exactly the binary32 midpoint 3/4 + 2^-25 (the
    8-element pattern 1 x 6, 2^-11, 0 tiled over the row, in a shuffled order,
    scaled by 4^k), and the same rows with a 2^-100 in one zero slot (just above
    the midpoint)."""
    rng = np.random.default_rng(seed)
    base = np.tile(np.array([1.0] * 6 + [2.0 ** -11, 0.0], np.float64), d // 8)
    rows = []
    for i in range(n):
        r = base.copy()
        if i % 2:
            r[7] = 2.0 ** -100
        r = r[rng.permutation(d)] * 4.0 ** int(rng.integers(-20, 20))
        rows.append(r * rng.choice([-1.0, 1.0], size=d))
    return f32_to_bf16_bits(np.array(rows, np.float32))


@pytest.mark.parametrize("d_in", [8, 64, 2048, 4096, 8192, 11008])
def test_rmsnorm_exact_path_rows(d_in):
    """Rows at (and just past) a rounding tie of the mean square, which the
    float64 estimate cannot decide; subnormal, mixed-range and overflowing rows."""
    x = _midpoint_rows(d_in, 8, d_in)
    g = np.random.default_rng(5)
    extra = np.zeros((4, d_in), np.uint16)
    extra[0] = 0x0001                                      # all smallest subnormals
    extra[1, ::3] = 0x0075                                 # subnormals and zeros
    extra[2] = f32_to_bf16_bits((np.exp2(g.uniform(-130, 60, d_in)) *
                                 g.choice([-1, 1], d_in)).astype(np.float32))
    extra[3] = 0x7F7F                                      # largest bf16: the mean square overflows
    check_rmsnorm(np.concatenate([x, extra]), None, 2.0 ** -149)
    check_rmsnorm(x, None, 1e-6)


def test_act_edge_rows():
    g = np.random.default_rng(9)
    x = f32_to_bf16_bits(g.standard_normal((8, 136)).astype(np.float32))
    x[0] = 0                                   # zero row
    x[1] = 0x8000                              # -0.0 row
    x[2] = 0
    x[2, 17] = 0xBF80                          # single -1.0
    x[3] = g.integers(0, 0x80, size=136).astype(np.uint16)                 # subnormal row
    x[4] = f32_to_bf16_bits((g.standard_normal(136) * 1e38).astype(np.float32))   # near FLT_MAX
    x[5] = f32_to_bf16_bits(np.array([1.984375] + [(2 * k + 1) / 128.0 for k in range(135)], np.float32))  # exact ties
    check_act(x)
    check_act(x[:0])


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def gpu_forward(W_bits, x_bits, n, out_dtype):
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W_bits), n)
    xq, a = sbl.act_quant(to_dev_bf16(x_bits))
    y = sbl.forward(codes, gamma, xq, a, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


def ref_forward(W_bits, x_bits, n, rows=None):
    w_eff, _, g = oracle.effective_weight(W_bits, n)
    xs = x_bits if rows is None else x_bits[rows]
    xq, a = oracle.act_quant(xs)
    acc = oracle.forward_acc(w_eff, xq)
    return acc, oracle.forward_y(acc, g, a)


FWD_SHAPES = [(64, 256, 256), (77, 200, 328), (1, 8, 8), (130, 136, 136), (513, 4864, 896), (33, 40, 1032),
              (100, 300, 192), (700, 1000, 1152)]


@pytest.mark.parametrize("n", [6, 2, 8, 4])
@pytest.mark.parametrize("T,d_out,d_in", FWD_SHAPES)
def test_forward_parity(T, d_out, d_in, n):
    W = weight(31, d_out + d_in, d_out, d_in)
    x = activation(31, d_out + d_in + T, T, d_in, dist="student_t4")
    acc_ref, y_ref = ref_forward(W, x, n)
    acc = gpu_forward(W, x, n, sbl.I32).cpu().numpy()
    np.testing.assert_array_equal(acc, acc_ref)
    y = gpu_forward(W, x, n, sbl.F32).cpu().numpy()
    assert_y_close(y, y_ref, acc_ref)
    yb = gpu_forward(W, x, n, sbl.BF16).float().cpu().numpy()
    assert np.all(np.abs(yb - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + 1e-30)


def test_forward_large_tiles_sampled():
    # big enough for the 256 x 256 tile path; compare 96 sampled tokens exactly
    T, d_out, d_in = 4096, 8192, 520          # d_in % 16 == 8 and d_in/8 % 8 != 0: unaligned loaders
    W = weight(41, 0, d_out, d_in)
    x = activation(41, 1, T, d_in)
    rows = sample_rows(41, 2, T, 96)
    acc = gpu_forward(W, x, 6, sbl.I32)[torch.from_numpy(rows).cuda()].cpu().numpy()
    acc_ref, y_ref = ref_forward(W, x, 6, rows)
    np.testing.assert_array_equal(acc, acc_ref)
    y = gpu_forward(W, x, 6, sbl.F32)[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert_y_close(y, y_ref, acc_ref)


@pytest.mark.parametrize("d_in", [256, 384])
def test_forward_several_tiles_per_block(d_in):
    # 17 x 17 = 289 tiles of 256 x 256 (more than one per CU, ragged in both
    # directions) with 2 or 3 K steps each: blocks walk several tiles and load
    # the next tile's first steps during the current one.  Rows from every row
    # tile (its first, last and a middle one), all outputs, exact int32, and
    # the bf16 output within one rounding.
    T, d_out = 4100, 4100
    W = weight(43, d_in, d_out, d_in)
    x = activation(43, d_out, T, d_in, dist="student_t4")
    rows = np.unique(np.concatenate([np.arange(0, T, 256), np.arange(255, T, 256), np.arange(100, T, 256), [T - 1]]))
    idx = torch.from_numpy(rows).cuda()
    acc_ref, y_ref = ref_forward(W, x, 6, rows)
    acc = gpu_forward(W, x, 6, sbl.I32)[idx].cpu().numpy()
    np.testing.assert_array_equal(acc, acc_ref)
    yb = gpu_forward(W, x, 6, sbl.BF16)[idx].float().cpu().numpy()
    assert np.all(np.abs(yb - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + 1e-30)
    y = gpu_forward(W, x, 6, sbl.F32)[idx].cpu().numpy()
    assert_y_close(y, y_ref, acc_ref)


# Decode (T <= 64): the streaming kernel, every mask, ragged row counts.
DECODE_T = [1, 5, 8, 16, 17, 33, 64]


@pytest.mark.parametrize("n", [6, 4, 2])
@pytest.mark.parametrize("d_out,d_in", [(256, 2048), (130, 448), (2050, 640), (7, 64)])
@pytest.mark.parametrize("T", DECODE_T)
def test_decode_parity(T, d_out, d_in, n):
    W = weight(61, d_out + d_in, d_out, d_in)
    x = activation(61, d_out + d_in + T, T, d_in, dist="student_t4")
    acc_ref, y_ref = ref_forward(W, x, n)
    acc = gpu_forward(W, x, n, sbl.I32).cpu().numpy()
    np.testing.assert_array_equal(acc, acc_ref)
    y = gpu_forward(W, x, n, sbl.F32).cpu().numpy()
    assert_y_close(y, y_ref, acc_ref)
    yb = gpu_forward(W, x, n, sbl.BF16).float().cpu().numpy()
    assert np.all(np.abs(yb - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + 1e-30)


@pytest.mark.parametrize("T", [1, 8, 64])
@pytest.mark.parametrize("name,d_out,d_in", [("gate", 11008, 2048), ("down", 2048, 11008)])
def test_decode_full_size(T, name, d_out, d_in):
    # decode workload: 3B-like matrices, Student-t(4) activations, T = 1 / 8 / 64, exact int32
    W = weight(71, d_in, d_out, d_in)
    x = activation(71, d_out + T, T, d_in, dist="student_t4")
    acc_ref, _ = ref_forward(W, x, 6)
    acc = gpu_forward(W, x, 6, sbl.I32).cpu().numpy()
    np.testing.assert_array_equal(acc, acc_ref)


# Fused decode (sbl_decode: act quant + forward in one launch, T <= 16): the
# same x_q and int32 sums as the two-call path, so every output is identical
# to it, and it matches the oracle.
@pytest.mark.parametrize("n", [6, 2])
@pytest.mark.parametrize("d_out,d_in", [(256, 2048), (130, 448), (2050, 640), (7, 64), (40, 2944)])
@pytest.mark.parametrize("T", [1, 3, 8, 16])
def test_decode_fused_parity(T, d_out, d_in, n):
    W = weight(63, d_out + d_in, d_out, d_in)
    x = activation(63, d_out + d_in + T, T, d_in, dist="student_t4")
    assert sbl.decode_supported(T, d_in)
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), n)
    xd = to_dev_bf16(x)
    acc_ref, y_ref = ref_forward(W, x, n)
    xq, a = sbl.act_quant(xd)
    for dt in (sbl.I32, sbl.F32, sbl.BF16):
        y_two = sbl.forward(codes, gamma, xq, a, out_dtype=dt)
        y_one = sbl.decode(codes, gamma, xd, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(y_one.view(torch.int32 if dt != sbl.BF16 else torch.int16),
                           y_two.view(torch.int32 if dt != sbl.BF16 else torch.int16)), dt
    np.testing.assert_array_equal(sbl.decode(codes, gamma, xd, out_dtype=sbl.I32).cpu().numpy(), acc_ref)
    assert_y_close(sbl.decode(codes, gamma, xd, out_dtype=sbl.F32).cpu().numpy(), y_ref, acc_ref)


DECODE_GROUPS = {"qkv": [(2048, 2048), (256, 2048), (256, 2048)], "gate_up": [(11008, 2048), (11008, 2048)],
                 "ragged": [(40, 1024), (8, 1024), (1000, 1024), (17, 1024)]}


def decode_group(group, T, n=6):
    shapes = DECODE_GROUPS[group]
    d_in = shapes[0][1]
    Ws = [weight(77, 10 * i + len(group), d_o, d_i) for i, (d_o, d_i) in enumerate(shapes)]
    mats = []
    for W in Ws:
        codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), n, want_mask=False)
        mats.append((codes, gamma))
    x = activation(77, 99 + T, T, d_in, dist="student_t4")
    return Ws, mats, x


def same_bits(a, b, dt):
    v = torch.int16 if dt == sbl.BF16 else torch.int32
    return torch.equal(a.view(v), b.view(v))


@pytest.mark.parametrize("group", sorted(DECODE_GROUPS))
@pytest.mark.parametrize("T", [1, 5, 16])
def test_decode_multi_matches_single(T, group):
    # several matrices sharing x in one launch: every output equals decode of that matrix alone
    Ws, mats, x = decode_group(group, T)
    xd = to_dev_bf16(x)
    for dt in (sbl.I32, sbl.BF16, sbl.F32):
        ys = sbl.decode_multi(mats, xd, out_dtype=dt)
        for (codes, gamma), y in zip(mats, ys):
            want = sbl.decode(codes, gamma, xd, out_dtype=dt)
            torch.cuda.synchronize()
            assert same_bits(y, want, dt), (group, T, dt)
    if group == "ragged":  # and, directly, against the oracle
        ys = sbl.decode_multi(mats, xd, out_dtype=sbl.I32)
        for W, y in zip(Ws, ys):
            acc_ref, _ = ref_forward(W, x, 6)
            np.testing.assert_array_equal(y.cpu().numpy(), acc_ref)


@pytest.mark.parametrize("T,shapes", [(8, [(8200, 128), (8200, 128), (40, 128)]),
                                      (12, [(8200, 128), (8200, 128), (40, 128)]),
                                      (16, [(8200, 128), (8200, 128), (40, 128)]),
                                      (16, [(8192, 2944), (8200, 2944)])])
def test_decode_multi_ragged_and_wide_rows(T, shapes):
    # x quantized in the launch (bf16 x given): ragged last tiles of 8200 and 40 rows at 8-16
    # tokens, and rows of 2944 whose 16-token activation tile fills most of a block's LDS over
    # more than 16384 output rows; every output equals decode of that matrix alone, and the
    # int32 sums equal the oracle's
    d_in = shapes[0][1]
    Ws = [weight(78, 10 * i + T, d_o, d_i) for i, (d_o, d_i) in enumerate(shapes)]
    mats = []
    for W in Ws:
        codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6, want_mask=False)
        mats.append((codes, gamma))
    x = activation(78, 200 + T, T, d_in, dist="student_t4")
    xd = to_dev_bf16(x)
    for dt in (sbl.I32, sbl.BF16):
        ys = sbl.decode_multi(mats, xd, out_dtype=dt)
        for (codes, gamma), y in zip(mats, ys):
            want = sbl.decode(codes, gamma, xd, out_dtype=dt)
            torch.cuda.synchronize()
            assert same_bits(y, want, dt), (shapes, T, dt)
    ys = sbl.decode_multi(mats, xd, out_dtype=sbl.I32)
    for W, y in zip(Ws, ys):
        acc_ref, _ = ref_forward(W, x, 6)
        np.testing.assert_array_equal(y.cpu().numpy(), acc_ref)


@pytest.mark.parametrize("group", sorted(DECODE_GROUPS))
@pytest.mark.parametrize("T", [1, 16, 33, 64])
def test_forward_decode_multi_matches_single(T, group):
    # the same with x_q given (every decode token count, one and four token tiles)
    Ws, mats, x = decode_group(group, T)
    xq, a = sbl.act_quant(to_dev_bf16(x))
    for dt in (sbl.I32, sbl.BF16, sbl.F32):
        ys = sbl.forward_decode_multi(mats, xq, a, out_dtype=dt)
        for (codes, gamma), y in zip(mats, ys):
            want = sbl.forward(codes, gamma, xq, a, out_dtype=dt)
            torch.cuda.synchronize()
            assert same_bits(y, want, dt), (group, T, dt)
    if group == "ragged":
        ys = sbl.forward_decode_multi(mats, xq, a, out_dtype=sbl.I32)
        for W, y in zip(Ws, ys):
            acc_ref, _ = ref_forward(W, x, 6)
            np.testing.assert_array_equal(y.cpu().numpy(), acc_ref)


@pytest.mark.parametrize("T,d_in", [(1, 8192), (5, 8192), (16, 3008)])
def test_decode_fused_largest_rows(T, d_in):
    # the longest rows the fused path takes (16 register chunks per lane, the 48 KB tile)
    d_out = 48
    W = weight(65, T, d_out, d_in)
    x = activation(65, d_in + T, T, d_in, dist="student_t4")
    assert sbl.decode_supported(T, d_in)
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6)
    acc_ref, _ = ref_forward(W, x, 6)
    acc = sbl.decode(codes, gamma, to_dev_bf16(x), out_dtype=sbl.I32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)


def test_decode_fused_zero_and_tiny_rows():
    # a zero row (a_t = 0, x_q = 0, y = 0), a row of one non-zero, a row at the
    # bf16 extremes: the fused quantization handles each as the act quant does
    d_out, d_in, T = 64, 256, 4
    W = weight(64, 0, d_out, d_in)
    x = activation(64, 1, T, d_in)
    x[0] = 0
    x[1] = 0
    x[1, 17] = f32_to_bf16_bits(np.array([-3.0e-30], np.float32))[0]
    x[2] = f32_to_bf16_bits(np.linspace(-3.0e38, 3.0e38, d_in).astype(np.float32))
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6)
    acc_ref, y_ref = ref_forward(W, x, 6)
    acc = sbl.decode(codes, gamma, to_dev_bf16(x), out_dtype=sbl.I32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    y = sbl.decode(codes, gamma, to_dev_bf16(x), out_dtype=sbl.F32).cpu().numpy()
    assert_y_close(y, y_ref, acc_ref)


@pytest.mark.parametrize("T,d_in", [(16, 448), (9, 2944), (3, 11008), (16, 64)])
def test_decode_fused_row_maxima_positions(T, d_in):
    # the in-launch row maxima are reduced per wave over runs of 64 consecutive 16-byte
    # chunks that may cross row ends: each row's largest magnitude is placed at its first
    # chunk, its last chunk, a chunk at a 64-chunk boundary or in between, and x_q (hence
    # the int32 sums) must equal the two-call path and the oracle
    d_out = 48
    nch = d_in // 8
    W = weight(66, T, d_out, d_in)
    x = activation(66, d_in + T, T, d_in)
    big = f32_to_bf16_bits(np.array([5.0e3, -7.5e3], np.float32))
    for t in range(T):
        c = t * nch
        choice = [c, c + nch - 1, ((c // 64) + 1) * 64, c + nch // 2][t % 4]
        if not c <= choice < c + nch:
            choice = c + (t * 13) % nch
        x[t, 8 * (choice - c) + t % 8] = big[t % 2]
    assert sbl.decode_supported(T, d_in)
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6)
    acc_ref, _ = ref_forward(W, x, 6)
    xd = to_dev_bf16(x)
    xq, a = sbl.act_quant(xd)
    two = sbl.forward(codes, gamma, xq, a, out_dtype=sbl.I32)
    one = sbl.decode(codes, gamma, xd, out_dtype=sbl.I32)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    np.testing.assert_array_equal(one.cpu().numpy(), acc_ref)


@pytest.mark.parametrize("T", [1, 8, 16])
@pytest.mark.parametrize("name,d_out,d_in", [("gate", 11008, 2048), ("q", 2048, 2048), ("k", 256, 2048)])
def test_decode_fused_full_size(T, name, d_out, d_in):
    # decode workload shapes that take the fused path: exact int32 sums
    W = weight(73, d_in, d_out, d_in)
    x = activation(73, d_out + T, T, d_in, dist="student_t4")
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6)
    acc_ref, _ = ref_forward(W, x, 6)
    acc = sbl.decode(codes, gamma, to_dev_bf16(x), out_dtype=sbl.I32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)


def test_decode_graph_replay_matches_eager():
    # act quant + forward captured in a HIP graph (as the decode measurement runs them):
    # every replay, with eager work between replays, equals the eager result
    W = weight(75, 0, 512, 1024)
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6, want_mask=False)
    x = to_dev_bf16(activation(75, 1, 8, 1024, dist="student_t4"))
    xq = torch.empty((8, 1024), dtype=torch.int8, device="cuda")
    a = torch.empty((8,), dtype=torch.float32, device="cuda")
    y = torch.empty((8, 512), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((8, 512), dtype=torch.bfloat16, device="cuda")

    def run():
        sbl.act_quant(x, x_q=xq, absmax=a)
        sbl.forward(codes, gamma, xq, a, out_dtype=sbl.BF16, y=y)
        sbl.decode(codes, gamma, x, out_dtype=sbl.BF16, y=y2)   # the fused form of the same step

    run()
    torch.cuda.synchronize()
    want = y.clone()
    assert torch.equal(y2.view(torch.int16), want.view(torch.int16))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(4):
        y.zero_()
        y2.zero_()
        xq.zero_()
        other = sbl.forward(codes, gamma, xq, a)        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"replay {i}"
        assert torch.equal(y2.view(torch.int16), want.view(torch.int16)), f"replay {i} (fused)"
        assert other.shape == (8, 512)


@pytest.mark.parametrize("T", [17, 64])
def test_forward_decode_multi_ragged_twin_rows(T):
    # a grid of 1026 blocks of 16 rows past 16 tokens takes 32-row blocks; d_out = 8200 leaves
    # each matrix a last block of 8 rows (and one of 40 a short last tile): outputs equal one
    # call per matrix (16-row blocks) and the oracle, bit for bit
    shapes = [(8200, 128), (8200, 128), (40, 128)]
    Ws = [weight(79, i, d_o, d_i) for i, (d_o, d_i) in enumerate(shapes)]
    mats = []
    for W in Ws:
        codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6, want_mask=False)
        mats.append((codes, gamma))
    x = activation(79, 9, T, 128, dist="student_t4")
    xq, a = sbl.act_quant(to_dev_bf16(x))
    ys = sbl.forward_decode_multi(mats, xq, a, out_dtype=sbl.I32)
    for W, (codes, gamma), y in zip(Ws, mats, ys):
        want = sbl.forward(codes, gamma, xq, a, out_dtype=sbl.I32)
        torch.cuda.synchronize()
        assert torch.equal(y, want)
        acc_ref, _ = ref_forward(W, x, 6)
        np.testing.assert_array_equal(y.cpu().numpy(), acc_ref)


@pytest.mark.parametrize("T", [8, 48])
def test_decode_multi_graph_replay_matches_eager(T):
    # the grouped launches captured in a HIP graph, as the decode measurement runs them
    # (the fused form up to 16 tokens, act quant + the grouped product past that, on the
    # 32-row blocks of a large grid): every replay equals the eager result
    Ws, mats, xb = decode_group("gate_up", T)
    x = to_dev_bf16(xb)
    xq = torch.empty((T, 2048), dtype=torch.int8, device="cuda")
    a = torch.empty((T,), dtype=torch.float32, device="cuda")
    ys = [torch.empty((T, 11008), dtype=torch.bfloat16, device="cuda") for _ in mats]

    def run():
        if sbl.decode_supported(T, 2048):
            sbl.decode_multi(mats, x, out_dtype=sbl.BF16, ys=ys)
        else:
            sbl.act_quant(x, x_q=xq, absmax=a)
            sbl.forward_decode_multi(mats, xq, a, out_dtype=sbl.BF16, ys=ys)

    run()
    torch.cuda.synchronize()
    want = [y.clone() for y in ys]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        for y in ys:
            y.zero_()
        other = sbl.decode_multi(mats[:1], x[:1], out_dtype=sbl.F32)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, w in zip(ys, want):
            assert torch.equal(y.view(torch.int16), w.view(torch.int16)), f"replay {i}"
        assert other[0].shape == (1, 11008)


# training shapes as timed: the 3B-like layer at 32768 tokens and the 1.5B-like one at 8192
FULL_SHAPES = [("gate", 32768, 11008, 2048), ("down", 32768, 2048, 11008), ("q", 32768, 2048, 2048),
               ("k", 32768, 256, 2048), ("gate_1.5b", 8192, 8960, 1536), ("down_1.5b", 8192, 1536, 8960),
               ("q_1.5b", 8192, 1536, 1536)]


@pytest.mark.parametrize("name,T,d_out,d_in", FULL_SHAPES)
def test_forward_full_size_sampled(name, T, d_out, d_in):
    # 64 sampled tokens, all outputs, exact int32
    W = weight(81, d_in, d_out, d_in)
    x = activation(81, d_out, T, d_in, dist="student_t4")
    rows = sample_rows(81, 2, T, 64)
    idx = torch.from_numpy(rows).cuda()
    acc = gpu_forward(W, x, 6, sbl.I32)[idx].cpu().numpy()
    acc_ref, y_ref = ref_forward(W, x, 6, rows)
    np.testing.assert_array_equal(acc, acc_ref)
    yb = gpu_forward(W, x, 6, sbl.BF16)[idx].float().cpu().numpy()
    assert np.all(np.abs(yb - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + 1e-30)


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def gpu_backward(W_bits, x_bits, dY_bits, n, dx_dtype=1):
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W_bits), n)
    xq, a = sbl.act_quant(to_dev_bf16(x_bits))
    dX, dW = sbl.backward(codes, gamma, xq, a, to_dev_bf16(dY_bits), dx_dtype=dx_dtype)
    torch.cuda.synchronize()
    return dX, dW


BWD_SHAPES = [(64, 256, 256), (77, 200, 328), (513, 136, 72), (1, 8, 8), (300, 40, 1032), (4096, 256, 2048),
              (45, 100, 64), (130, 12, 264), (1000, 520, 776)]


@pytest.mark.parametrize("T,d_out,d_in", BWD_SHAPES)
def test_backward_parity(T, d_out, d_in):
    W = weight(51, d_out + d_in, d_out, d_in)
    x = activation(51, d_out + d_in + T, T, d_in, dist="student_t4")
    dY = grad_out(51, d_out + d_in + T, T, d_out)
    r = oracle.sparse_bitlinear_step(W, x, dY, 6)
    dX, dW = gpu_backward(W, x, dY, 6)
    assert_grad_close(bf16_to_f64(dX), r["dX"])
    assert_grad_close(dW.cpu().numpy(), r["dW"])
    assert_grad_close(bf16_to_f64(dX), r["dX"], tol=ERR_MODEL_BF16)
    assert_grad_close(dW.cpu().numpy(), r["dW"], tol=ERR_MODEL_BF16)
    dX32, _ = gpu_backward(W, x, dY, 6, dx_dtype=0)
    assert_grad_close(dX32.cpu().numpy().astype(np.float64), r["dX"], tol=ERR_MODEL_F32)
    # Dual STE: masked positions receive their (non-zero) dense gradient
    masked = ~r["mask"]
    if masked.any():
        assert np.count_nonzero(dW.cpu().numpy()[masked]) > 0.99 * masked.sum()


@pytest.mark.parametrize("d_out", [64, 128, 192, 256, 320, 448, 200])
def test_backward_dx_k_step_counts(d_out):
    # the dX product runs its K steps (64 wide, K = d_out) in rounds of three LDS stages
    # and the remaining one or two in straight code: 1 to 7 steps, and a ragged tail
    # (200 = 3 steps + 8); 600 tokens make 5 row tiles, the last ragged
    T, d_in = 600, 1024
    W = weight(57, d_out, d_out, d_in)
    x = activation(57, d_out + 1, T, d_in)
    dY = grad_out(57, d_out + 2, T, d_out)
    rows = sample_rows(57, d_out, T, 64)
    dX, _ = gpu_backward(W, x, dY, 6)
    w_eff, _, g = oracle.effective_weight(W, 6)
    xq, a = oracle.act_quant(x)
    dX_ref, _ = oracle.backward(dY[rows], w_eff, g, xq[rows], a[rows])
    assert_grad_close(bf16_to_f64(dX)[rows], dX_ref)
    assert_grad_close(bf16_to_f64(dX)[rows], dX_ref, tol=ERR_MODEL_BF16)
    dX32, _ = gpu_backward(W, x, dY, 6, dx_dtype=0)
    assert_grad_close(dX32.cpu().numpy().astype(np.float64)[rows], dX_ref, tol=ERR_MODEL_F32)


def test_backward_dx_large_tiles_sampled():
    T, d_out, d_in = 4096, 264, 8192
    W = weight(61, 0, d_out, d_in)
    x = activation(61, 1, T, d_in)
    dY = grad_out(61, 2, T, d_out)
    rows = sample_rows(61, 3, T, 64)
    dX, dW = gpu_backward(W, x, dY, 6)
    w_eff, _, g = oracle.effective_weight(W, 6)
    xq, a = oracle.act_quant(x)
    dX_ref, _ = oracle.backward(dY[rows], w_eff, g, xq[rows], a[rows])
    assert_grad_close(bf16_to_f64(dX)[rows], dX_ref)
    assert_grad_close(bf16_to_f64(dX)[rows], dX_ref, tol=ERR_MODEL_BF16)
    cols = sample_rows(61, 4, d_out, 32)       # sampled rows o of dW over all T
    dW_ref = oracle.bf16_to_f64(dY[:, cols]).T @ oracle.dequant_act(xq, a)
    assert_grad_close(dW.cpu().numpy()[cols], dW_ref)
    assert_grad_close(dW.cpu().numpy()[cols], dW_ref, tol=ERR_MODEL_BF16)


@pytest.mark.parametrize("name,T,d_out,d_in", FULL_SHAPES)
def test_backward_full_size_sampled(name, T, d_out, d_in):
    # dX on 256 sampled tokens, dW on 64 sampled output rows over all tokens (split-K
    # and transposes included)
    W = weight(91, d_in, d_out, d_in)
    x = activation(91, d_out, T, d_in, dist="student_t4")
    dY = grad_out(91, d_out + 1, T, d_out)
    dX, dW = gpu_backward(W, x, dY, 6)
    w_eff, _, g = oracle.effective_weight(W, 6)
    xq, a = oracle.act_quant(x)
    rows = sample_rows(91, 3, T, 256)
    dX_ref, _ = oracle.backward(dY[rows], w_eff, g, xq[rows], a[rows])
    assert_grad_close(bf16_to_f64(dX)[rows], dX_ref)
    assert_grad_close(bf16_to_f64(dX)[rows], dX_ref, tol=ERR_MODEL_BF16)
    cols = sample_rows(91, 4, d_out, min(64, d_out))
    dW_ref = oracle.bf16_to_f64(dY[:, cols]).T @ oracle.dequant_act(xq, a)
    assert_grad_close(dW.cpu().numpy()[cols], dW_ref)
    assert_grad_close(dW.cpu().numpy()[cols], dW_ref, tol=ERR_MODEL_BF16)


@pytest.mark.parametrize("T,d_out,d_in,planes", [(4096, 4608, 4096, 5), (2000, 4504, 4112, 2)])
def test_backward_dw_split_tail_full(T, d_out, d_in, planes):
    # 288 (306) tiles of 256 x 256: the first 256 take one full-K range (a whole
    # round of blocks, summed straight into dW), the last 32 (50, ragged in both
    # dimensions) a deeper split with a ragged last K range, planes 1.. of it in
    # the workspace; every dW entry against the oracle
    assert sbl.backward_workspace_size(T, d_in, d_out) >= planes * d_out * d_in * 4
    W = weight(97, 0, d_out, d_in)
    x = activation(97, 1, T, d_in, dist="student_t4")
    dY = grad_out(97, 2, T, d_out)
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6)
    xq, a = sbl.act_quant(to_dev_bf16(x))
    _, dW = sbl.backward(codes, gamma, xq, a, to_dev_bf16(dY), need_dx=False)
    _, dW2 = sbl.backward(codes, gamma, xq, a, to_dev_bf16(dY))  # fused with dX: same bits
    torch.cuda.synchronize()
    assert torch.equal(dW, dW2)
    xq_h, a_h = oracle.act_quant(x)
    dW_ref = oracle.bf16_to_f64(dY).T @ oracle.dequant_act(xq_h, a_h)
    assert_grad_close(dW.cpu().numpy(), dW_ref)
    assert_grad_close(dW.cpu().numpy(), dW_ref, tol=ERR_MODEL_BF16)


@pytest.mark.parametrize("T,d_out,d_in", [(1000, 520, 776), (77, 200, 328), (4096, 256, 2048), (300, 2048, 512)])
def test_backward_fused_matches_separate(T, d_out, d_in):
    # dX and dW in one call (the dX product writes dY^T for dW) equal the two separate calls bit for bit
    W = weight(95, d_out + d_in, d_out, d_in)
    x = activation(95, d_out + d_in + T, T, d_in, dist="student_t4")
    dY = to_dev_bf16(grad_out(95, d_out + d_in + T + 1, T, d_out))
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6)
    xq, a = sbl.act_quant(to_dev_bf16(x))
    dX, dW = sbl.backward(codes, gamma, xq, a, dY)
    dX1, _ = sbl.backward(codes, gamma, xq, a, dY, need_dw=False)
    _, dW1 = sbl.backward(codes, gamma, xq, a, dY, need_dx=False)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.int16), dX1.view(torch.int16))
    assert torch.equal(dW, dW1)


def test_backward_zero_tokens():
    W = weight(71, 0, 64, 64)
    codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6)
    xq = torch.empty((0, 64), dtype=torch.int8, device="cuda")
    a = torch.empty((0,), dtype=torch.float32, device="cuda")
    dY = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    dW = torch.full((64, 64), 7.0, device="cuda")
    dX, dW = sbl.backward(codes, gamma, xq, a, dY, dW=dW)
    torch.cuda.synchronize()
    assert dX.shape == (0, 64) and torch.all(dW == 0)
    y = sbl.forward(codes, gamma, xq, a)
    assert y.shape == (0, 64)


# ---------------------------------------------------------------------------
# whole step, determinism, autograd wrapper
# ---------------------------------------------------------------------------

def test_step_bitwise_deterministic():
    W = weight(81, 0, 512, 1024)
    x = activation(81, 1, 1000, 1024, dist="student_t4")
    dY = grad_out(81, 2, 1000, 512)
    outs = []
    for _ in range(2):
        codes, mask, gamma = sbl.quant_mask_pack(to_dev_bf16(W), 6)
        xq, a = sbl.act_quant(to_dev_bf16(x))
        y = sbl.forward(codes, gamma, xq, a)
        dX, dW = sbl.backward(codes, gamma, xq, a, to_dev_bf16(dY))
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (codes, mask, gamma, xq, a, y, dX.view(torch.int16), dW)])
    for u, v in zip(*outs):
        assert torch.equal(u, v)


@pytest.mark.parametrize("d_out,d_in,T", [(256, 256, 64), (512, 1024, 1000), (4864, 896, 512)])
def test_step_graph_replay_matches_eager(d_out, d_in, T):
    # a whole step (packing, act quant, forward, backward with its split-K sums) captured in one
    # HIP graph, as bench.py times the launch-bound workloads: every replay, with eager work and
    # cleared outputs between the replays, equals the eager step bit for bit
    W = to_dev_bf16(weight(83, d_out, d_out, d_in))
    x = to_dev_bf16(activation(83, d_in, T, d_in, dist="student_t4"))
    dY = to_dev_bf16(grad_out(83, T, T, d_out))
    codes, mask, gamma = sbl.quant_mask_pack(W, 6)
    xq, a = sbl.act_quant(x)
    y = sbl.forward(codes, gamma, xq, a, out_dtype=sbl.BF16)
    dX, dW = sbl.backward(codes, gamma, xq, a, dY, dx_dtype=sbl.BF16)
    torch.cuda.synchronize()
    want = [t.clone() for t in (codes, mask, gamma, xq, a, y, dX, dW)]
    outs = [torch.empty_like(t) for t in want]
    qws = torch.empty((max(16, sbl.quant_workspace_size(d_out, d_in)),), dtype=torch.uint8, device="cuda")
    bws = torch.empty((max(16, sbl.backward_workspace_size(T, d_in, d_out, sbl.BWD_DX | sbl.BWD_DW)),),
                      dtype=torch.uint8, device="cuda")

    def run():
        c, m, g, q, s, yy, dx, dw = outs
        sbl.quant_mask_pack(W, 6, codes=c, mask=m, gamma=g, workspace=qws)
        sbl.act_quant(x, x_q=q, absmax=s)
        sbl.forward(c, g, q, s, out_dtype=sbl.BF16, y=yy)
        sbl.backward(c, g, q, s, dY, dx_dtype=sbl.BF16, dX=dx, dW=dw, workspace=bws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        for t in outs:
            t.zero_()
        other = sbl.act_quant(x[:7])                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (got, ref) in enumerate(zip(outs, want)):
            if got.dtype.is_floating_point:
                got, ref = got.view(torch.int16 if got.element_size() == 2 else torch.int32), \
                    ref.view(torch.int16 if ref.element_size() == 2 else torch.int32)
            assert torch.equal(got, ref), f"replay {i}, output {k}"
        assert other[0].shape == (7, d_in)
    del g


def test_autograd_function_matches_oracle():
    W = weight(91, 0, 96, 128)
    x = activation(91, 1, 40, 128)
    dY = grad_out(91, 2, 40, 96)
    xt = to_dev_bf16(x).requires_grad_(True)
    Wt = to_dev_bf16(W).requires_grad_(True)
    y = sbl.sparse_bitlinear(xt, Wt, 6)
    y.backward(to_dev_bf16(dY).float())
    r = oracle.sparse_bitlinear_step(W, x, dY, 6)
    assert_y_close(y.detach().cpu().numpy(), r["y"], r["acc"])
    assert_grad_close(bf16_to_f64(xt.grad), r["dX"])
    assert_grad_close(Wt.grad.float().cpu().numpy().astype(np.float64), r["dW"], tol=2e-2)


# ---------------------------------------------------------------------------
# the contract symbol itself, and the binding's checks before any launch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape,n", [((256, 256), 6), ((333, 72), 2), ((1, 8), 8)])
def test_pack_contract_symbol(shape, n):
    """sbl_quant_mask_pack called through ctypes (with and without a mask plane)."""
    import ctypes
    W_bits = weight(13, shape[0] + shape[1], *shape)
    d_out, d_in = shape
    W = to_dev_bf16(W_bits)
    codes = torch.empty((d_out, d_in // 8), dtype=torch.int16, device="cuda")
    mask = torch.empty((d_out, d_in // 8), dtype=torch.uint8, device="cuda")
    gamma = torch.empty((1,), dtype=torch.float32, device="cuda")
    need = sbl.lib.sbl_quant_mask_pack_workspace_size(d_out, d_in)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc, rm, rg = oracle.quant_mask_pack(W_bits, n)
    for with_mask in (True, False):
        st = sbl.lib.sbl_quant_mask_pack(vp(W), d_out, d_in, n, vp(codes), vp(mask) if with_mask else None,
                                         vp(gamma), vp(ws), need, None)
        assert st == 0, sbl.lib.sbl_last_error()
        torch.cuda.synchronize()
        assert f32_bits(gamma.cpu().numpy()[0]) == f32_bits(rg)
        np.testing.assert_array_equal(bits16(codes), rc)
        if with_mask:
            np.testing.assert_array_equal(mask.cpu().numpy(), rm)


def test_binding_rejects_mismatched_operands():
    W = to_dev_bf16(weight(17, 0, 64, 128))
    codes, _, gamma = sbl.quant_mask_pack(W, 6)
    xq, a = sbl.act_quant(to_dev_bf16(activation(17, 1, 16, 128)))
    dY = to_dev_bf16(grad_out(17, 2, 16, 64))
    torch.cuda.synchronize()
    bad = [
        (ValueError, lambda: sbl.backward(codes[:, :8], gamma, xq, a, dY)),          # G * 8 != d_in
        (ValueError, lambda: sbl.backward(codes, gamma, xq, a[:8], dY)),             # absmax length != T
        (ValueError, lambda: sbl.backward(codes, gamma[:0], xq, a, dY)),             # no gamma
        (TypeError, lambda: sbl.backward(codes.float(), gamma, xq, a, dY)),          # codes dtype
        (TypeError, lambda: sbl.backward(codes, gamma, xq.to(torch.int16), a, dY)),  # x_q dtype
        (TypeError, lambda: sbl.backward(codes, gamma.double(), xq, a, dY)),         # gamma dtype
        (ValueError, lambda: sbl.backward(codes, gamma, xq, a, dY.cpu())),           # dY on the host
        (ValueError, lambda: sbl.backward(codes.t(), gamma, xq, a, dY)),             # not contiguous
        (ValueError, lambda: sbl.forward(codes, gamma, xq, a[:3])),
        (ValueError, lambda: sbl.forward(codes[:, :4], gamma, xq, a)),
        (TypeError, lambda: sbl.forward(codes, gamma, xq.float(), a)),
        (ValueError, lambda: sbl.forward_decode_multi([(codes, gamma)], xq, a[:1])),
        (ValueError, lambda: sbl.decode(codes, gamma[:0], to_dev_bf16(activation(17, 3, 2, 128)))),
    ]
    for exc, call in bad:
        with pytest.raises(exc):
            call()


# ---------------------------------------------------------------------------
# pair plane (one byte per group of 8, masks keeping at most 2 of 8): packing
# against the oracle, and the decode-size forward on it against the code plane
# and the oracle (exact int32)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [2, 1])
@pytest.mark.parametrize("d_out,d_in", [(256, 2048), (37, 1024), (11008, 2048), (5, 8)])
def test_pack_pairs_parity(d_out, d_in, n):
    W = weight(93, d_out + d_in + n, d_out, d_in)
    codes, _, _ = sbl.quant_mask_pack(to_dev_bf16(W), n, want_mask=False)
    plane, bad = sbl.pack_pairs(codes)
    torch.cuda.synchronize()
    w_eff, _, _ = oracle.effective_weight(W, n) if d_out * d_in <= 4 << 20 else (None, None, None)
    if w_eff is not None:
        np.testing.assert_array_equal(plane.cpu().numpy(), oracle.pack_pairs(w_eff))
    else:  # large: the plane unpacks to the GPU's own code plane
        np.testing.assert_array_equal(oracle.unpack_pairs(plane.cpu().numpy()), oracle.unpack_codes(bits16(codes)))
    assert int(bad.item()) == 0


def test_pack_pairs_counts_unrepresentable_groups():
    # a 6:8 code plane has groups with more than 2 non-zeros: each is counted and written as 0
    W = weight(94, 0, 64, 256)
    codes, _, _ = sbl.quant_mask_pack(to_dev_bf16(W), 6, want_mask=False)
    plane, bad = sbl.pack_pairs(codes)
    torch.cuda.synchronize()
    nz = (oracle.unpack_codes(bits16(codes)) != 0).reshape(64, 32, 8).sum(axis=2)
    assert int(bad.item()) == int((nz > 2).sum()) > 0
    assert np.all(plane.cpu().numpy()[nz > 2] == 0)


def _pairs_mats(shapes, n, seed):
    Ws, codes_mats, pair_mats = [], [], []
    for i, (d_o, d_i) in enumerate(shapes):
        W = weight(seed, 10 * i + n, d_o, d_i)
        codes, _, gamma = sbl.quant_mask_pack(to_dev_bf16(W), n, want_mask=False)
        plane, bad = sbl.pack_pairs(codes)
        Ws.append(W)
        codes_mats.append((codes, gamma))
        pair_mats.append((plane, gamma))
    torch.cuda.synchronize()
    return Ws, codes_mats, pair_mats


PAIR_SHAPES = {"qkv": [(2048, 2048), (256, 2048), (256, 2048)], "down": [(2048, 11008)],
               "ragged": [(40, 1024), (8200, 1024), (17, 1024)], "small": [(7, 128)]}


@pytest.mark.parametrize("n", [2, 1])
@pytest.mark.parametrize("group", sorted(PAIR_SHAPES))
@pytest.mark.parametrize("T", [1, 5, 8, 16, 17, 33, 64])
def test_decode_pairs_parity(T, group, n):
    shapes = PAIR_SHAPES[group]
    d_in = shapes[0][1]
    Ws, cm, pm = _pairs_mats(shapes, n, 95)
    x = activation(95, T + d_in, T, d_in, dist="student_t4")
    xd = to_dev_bf16(x)
    xq, a = sbl.act_quant(xd)
    for dt in (sbl.I32, sbl.F32, sbl.BF16):
        yc = sbl.forward_plane_multi(sbl.PLANE_CODES, cm, x_q=xq, absmax=a, out_dtype=dt)
        yp = sbl.forward_plane_multi(sbl.PLANE_PAIRS, pm, x_q=xq, absmax=a, out_dtype=dt)
        fused = sbl.decode_plane_supported(sbl.PLANE_PAIRS, T, d_in)
        yf = sbl.forward_plane_multi(sbl.PLANE_PAIRS, pm, x=xd, out_dtype=dt) if fused else yp
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert same_bits(yp[i], yc[i], dt), (i, dt)
            assert same_bits(yf[i], yc[i], dt), (i, dt)
    # exact sums against the oracle (the largest matrix on sampled rows)
    rq, _ = oracle.act_quant(x)
    yp = sbl.forward_plane_multi(sbl.PLANE_PAIRS, pm, x_q=xq, absmax=a, out_dtype=sbl.I32)
    torch.cuda.synchronize()
    for i, W in enumerate(Ws):
        rows = sample_rows(95, i, W.shape[0], 512)
        w_eff = oracle.unpack_codes(bits16(cm[i][0]))[rows]
        # the GPU's code plane equals the oracle's (pinned elsewhere); check it on these rows too
        w_ref, _, _ = oracle.effective_weight(W, n) if W.size <= 4 << 20 else (None, None, None)
        if w_ref is not None:
            np.testing.assert_array_equal(w_eff, w_ref[rows])
        acc_ref = oracle.forward_acc(w_eff, rq)
        np.testing.assert_array_equal(yp[i].cpu().numpy()[:, rows], acc_ref)


def test_decode_pairs_moves_half_the_code_bytes():
    # the plane a 2:8 decode streams: d_in / 8 bytes per row against d_in / 4
    W = weight(96, 0, 2048, 11008)
    codes, _, _ = sbl.quant_mask_pack(to_dev_bf16(W), 2, want_mask=False)
    plane, bad = sbl.pack_pairs(codes)
    assert plane.numel() * plane.element_size() * 2 == codes.numel() * codes.element_size()
