"""The no-allocation packing entry point (sbl_quant_mask_pack_noalloc, static
per-GPU scratch) against sbl_quant_mask_pack with a caller workspace, called
through the C ABI: two calls in a row, the second on a smaller matrix, codes,
mask plane and gamma bits identical (and equal to the oracle on the small one)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sbl_inputs import f32_to_bf16_bits, weight

from gpu_util import bits16, f32_bits, to_dev_bf16

pytestmark = pytest.mark.gpu

try:
    import sparsity_sparse_bitlinear_amd as sbl
except ImportError:
    if torch.cuda.is_available():  # a GPU without the library is a failure, not a skip
        raise
    pytest.skip("no GPU and no libsbl.so", allow_module_level=True)


def _vp(t):
    return ctypes.c_void_p(t.data_ptr())


def _pack_both(W_bits, n):
    lib = sbl.lib
    d_out, d_in = W_bits.shape
    W = to_dev_bf16(W_bits)
    outs = []
    for use_ws in (True, False):
        codes = torch.empty((d_out, d_in // 8), dtype=torch.int16, device="cuda:0")
        mask = torch.empty((d_out, d_in // 8), dtype=torch.uint8, device="cuda:0")
        gamma = torch.empty((1,), dtype=torch.float32, device="cuda:0")
        if use_ws:
            need = lib.sbl_quant_mask_pack_workspace_size(d_out, d_in)
            ws = torch.empty((need,), dtype=torch.uint8, device="cuda:0")
            rc = lib.sbl_quant_mask_pack(_vp(W), d_out, d_in, n, _vp(codes), _vp(mask), _vp(gamma), _vp(ws), need,
                                         None)
        else:
            rc = lib.sbl_quant_mask_pack_noalloc(_vp(W), d_out, d_in, n, _vp(codes), _vp(mask), _vp(gamma), None)
        assert rc == 0, lib.sbl_last_error()
        torch.cuda.synchronize()
        outs.append((bits16(codes), mask.cpu().numpy(), f32_bits(gamma.cpu().numpy()[0])))
    return outs


def _extreme_weight(d_out, d_in, seed):
    # values far outside the float64 window of the gamma reduction, so its blocks
    # write per-exponent histograms into the scratch
    g = np.random.default_rng(seed)
    base = g.standard_normal((d_out, d_in)).astype(np.float32) * 0.02
    base[g.random(base.shape) < 0.01] *= 1e30
    base[g.random(base.shape) < 0.01] *= 1e-30
    return f32_to_bf16_bits(base)


def test_noalloc_pack_two_calls_second_smaller():
    assert sbl.lib.sbl_quant_mask_pack_noalloc_scratch_bytes() >= sbl.lib.sbl_quant_mask_pack_workspace_size(
        11008, 2048)
    big = _extreme_weight(11008, 2048, 1)        # the largest grid of the reduction (1024 blocks)
    small = weight(7, 1, 300, 264)               # a few blocks, no histogram
    (c0, m0, g0), (c1, m1, g1) = _pack_both(big, 6)
    assert g0 == g1
    np.testing.assert_array_equal(c1, c0)
    np.testing.assert_array_equal(m1, m0)
    (c0, m0, g0), (c1, m1, g1) = _pack_both(small, 4)
    assert g0 == g1
    np.testing.assert_array_equal(c1, c0)
    np.testing.assert_array_equal(m1, m0)
    rc, rm, rg = oracle.quant_mask_pack(small, 4)
    assert g1 == f32_bits(rg)
    np.testing.assert_array_equal(c1, rc)
    np.testing.assert_array_equal(m1, rm)


def test_noalloc_pack_rejects_bad_arguments():
    lib = sbl.lib
    P = ctypes.c_void_p(0x10000)
    assert lib.sbl_quant_mask_pack_noalloc(P, 256, 12, 6, P, P, P, None) == -2       # d_in % 8
    assert lib.sbl_quant_mask_pack_noalloc(P, 256, 256, 9, P, P, P, None) == -3      # N > 8
    assert lib.sbl_quant_mask_pack_noalloc(None, 256, 256, 6, P, P, P, None) == -1
