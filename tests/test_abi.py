"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, rejects bad arguments before touching the GPU, and its exact
gamma rounding (the device routine, compiled for the host) matches the oracle."""
import ctypes
import os
import re
from fractions import Fraction

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sbl.h")

import sparsity_sparse_bitlinear_amd as sbl  # the built library must load: a missing one fails here
lib = sbl.lib

OK, INVALID, SHAPE, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3, -4
P = ctypes.c_void_p(0x10000)        # a fake, aligned, non-NULL address (never dereferenced)
P_MIS = ctypes.c_void_p(0x10002)    # misaligned
NULL = ctypes.c_void_p(0)


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SBL_API\s+[\w\s\*]+?\b(sbl_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    for n in ("sbl_quant_mask_pack", "sbl_act_quant", "sbl_forward", "sbl_backward"):
        assert n in names


def test_status_strings():
    assert lib.sbl_status_string(0) == b"ok"
    for code in (INVALID, SHAPE, UNSUPPORTED, WORKSPACE, -5):
        assert lib.sbl_status_string(code) not in (b"ok", b"unknown status")
    assert lib.sbl_version().startswith(b"sbl")


def test_quant_mask_pack_validation():
    ws = lib.sbl_quant_mask_pack_workspace_size(256, 256)
    assert ws > 0
    assert lib.sbl_quant_mask_pack_workspace_size(256, 12) == 0
    f = lib.sbl_quant_mask_pack
    assert f(P, 256, 12, 6, P, P, P, P, ws, NULL) == SHAPE          # d_in not a multiple of 8
    assert f(P, 256, 0, 6, P, P, P, P, ws, NULL) == SHAPE
    assert f(P, 0, 256, 6, P, P, P, P, ws, NULL) == SHAPE
    assert f(P, 256, 256, 9, P, P, P, P, ws, NULL) == UNSUPPORTED   # N > 8
    assert f(P, 256, 256, 0, P, P, P, P, ws, NULL) == UNSUPPORTED
    assert f(NULL, 256, 256, 6, P, P, P, P, ws, NULL) == INVALID
    assert f(P, 256, 256, 6, NULL, P, P, P, ws, NULL) == INVALID
    assert f(P, 256, 256, 6, P, P, NULL, P, ws, NULL) == INVALID
    assert f(P_MIS, 256, 256, 6, P, P, P, P, ws, NULL) == INVALID
    assert f(P, 256, 256, 6, P, P, P, P, ws - 1, NULL) == WORKSPACE
    assert f(P, 256, 256, 6, P, P, P, NULL, ws, NULL) == WORKSPACE
    assert b"workspace" in lib.sbl_last_error()
    assert f(P, 1 << 20, 1 << 20, 6, P, P, P, P, ws, NULL) == SHAPE  # above the weight limit


def test_quant_mask_pack_nm_validation():
    ws = lib.sbl_quant_mask_pack_workspace_size(256, 256)
    f = lib.sbl_quant_mask_pack_nm
    assert f(P, 256, 256, 5, 4, 0, P, P, P, P, ws, NULL) == UNSUPPORTED     # 5:4
    assert f(P, 256, 256, 2, 16, 0, P, P, P, P, ws, NULL) == UNSUPPORTED    # M = 16
    assert f(P, 256, 256, 2, 4, 2, P, P, P, P, ws, NULL) == INVALID         # unknown flag bit
    assert f(P, 256, 12, 2, 4, 0, P, P, P, P, ws, NULL) == SHAPE
    assert f(NULL, 256, 256, 2, 4, 1, P, P, P, P, ws, NULL) == INVALID
    assert f(P, 256, 256, 2, 4, 1, P, P, P, P, ws - 1, NULL) == WORKSPACE


def test_quant_mask_pack_batch_validation():
    import sparsity_sparse_bitlinear_amd as sbl
    items = (sbl.PackItem * 3)(sbl.PackItem(0x10000, 256, 256, 0x20000, 0x30000, 0x40000),
                               sbl.PackItem(0x50000, 8, 64, 0x60000, None, 0x70000),
                               sbl.PackItem(0x80000, 11008, 2048, 0x90000, None, 0xA0000))
    ip = ctypes.c_void_p(ctypes.addressof(items))
    ws = lib.sbl_quant_mask_pack_batch_workspace_size(3, ip)
    single = sum(lib.sbl_quant_mask_pack_workspace_size(d_o, d_i) for d_o, d_i in ((256, 256), (8, 64), (11008, 2048)))
    assert ws == single
    f = lib.sbl_quant_mask_pack_batch
    assert f(0, ip, 6, 8, 0, P, ws, NULL) == INVALID
    assert f(17, ip, 6, 8, 0, P, ws, NULL) == INVALID
    assert f(3, NULL, 6, 8, 0, P, ws, NULL) == INVALID
    assert f(3, ip, 5, 4, 0, P, ws, NULL) == UNSUPPORTED
    assert f(3, ip, 6, 8, 4, P, ws, NULL) == INVALID
    assert f(3, ip, 6, 8, 0, P, ws - 1, NULL) == WORKSPACE
    items[1].d_in = 60
    assert f(3, ip, 6, 8, 0, P, ws, NULL) == SHAPE
    items[1].d_in = 64
    items[2].codes = 0x90002                                                  # misaligned
    assert f(3, ip, 6, 8, 0, P, ws, NULL) == INVALID


def test_mask_grad_validation():
    f = lib.sbl_mask_grad
    assert f(NULL, P, 256, 256, NULL) == INVALID
    assert f(P, NULL, 256, 256, NULL) == INVALID
    assert f(P_MIS, P, 256, 256, NULL) == INVALID
    assert f(P, P, 256, 12, NULL) == SHAPE


def test_adamw_repack_validation():
    import sparsity_sparse_bitlinear_amd as sbl
    ws = lib.sbl_adamw_repack_workspace_size(256, 256)
    assert ws > 0 and lib.sbl_adamw_repack_workspace_size(256, 12) == 0
    f = lib.sbl_adamw_repack

    keep = []

    def hp(**kw):
        d = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-5, weight_decay=0.1, grad_scale=1.0, step=1)
        d.update(kw)
        keep.append(sbl.AdamwParams(**d))      # alive until the call returns
        return ctypes.c_void_p(ctypes.addressof(keep[-1]))

    def call(h, n=6, m=8, W=P, mask=P, w=ws, flips=NULL):
        return f(W, P, P, P, 256, 256, h, n, m, NULL, mask, P, P, flips, P, w, NULL)

    assert call(NULL) == INVALID                                    # no parameters
    assert call(hp(step=0)) == INVALID
    assert call(hp(beta1=1.0)) == INVALID
    assert call(hp(eps=0.0)) == INVALID
    assert call(hp(lr=float("nan"))) == INVALID
    assert call(hp(grad_scale=-1.0)) == INVALID
    assert call(hp(), n=5, m=4) == UNSUPPORTED
    assert call(hp(), W=NULL) == INVALID
    assert call(hp(), mask=NULL) == INVALID
    assert call(hp(), W=P_MIS) == INVALID
    assert call(hp(), flips=ctypes.c_void_p(0x10004)) == INVALID  # flips not 8-byte aligned
    assert call(hp(), w=ws - 1) == WORKSPACE
    assert f(P, P, P, P, 256, 12, hp(), 6, 8, NULL, P, P, P, NULL, P, ws, NULL) == SHAPE


def test_rmsnorm_act_quant_validation():
    f = lib.sbl_rmsnorm_act_quant
    assert f(NULL, NULL, 1e-6, 0, 256, NULL, NULL, NULL, NULL) == OK              # T = 0
    assert f(P, NULL, 1e-6, 4, 100, P, P, NULL, NULL) == SHAPE
    assert f(P, NULL, 1e-6, 4, 16392, P, P, NULL, NULL) == UNSUPPORTED
    assert f(P, NULL, -1.0, 4, 256, P, P, NULL, NULL) == INVALID
    assert f(P, NULL, 0.0, 4, 256, P, P, NULL, NULL) == INVALID                  # eps must be > 0
    assert f(P, NULL, float("inf"), 4, 256, P, P, NULL, NULL) == INVALID
    assert f(NULL, NULL, 1e-6, 4, 256, P, P, NULL, NULL) == INVALID
    assert f(P, P_MIS, 1e-6, 4, 256, P, P, NULL, NULL) == INVALID
    assert f(P, NULL, 1e-6, 4, 256, P, P, ctypes.c_void_p(0x10002), NULL) == INVALID  # rstd misaligned


def test_act_quant_validation():
    f = lib.sbl_act_quant
    assert f(NULL, 0, 256, NULL, NULL, NULL) == OK                   # T = 0 is a no-op
    assert f(P, -1, 256, P, P, NULL) == SHAPE
    assert f(P, 4, 100, P, P, NULL) == SHAPE
    assert f(NULL, 4, 256, P, P, NULL) == INVALID
    assert f(P, 4, 256, P_MIS, P, NULL) == INVALID


def test_forward_validation():
    f = lib.sbl_forward
    assert f(NULL, NULL, NULL, NULL, 0, 256, 256, NULL, 0, NULL) == OK
    assert f(P, P, P, P, 4, 256, 256, P, 7, NULL) == INVALID          # bad dtype
    assert f(P, P, P, P, 4, 250, 256, P, 0, NULL) == SHAPE
    assert f(P, P, NULL, P, 4, 256, 256, P, 0, NULL) == INVALID
    assert f(P, P, P, P, 4, 256, 256, P_MIS, 0, NULL) == INVALID


def test_decode_validation():
    f = lib.sbl_decode
    assert f(NULL, NULL, NULL, 0, 256, 256, NULL, 0, NULL) == OK                 # T = 0: no-op
    assert f(P, P, P, 4, 256, 256, P, 7, NULL) == INVALID                       # bad dtype
    assert f(P, P, P, 4, 250, 256, P, 0, NULL) == SHAPE                         # d_in % 8
    assert f(P, P, P, 17, 256, 256, P, 0, NULL) == UNSUPPORTED                  # T > 16
    assert f(P, P, P, 4, 264, 256, P, 0, NULL) == UNSUPPORTED                   # d_in % 64
    assert f(P, P, P, 4, 16448, 256, P, 0, NULL) == UNSUPPORTED                 # T * d_in > 65536
    assert f(P, P, NULL, 4, 256, 256, P, 0, NULL) == INVALID
    assert f(P, P, P_MIS, 4, 256, 256, P, 0, NULL) == INVALID
    assert f(P, P, P, 8, 8192, 256, P, 0, NULL) == UNSUPPORTED                  # tile over 56832 bytes
    s = lib.sbl_decode_supported
    assert s(1, 64) == 1 and s(1, 8192) == 1 and s(5, 8192) == 1 and s(16, 3008) == 1
    assert s(1, 11008) == 1 and s(4, 11008) == 1 and s(6, 8192) == 1 and s(16, 3072) == 1
    assert s(0, 64) == 0 and s(17, 64) == 0 and s(8, 96) == 0 and s(1, 65600) == 0
    assert s(8, 8192) == 0 and s(16, 4096) == 0
    sp = lib.sbl_decode_plane_supported
    assert sp(0, 5, 11008) == 1 and sp(1, 5, 11008) == 0 and sp(1, 4, 11008) == 1 and sp(1, 1, 64) == 0
    assert sp(2, 1, 2048) == 0


def test_decode_multi_validation():
    import sparsity_sparse_bitlinear_amd as sbl
    items = (sbl.DecodeItem * 3)(sbl.DecodeItem(0x10000, 0x20000, 2048, 0x30000),
                                 sbl.DecodeItem(0x40000, 0x50000, 256, 0x60000),
                                 sbl.DecodeItem(0x70000, 0x80000, 40, 0x90000))
    ip = ctypes.c_void_p(ctypes.addressof(items))
    for f, extra in ((lib.sbl_decode_multi, (P,)), (lib.sbl_forward_decode_multi, (P, P))):
        assert f(3, ip, *extra, 0, 256, 0, NULL) == OK                            # T = 0: no-op
        assert f(0, ip, *extra, 4, 256, 0, NULL) == INVALID
        assert f(5, ip, *extra, 4, 256, 0, NULL) == INVALID
        assert f(3, NULL, *extra, 4, 256, 0, NULL) == INVALID
        assert f(3, ip, *extra, 4, 256, 7, NULL) == INVALID                       # bad dtype
        assert f(3, ip, *extra, 4, 250, 0, NULL) == SHAPE                         # d_in % 8
        assert f(3, ip, *extra, 4, 264, 0, NULL) == UNSUPPORTED                   # d_in % 64
        assert f(3, ip, *extra, 65, 256, 0, NULL) == UNSUPPORTED                  # T > 64
        items[1].y = 0x60008                                                      # misaligned y
        assert f(3, ip, *extra, 4, 256, 0, NULL) == INVALID
        items[1].y = 0x60000
        items[2].gamma = None
        assert f(3, ip, *extra, 4, 256, 0, NULL) == INVALID
        items[2].gamma = 0x80000
    assert lib.sbl_decode_multi(3, ip, P, 17, 256, 0, NULL) == UNSUPPORTED        # T > 16 (fused form)
    assert lib.sbl_decode_multi(3, ip, NULL, 4, 256, 0, NULL) == INVALID
    assert lib.sbl_forward_decode_multi(3, ip, P, NULL, 4, 256, 0, NULL) == INVALID


def test_pairs_validation():
    import sparsity_sparse_bitlinear_amd as sbl
    f = lib.sbl_pack_pairs
    assert f(P, 256, 12, P, NULL, NULL) == SHAPE                                # d_in % 8
    assert f(NULL, 256, 256, P, NULL, NULL) == INVALID
    assert f(P, 256, 256, P_MIS, NULL, NULL) == INVALID
    assert f(P, 256, 256, P, ctypes.c_void_p(0x10004), NULL) == INVALID        # bad not 8-byte aligned
    items = (sbl.DecodeItem * 2)(sbl.DecodeItem(0x10000, 0x20000, 2048, 0x30000),
                                 sbl.DecodeItem(0x40000, 0x50000, 256, 0x60000))
    ip = ctypes.c_void_p(ctypes.addressof(items))
    g = lib.sbl_forward_plane_multi
    assert g(1, 2, ip, P, P, NULL, 0, 256, 0, NULL) == OK                      # T = 0
    assert g(2, 2, ip, P, P, NULL, 4, 256, 0, NULL) == INVALID                 # unknown format
    assert g(1, 2, ip, P, P, NULL, 4, 192, 0, NULL) == UNSUPPORTED             # pairs: d_in % 128
    assert g(1, 2, ip, P, P, NULL, 65, 256, 0, NULL) == UNSUPPORTED            # T > 64
    assert g(1, 2, ip, NULL, NULL, P, 17, 256, 0, NULL) == UNSUPPORTED         # fused form: T > 16
    assert g(1, 2, ip, P, P, P, 4, 256, 0, NULL) == INVALID                    # both x_q and x
    assert g(1, 2, ip, P, NULL, NULL, 4, 256, 0, NULL) == INVALID              # x_q without absmax
    assert g(1, 2, ip, NULL, NULL, P_MIS, 4, 256, 0, NULL) == INVALID


def test_sparse24_validation():
    f = lib.sbl_pack_sparse24
    assert f(P, 256, 96, P, NULL, NULL) == SHAPE                               # d_in % 64
    assert f(NULL, 256, 256, P, NULL, NULL) == INVALID
    assert f(P, 256, 256, P_MIS, NULL, NULL) == INVALID
    g = lib.sbl_forward_sparse24
    assert g(NULL, NULL, NULL, NULL, 0, 256, 256, NULL, 0, NULL) == OK           # T = 0
    assert g(P, P, P, P, 4, 192, 256, P, 0, NULL) == UNSUPPORTED                # d_in % 128
    assert g(P, P, P, P, 4, 256, 256, P, 9, NULL) == INVALID
    assert g(P, P, NULL, P, 4, 256, 256, P, 0, NULL) == INVALID


def test_backward_validation():
    f = lib.sbl_backward
    # dX: the transposed 2-bit code plane (d_in rows of d_out rounded up to 64,
    # 2 bits each) when d_out % 8 == 0, else no workspace
    assert lib.sbl_backward_workspace_size(64, 256, 256, 1) == 256 * 256 // 4
    assert lib.sbl_backward_workspace_size(64, 256, 264, 1) == 256 * 320 // 4
    assert lib.sbl_backward_workspace_size(64, 256, 252, 1) == 0
    assert lib.sbl_backward_workspace_size(0, 256, 256, 1) == 0
    assert f(P, P, P, P, P, 4, 256, 256, P, 1, P, 1, NULL, 0, NULL) == WORKSPACE
    assert f(P, P, P, P, P, 4, 256, 256, P, 1, P, 0, NULL, 0, NULL) == INVALID   # no flags
    assert f(P, P, P, P, P, 4, 256, 256, P, 2, P, 4, NULL, 0, NULL) == INVALID   # unknown flag
    assert f(P, P, P, P, P, 4, 256, 256, P, 2, P, 1, NULL, 0, NULL) == INVALID   # I32 dX
    assert f(P, P, P, P, P, 4, 256, 256, NULL, 1, P, 1, NULL, 0, NULL) == INVALID
    assert f(P, P, P, P, P, 4, 256, 256, P, 1, NULL, 2, NULL, 0, NULL) == INVALID
    # a shape that needs split-K workspace
    need = lib.sbl_backward_workspace_size(32768, 2048, 256, 2)
    assert need > 0
    assert f(P, P, P, P, P, 32768, 2048, 256, P, 1, P, 2, NULL, 0, NULL) == WORKSPACE
    assert f(P, P, P, P, P, 32768, 2048, 256, P, 1, P, 2, P, need - 16, NULL) == WORKSPACE
    assert f(NULL, NULL, NULL, NULL, NULL, 0, 256, 256, NULL, 1, NULL, 1, NULL, 0, NULL) == OK


@pytest.mark.parametrize("T,d_in,d_out,planes", [
    (32768, 2048, 11008, 4),  # 344 tiles: 256 over all of K into dW, 88 in 5 K ranges (planes 1-4)
    (32768, 11008, 2048, 4),  # the same plan for the transposed shape
    (4096, 4096, 4608, 5),    # 288 tiles: 32 tail tiles in 6 ranges
    (2000, 4112, 4504, 2),    # 306 tiles, ragged in both dimensions: 50 tail tiles in 3 ranges
    (32768, 2048, 2048, 4),   # 64 tiles: a uniform 4-way split fills the 256 CUs
    (32768, 2048, 256, 32),   # 8 tiles: 32-way split
    (8192, 1536, 8960, 0),    # 210 tiles: one round without a split
    (8192, 8960, 1536, 0),
])
def test_backward_dw_workspace_plan(T, d_in, d_out, planes):
    # dW alone on the int8 form: the scaled dY^T (run-major bf16, 256-byte aligned) and
    # the split-K planes of float32 [d_out][d_in] that the plan needs
    T8 = (T + 7) // 8 * 8
    dyt = (d_out * T8 * 2 + 255) // 256 * 256
    assert lib.sbl_backward_workspace_size(T, d_in, d_out, 2) == dyt + planes * d_out * d_in * 4


def _round_mean_lib(S: int, count: int) -> float:
    words = (ctypes.c_uint32 * 10)(*[(S >> (32 * i)) & 0xFFFFFFFF for i in range(10)])
    out = ctypes.c_float()
    assert lib.sbl_test_round_mean(words, 10, count, ctypes.byref(out)) == OK
    return out.value


def test_gamma_rounding_routine_matches_oracle():
    g = np.random.default_rng(21)
    cases = []
    for _ in range(3000):
        count = int(g.integers(1, 1 << 36))
        bits = int(g.integers(1, 300))
        S = int(g.integers(0, 1 << 62)) << max(0, bits - 62) | int(g.integers(0, 1 << 20))
        S &= (1 << 300) - 1
        cases.append((S, count))
    # subnormal results, ties, exact values
    for count in (1, 3, 8, 65536, 12345, (1 << 36) - 1):
        for S in (1, 2, 3, 7, 1 << 23, (1 << 24) + 1, 3 << 130, (1 << 40) - 1, 123456789 << 200):
            cases.append((S, count))
    for S, count in cases:
        want = oracle.round_rational_to_f32(S, count << 133)
        got = _round_mean_lib(S, count)
        assert np.float32(got) == np.float32(want), (S, count, got, want)


def test_gamma_rounding_routine_on_real_sums():
    from sbl_inputs import weight
    for i, (d_out, d_in) in enumerate(((256, 256), (17, 24), (1536, 1536))):
        W = weight(5, i, d_out, d_in)
        S = oracle.abs_sum_exact(W)
        assert np.float32(_round_mean_lib(S, W.size)) == oracle.gamma_f32(W)
