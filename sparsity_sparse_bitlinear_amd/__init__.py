"""Sparse-BitLinear for AMD MI355X (gfx950): Python binding of ``libsbl.so``.

Thin argument marshalling over the C ABI declared in ``include/sbl.h``; every
step of the operator runs in the library's HIP kernels.  PyTorch supplies
device memory and the current HIP stream only.  There is no fallback: if the
library is missing or no GPU is present, calls raise.

Functions mirror the C entry points:

* ``quant_mask_pack(W, n_keep)`` -> ``(codes, mask, gamma)``
* ``act_quant(x)`` -> ``(x_q, absmax)``
* ``forward(codes, gamma, x_q, absmax, d_out, out_dtype)`` -> ``y``
* ``backward(codes, gamma, x_q, absmax, dY, ...)`` -> ``(dX, dW)``

``SparseBitLinearFunction`` wraps them as a ``torch.autograd.Function``
(quantize/mask/pack every call, Dual-STE backward).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "LIB_PATH", "lib", "SblError", "quant_mask_pack", "act_quant", "forward", "backward",
    "quant_workspace_size", "backward_workspace_size", "SparseBitLinearFunction", "sparse_bitlinear",
    "F32", "BF16", "I32", "BWD_DX", "BWD_DW",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsbl.so")

F32, BF16, I32 = 0, 1, 2
BWD_DX, BWD_DW = 1, 2
MASK_FROM_QUANTIZED = 1

_c_i64 = ctypes.c_int64
_c_ptr = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size = ctypes.c_size_t

_SIGNATURES = {
    "sbl_quant_mask_pack_workspace_size": (_c_size, [_c_i64, _c_i64]),
    "sbl_quant_mask_pack": (_c_int, [_c_ptr, _c_i64, _c_i64, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr]),
    "sbl_quant_mask_pack_nm": (_c_int, [_c_ptr, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                        _c_size, _c_ptr]),
    "sbl_quant_mask_pack_noalloc": (_c_int, [_c_ptr, _c_i64, _c_i64, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "sbl_quant_mask_pack_noalloc_scratch_bytes": (_c_size, []),
    "sbl_mask_grad": (_c_int, [_c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr]),
    "sbl_quant_mask_pack_batch_workspace_size": (_c_size, [_c_int, ctypes.c_void_p]),
    "sbl_quant_mask_pack_batch": (_c_int, [_c_int, ctypes.c_void_p, _c_int, _c_int, _c_int, _c_ptr, _c_size, _c_ptr]),
    "sbl_adamw_repack_workspace_size": (_c_size, [_c_i64, _c_i64]),
    "sbl_adamw_repack": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, ctypes.c_void_p, _c_int, _c_int,
                                  _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr]),
    "sbl_act_quant": (_c_int, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr]),
    "sbl_forward": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_ptr, _c_int, _c_ptr]),
    "sbl_rmsnorm_act_quant": (_c_int, [_c_ptr, _c_ptr, ctypes.c_float, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr,
                                       _c_ptr]),
    "sbl_pack_sparse24": (_c_int, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr]),
    "sbl_pack_pairs": (_c_int, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr]),
    "sbl_decode_plane_supported": (_c_int, [_c_int, _c_i64, _c_i64]),
    "sbl_forward_plane_multi": (_c_int, [_c_int, _c_int, ctypes.c_void_p, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64,
                                         _c_int, _c_ptr]),
    "sbl_forward_sparse24": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_ptr, _c_int, _c_ptr]),
    "sbl_decode": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_ptr, _c_int, _c_ptr]),
    "sbl_decode_supported": (_c_int, [_c_i64, _c_i64]),
    "sbl_decode_multi": (_c_int, [_c_int, ctypes.c_void_p, _c_ptr, _c_i64, _c_i64, _c_int, _c_ptr]),
    "sbl_forward_decode_multi": (_c_int, [_c_int, ctypes.c_void_p, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_int, _c_ptr]),
    "sbl_backward_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i64, _c_int]),
    "sbl_backward": (_c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_ptr, _c_int,
                              _c_ptr, _c_int, _c_ptr, _c_size, _c_ptr]),
    "sbl_peak_mfma": (_c_int, [_c_int, _c_i64, _c_int, _c_ptr, _c_ptr]),
    "sbl_peak_read": (_c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr]),
    "sbl_status_string": (ctypes.c_char_p, [_c_int]),
    "sbl_last_error": (ctypes.c_char_p, []),
    "sbl_version": (ctypes.c_char_p, []),
    "sbl_test_round_mean": (_c_int, [ctypes.POINTER(ctypes.c_uint32), _c_int, _c_i64, ctypes.POINTER(ctypes.c_float)]),
}


class PackItem(ctypes.Structure):
    """sbl_pack_item (host struct)."""
    _fields_ = [("W", ctypes.c_void_p), ("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("gamma", ctypes.c_void_p)]


PACK_BATCH_MAX = 16


class DecodeItem(ctypes.Structure):
    """sbl_decode_item (host struct)."""
    _fields_ = [("codes", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("d_out", ctypes.c_int64),
                ("y", ctypes.c_void_p)]


DECODE_MULTI_MAX = 4


class AdamwParams(ctypes.Structure):
    """sbl_adamw_params (host struct)."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("grad_scale", ctypes.c_float),
                ("step", ctypes.c_int64)]


class SblError(RuntimeError):
    """A libsbl call returned a non-zero status."""

    def __init__(self, status: int, func: str):
        self.status = status
        msg = lib.sbl_status_string(status).decode()
        detail = lib.sbl_last_error().decode()
        super().__init__(f"{func} failed: {msg} ({status}): {detail}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python sparsity_sparse_bitlinear_amd/build.py` "
            "(hipcc for gfx950).  There is no fallback implementation.")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


def _check(status: int, func: str) -> None:
    if status != 0:
        raise SblError(status, func)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _typed(t: torch.Tensor, name: str, dtypes, ndim: int) -> None:
    """A contiguous GPU tensor of one of ``dtypes`` with ``ndim`` dimensions."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    _dev(t, name)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def _gamma_ok(gamma: torch.Tensor, name: str = "gamma") -> None:
    _typed(gamma, name, (torch.float32,), 1)
    if gamma.numel() < 1:
        raise ValueError(f"{name} must hold one float32")


def _act_operands(x_q: torch.Tensor, absmax: torch.Tensor):
    """x_q int8 [T, d_in] and absmax float32 [T] on one device; returns (T, d_in)."""
    _typed(x_q, "x_q", (torch.int8,), 2)
    _typed(absmax, "absmax", (torch.float32,), 1)
    T, d_in = x_q.shape
    if absmax.numel() != T:
        raise ValueError(f"absmax has {absmax.numel()} entries, expected T = {T}")
    if absmax.device != x_q.device:
        raise ValueError("x_q and absmax must be on one device")
    return T, d_in


def _code_operands(codes: torch.Tensor, gamma: torch.Tensor, d_in: int, dev, name: str = "codes",
                   plane: int = 0):
    """codes int16 [d_out, d_in/8] (or, for the pair plane, uint8 [d_out, d_in/8]) and gamma float32 [>= 1]
    on ``dev``; returns d_out."""
    _typed(codes, name, (torch.uint8,) if plane == PLANE_PAIRS else (torch.int16, torch.uint16), 2)
    _gamma_ok(gamma)
    d_out, G = codes.shape
    if G * 8 != d_in:
        raise ValueError(f"{name} [{d_out}, {G}] do not match d_in = {d_in}")
    if codes.device != dev or gamma.device != dev:
        raise ValueError(f"{name} and gamma must be on the device of the activations")
    return d_out


def _out(t: torch.Tensor, shape, dtypes, device, name: str) -> torch.Tensor:
    """Check a caller-provided output buffer: the kernels write exactly ``shape`` elements of one of ``dtypes``."""
    _dev(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _as_bits16(t: torch.Tensor, name: str) -> torch.Tensor:
    _dev(t, name)
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bfloat16 values (bfloat16, or int16/uint16 bit patterns)")
    return t


def quant_workspace_size(d_out: int, d_in: int) -> int:
    return int(lib.sbl_quant_mask_pack_workspace_size(d_out, d_in))


def backward_workspace_size(T: int, d_in: int, d_out: int, flags: int = BWD_DX | BWD_DW) -> int:
    return int(lib.sbl_backward_workspace_size(T, d_in, d_out, flags))


def quant_mask_pack(W: torch.Tensor, n_keep: int = 6, *, m: int = 8, from_quantized: bool = False,
                    codes: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                    gamma: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    want_mask: bool = True, stream=None):
    """gamma, N:M mask and 2-bit ternary code plane of the bf16 master weight ``W`` [d_out, d_in].

    ``m`` is 8 (N:8) or 4 (N:4, e.g. 2:4); ``from_quantized`` selects the mask-from-quantized-weight
    ablation.  Returns ``(codes int16 [d_out, d_in/8] (uint16 bit patterns), mask uint8
    [d_out, d_in/8] or None, gamma float32 [1])``; all on W's device.
    """
    _as_bits16(W, "W")
    d_out, d_in = W.shape
    dev = W.device
    if codes is None:
        codes = torch.empty((d_out, d_in // 8), dtype=torch.int16, device=dev)
    _out(codes, (d_out, d_in // 8), (torch.int16, torch.uint16), dev, "codes")
    if mask is None and want_mask:
        mask = torch.empty((d_out, d_in // 8), dtype=torch.uint8, device=dev)
    if mask is not None:
        _out(mask, (d_out, d_in // 8), (torch.uint8,), dev, "mask")
    if gamma is None:
        gamma = torch.empty((1,), dtype=torch.float32, device=dev)
    _out(gamma, (1,), (torch.float32,), dev, "gamma")
    need = quant_workspace_size(d_out, d_in)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _out(workspace, (workspace.numel(),), (torch.uint8,), dev, "workspace")
    flags = MASK_FROM_QUANTIZED if from_quantized else 0
    _check(lib.sbl_quant_mask_pack_nm(_ptr(W), d_out, d_in, int(n_keep), int(m), flags, _ptr(codes), _ptr(mask),
                                      _ptr(gamma), _ptr(workspace), workspace.numel(), _stream(stream)),
           "sbl_quant_mask_pack_nm")
    return codes, mask, gamma


def adamw_repack(W: torch.Tensor, dW: torch.Tensor, m: torch.Tensor, v: torch.Tensor, *, step: int, lr: float,
                 beta1: float = 0.9, beta2: float = 0.95, eps: float = 1e-5, weight_decay: float = 0.1,
                 grad_scale: float = 1.0, n_keep: int = 6, m_group: int = 8,
                 mask_prev: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                 codes: Optional[torch.Tensor] = None, gamma: Optional[torch.Tensor] = None,
                 flips: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """AdamW step on the bf16 master ``W`` (in place, with ``m``, ``v``) and the next step's packing.

    Returns ``(codes, mask, gamma, flips)``; ``flips`` (int64 [1]) is None without ``mask_prev``.
    """
    _as_bits16(W, "W")
    d_out, d_in = W.shape
    dev = W.device
    for t, n in ((dW, "dW"), (m, "m"), (v, "v")):
        _out(t, (d_out, d_in), (torch.float32,), dev, n)
    if codes is None:
        codes = torch.empty((d_out, d_in // 8), dtype=torch.int16, device=dev)
    _out(codes, (d_out, d_in // 8), (torch.int16, torch.uint16), dev, "codes")
    if mask is None:
        mask = torch.empty((d_out, d_in // 8), dtype=torch.uint8, device=dev)
    _out(mask, (d_out, d_in // 8), (torch.uint8,), dev, "mask")
    if mask_prev is not None:
        _out(mask_prev, (d_out, d_in // 8), (torch.uint8,), dev, "mask_prev")
        if flips is None:
            flips = torch.zeros((1,), dtype=torch.int64, device=dev)
        _out(flips, (1,), (torch.int64,), dev, "flips")
    if gamma is None:
        gamma = torch.empty((1,), dtype=torch.float32, device=dev)
    _out(gamma, (1,), (torch.float32,), dev, "gamma")
    need = lib.sbl_adamw_repack_workspace_size(d_out, d_in)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _out(workspace, (workspace.numel(),), (torch.uint8,), dev, "workspace")
    hp = AdamwParams(lr, beta1, beta2, eps, weight_decay, grad_scale, int(step))
    _check(lib.sbl_adamw_repack(_ptr(W), _ptr(dW), _ptr(m), _ptr(v), d_out, d_in,
                                ctypes.c_void_p(ctypes.addressof(hp)), int(n_keep), int(m_group), _ptr(mask_prev), _ptr(mask),
                                _ptr(codes), _ptr(gamma), _ptr(flips if mask_prev is not None else None),
                                _ptr(workspace), workspace.numel(), _stream(stream)), "sbl_adamw_repack")
    return codes, mask, gamma, (flips if mask_prev is not None else None)


def quant_mask_pack_batch(Ws, n_keep: int = 6, *, m: int = 8, from_quantized: bool = False, codes=None,
                          masks=None, gammas=None, workspace: Optional[torch.Tensor] = None, want_mask: bool = True,
                          stream=None):
    """``quant_mask_pack`` for up to 16 matrices in three launches in all.  Returns lists
    ``(codes, masks, gammas)`` in the order of ``Ws``; the results equal one call per matrix."""
    Ws = list(Ws)
    n = len(Ws)
    if not 1 <= n <= PACK_BATCH_MAX:
        raise ValueError(f"1..{PACK_BATCH_MAX} matrices per batch, got {n}")
    codes = list(codes) if codes is not None else [None] * n
    masks = list(masks) if masks is not None else [None] * n
    gammas = list(gammas) if gammas is not None else [None] * n
    items = (PackItem * n)()
    for i, W in enumerate(Ws):
        _as_bits16(W, f"W[{i}]")
        d_out, d_in = W.shape
        dev = W.device
        if codes[i] is None:
            codes[i] = torch.empty((d_out, d_in // 8), dtype=torch.int16, device=dev)
        _out(codes[i], (d_out, d_in // 8), (torch.int16, torch.uint16), dev, f"codes[{i}]")
        if masks[i] is None and want_mask:
            masks[i] = torch.empty((d_out, d_in // 8), dtype=torch.uint8, device=dev)
        if masks[i] is not None:
            _out(masks[i], (d_out, d_in // 8), (torch.uint8,), dev, f"mask[{i}]")
        if gammas[i] is None:
            gammas[i] = torch.empty((1,), dtype=torch.float32, device=dev)
        _out(gammas[i], (1,), (torch.float32,), dev, f"gamma[{i}]")
        items[i] = PackItem(W.data_ptr(), d_out, d_in, codes[i].data_ptr(),
                            masks[i].data_ptr() if masks[i] is not None else None, gammas[i].data_ptr())
    need = lib.sbl_quant_mask_pack_batch_workspace_size(n, ctypes.c_void_p(ctypes.addressof(items)))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=Ws[0].device)
    _out(workspace, (workspace.numel(),), (torch.uint8,), Ws[0].device, "workspace")
    flags = MASK_FROM_QUANTIZED if from_quantized else 0
    _check(lib.sbl_quant_mask_pack_batch(n, ctypes.c_void_p(ctypes.addressof(items)), int(n_keep), int(m), flags,
                                         _ptr(workspace), workspace.numel(), _stream(stream)),
           "sbl_quant_mask_pack_batch")
    return codes, masks, gammas


def quant_batch_workspace_size(shapes) -> int:
    """Workspace bytes of ``quant_mask_pack_batch`` for [(d_out, d_in), ...]."""
    shapes = list(shapes)
    items = (PackItem * len(shapes))()
    for i, (d_out, d_in) in enumerate(shapes):
        items[i] = PackItem(None, d_out, d_in, None, None, None)
    return int(lib.sbl_quant_mask_pack_batch_workspace_size(len(shapes), ctypes.c_void_p(ctypes.addressof(items))))


def mask_grad(dW: torch.Tensor, mask: torch.Tensor, *, stream=None) -> torch.Tensor:
    """Mask-without-grad ablation, in place: dW = +0 where the mask plane's bit is clear."""
    _out(dW, tuple(dW.shape), (torch.float32,), dW.device, "dW")
    d_out, d_in = dW.shape
    _out(mask, (d_out, d_in // 8), (torch.uint8,), dW.device, "mask")
    _check(lib.sbl_mask_grad(_ptr(dW), _ptr(mask), d_out, d_in, _stream(stream)), "sbl_mask_grad")
    return dW


def act_quant(x: torch.Tensor, *, x_q: Optional[torch.Tensor] = None, absmax: Optional[torch.Tensor] = None,
              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-token absmax int8 quantization of bf16 ``x`` [T, d_in] -> (x_q int8, absmax float32 [T])."""
    _as_bits16(x, "x")
    T, d_in = x.shape
    if x_q is None:
        x_q = torch.empty((T, d_in), dtype=torch.int8, device=x.device)
    if absmax is None:
        absmax = torch.empty((T,), dtype=torch.float32, device=x.device)
    _out(x_q, (T, d_in), (torch.int8,), x.device, "x_q")
    _out(absmax, (T,), (torch.float32,), x.device, "absmax")
    _check(lib.sbl_act_quant(_ptr(x), T, d_in, _ptr(x_q), _ptr(absmax), _stream(stream)), "sbl_act_quant")
    return x_q, absmax


def rmsnorm_act_quant(x: torch.Tensor, g: Optional[torch.Tensor] = None, eps: float = 1e-6, *,
                      x_q: Optional[torch.Tensor] = None, absmax: Optional[torch.Tensor] = None,
                      rstd: Optional[torch.Tensor] = None, with_rstd: bool = False, stream=None):
    """Q_a(RMSNorm(x)) in one pass: ``(x_q int8 [T, d_in], absmax float32 [T])``, plus ``rstd`` float32 [T]
    (the per-row 1/sqrt(mean square + eps)) as a third item when ``with_rstd`` or ``rstd`` is given;
    ``g`` bf16 [d_in] or None."""
    _as_bits16(x, "x")
    T, d_in = x.shape
    if g is not None:
        _as_bits16(g, "g")
        if tuple(g.shape) != (d_in,):
            raise ValueError(f"g has shape {tuple(g.shape)}, expected ({d_in},)")
        if g.device != x.device:
            raise ValueError("g must be on the device of x")
    if x_q is None:
        x_q = torch.empty((T, d_in), dtype=torch.int8, device=x.device)
    if absmax is None:
        absmax = torch.empty((T,), dtype=torch.float32, device=x.device)
    want_rstd = with_rstd or rstd is not None
    if want_rstd and rstd is None:
        rstd = torch.empty((T,), dtype=torch.float32, device=x.device)
    _out(x_q, (T, d_in), (torch.int8,), x.device, "x_q")
    _out(absmax, (T,), (torch.float32,), x.device, "absmax")
    if want_rstd:
        _out(rstd, (T,), (torch.float32,), x.device, "rstd")
    _check(lib.sbl_rmsnorm_act_quant(_ptr(x), _ptr(g), float(eps), T, d_in, _ptr(x_q), _ptr(absmax),
                                     _ptr(rstd), _stream(stream)), "sbl_rmsnorm_act_quant")
    return (x_q, absmax, rstd) if want_rstd else (x_q, absmax)


_OUT_TORCH = {F32: torch.float32, BF16: torch.bfloat16, I32: torch.int32}

PLANE_CODES, PLANE_PAIRS = 0, 1


def pack_pairs(codes: torch.Tensor, *, plane: Optional[torch.Tensor] = None, stream=None):
    """Pair plane (one byte per group of 8) of a code plane whose mask keeps at most 2 of 8:
    ``(plane uint8 [d_out, d_in/8], bad int64 [1])``; ``bad`` counts groups with more than 2 non-zeros."""
    _typed(codes, "codes", (torch.int16, torch.uint16), 2)
    d_out, G = codes.shape
    if plane is None:
        plane = torch.empty((d_out, G), dtype=torch.uint8, device=codes.device)
    _out(plane, (d_out, G), (torch.uint8,), codes.device, "plane")
    bad = torch.zeros((1,), dtype=torch.int64, device=codes.device)
    _check(lib.sbl_pack_pairs(_ptr(codes), d_out, 8 * G, _ptr(plane), _ptr(bad), _stream(stream)), "sbl_pack_pairs")
    return plane, bad


def decode_plane_supported(plane_format: int, T: int, d_in: int) -> bool:
    """True if ``forward_plane_multi`` takes ``x`` (the quantization fused in) at this (T, d_in)."""
    return bool(lib.sbl_decode_plane_supported(int(plane_format), int(T), int(d_in)))


def forward_plane_multi(plane_format: int, mats, *, x_q: Optional[torch.Tensor] = None,
                        absmax: Optional[torch.Tensor] = None, x: Optional[torch.Tensor] = None,
                        out_dtype: int = F32, ys=None, stream=None):
    """Decode-size forward (T <= 64) of up to 4 matrices sharing one input, on the code plane
    (``PLANE_CODES``) or the pair plane (``PLANE_PAIRS``, ``mats`` holding ``(plane, gamma)``); with ``x``
    (bf16) the activation quantization runs in the same launch, else ``x_q`` and ``absmax`` are given."""
    if plane_format not in (PLANE_CODES, PLANE_PAIRS):
        raise ValueError(f"unknown plane format {plane_format}")
    if (x is None) == (x_q is None):
        raise ValueError("give either x (bf16) or x_q with absmax")
    if x is not None:
        _typed(x, "x", (torch.bfloat16,), 2)
        T, d_in = x.shape
        dev = x.device
    else:
        T, d_in = _act_operands(x_q, absmax)
        dev = x_q.device
    items, ys = _decode_items(mats, T, d_in, out_dtype, ys, dev, plane=plane_format)
    _check(lib.sbl_forward_plane_multi(int(plane_format), len(ys), ctypes.c_void_p(ctypes.addressof(items)),
                                       _ptr(x_q), _ptr(absmax), _ptr(x), T, d_in, int(out_dtype), _stream(stream)),
           "sbl_forward_plane_multi")
    return ys


def pack_sparse24(codes: torch.Tensor, *, plane: Optional[torch.Tensor] = None, stream=None):
    """Kept-only 2:4 plane of a 2:8 / 2:4 code plane: ``(plane uint8 [d_out, d_in/64, 16], bad int64 [1])``;
    ``bad`` counts groups of 4 with more than 2 non-zeros (0 for 2:8 and 2:4 masks)."""
    _dev(codes, "codes")
    d_out, G = codes.shape
    d_in = 8 * G
    if plane is None:
        plane = torch.empty((d_out, d_in // 64, 16), dtype=torch.uint8, device=codes.device)
    _out(plane, (d_out, d_in // 64, 16), (torch.uint8,), codes.device, "plane")
    bad = torch.zeros((1,), dtype=torch.int64, device=codes.device)
    _check(lib.sbl_pack_sparse24(_ptr(codes), d_out, d_in, _ptr(plane), _ptr(bad), _stream(stream)),
           "sbl_pack_sparse24")
    return plane, bad


def forward_sparse24(plane: torch.Tensor, gamma: torch.Tensor, x_q: torch.Tensor, absmax: torch.Tensor, *,
                     out_dtype: int = F32, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``forward`` on the kept-only 2:4 plane (sparse matrix instruction); same result as ``forward``."""
    T, d_in = _act_operands(x_q, absmax)
    _typed(plane, "plane", (torch.uint8,), 3)
    _gamma_ok(gamma)
    d_out, steps, sixteen = plane.shape
    if steps * 64 != d_in or sixteen != 16:
        raise ValueError(f"plane {tuple(plane.shape)} does not match x_q [{T}, {d_in}]")
    if plane.device != x_q.device or gamma.device != x_q.device:
        raise ValueError("plane and gamma must be on the device of x_q")
    if out_dtype not in _OUT_TORCH:
        raise ValueError(f"unknown out_dtype {out_dtype}")
    if y is None:
        y = torch.empty((T, d_out), dtype=_OUT_TORCH[out_dtype], device=x_q.device)
    _out(y, (T, d_out), (_OUT_TORCH[out_dtype],), x_q.device, "y")
    _check(lib.sbl_forward_sparse24(_ptr(plane), _ptr(gamma), _ptr(x_q), _ptr(absmax), T, d_in, d_out, _ptr(y),
                                    int(out_dtype), _stream(stream)), "sbl_forward_sparse24")
    return y


def forward(codes: torch.Tensor, gamma: torch.Tensor, x_q: torch.Tensor, absmax: torch.Tensor, *,
            out_dtype: int = F32, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y[t, o] = (sum_i x_q[t, i] W_eff[o, i]) * gamma * absmax[t] / 127  (or the raw int32 sums)."""
    T, d_in = _act_operands(x_q, absmax)
    d_out = _code_operands(codes, gamma, d_in, x_q.device)
    if out_dtype not in _OUT_TORCH:
        raise ValueError(f"unknown out_dtype {out_dtype}")
    if y is None:
        y = torch.empty((T, d_out), dtype=_OUT_TORCH[out_dtype], device=x_q.device)
    _out(y, (T, d_out), (_OUT_TORCH[out_dtype],), x_q.device, "y")
    _check(lib.sbl_forward(_ptr(codes), _ptr(gamma), _ptr(x_q), _ptr(absmax), T, d_in, d_out, _ptr(y),
                           int(out_dtype), _stream(stream)), "sbl_forward")
    return y


def decode_supported(T: int, d_in: int) -> bool:
    """True if ``decode`` takes this token count and input width."""
    return bool(lib.sbl_decode_supported(int(T), int(d_in)))


def decode(codes: torch.Tensor, gamma: torch.Tensor, x: torch.Tensor, *, out_dtype: int = F32,
           y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """act_quant + forward in one launch for decode-sized T (see ``decode_supported``): same bits as the two calls."""
    _typed(x, "x", (torch.bfloat16,), 2)
    T, d_in = x.shape
    d_out = _code_operands(codes, gamma, d_in, x.device)
    if out_dtype not in _OUT_TORCH:
        raise ValueError(f"unknown out_dtype {out_dtype}")
    if y is None:
        y = torch.empty((T, d_out), dtype=_OUT_TORCH[out_dtype], device=x.device)
    _out(y, (T, d_out), (_OUT_TORCH[out_dtype],), x.device, "y")
    _check(lib.sbl_decode(_ptr(codes), _ptr(gamma), _ptr(x), T, d_in, d_out, _ptr(y), int(out_dtype),
                          _stream(stream)), "sbl_decode")
    return y


def _decode_items(mats, T: int, d_in: int, out_dtype: int, ys, dev, plane: int = 0):
    mats = list(mats)
    n = len(mats)
    if not 1 <= n <= DECODE_MULTI_MAX:
        raise ValueError(f"1..{DECODE_MULTI_MAX} matrices per call, got {n}")
    if out_dtype not in _OUT_TORCH:
        raise ValueError(f"unknown out_dtype {out_dtype}")
    ys = list(ys) if ys is not None else [None] * n
    items = (DecodeItem * n)()
    for i, (codes, gamma) in enumerate(mats):
        d_out = _code_operands(codes, gamma, d_in, dev, name=f"codes[{i}]", plane=plane)
        if ys[i] is None:
            ys[i] = torch.empty((T, d_out), dtype=_OUT_TORCH[out_dtype], device=dev)
        _out(ys[i], (T, d_out), (_OUT_TORCH[out_dtype],), dev, f"y[{i}]")
        items[i] = DecodeItem(codes.data_ptr(), gamma.data_ptr(), d_out, ys[i].data_ptr())
    return items, ys


def decode_multi(mats, x: torch.Tensor, *, out_dtype: int = F32, ys=None, stream=None):
    """``decode`` of up to 4 matrices that read the same ``x`` (a layer's q, k, v or gate, up), in one
    launch.  ``mats`` is a list of ``(codes, gamma)``; returns the list of outputs, each bit-identical to
    ``decode`` of that matrix alone."""
    _typed(x, "x", (torch.bfloat16,), 2)
    T, d_in = x.shape
    items, ys = _decode_items(mats, T, d_in, out_dtype, ys, x.device)
    _check(lib.sbl_decode_multi(len(ys), ctypes.c_void_p(ctypes.addressof(items)), _ptr(x), T, d_in,
                                int(out_dtype), _stream(stream)), "sbl_decode_multi")
    return ys


def forward_decode_multi(mats, x_q: torch.Tensor, absmax: torch.Tensor, *, out_dtype: int = F32, ys=None,
                         stream=None):
    """``forward`` of up to 4 matrices that read the same ``x_q`` at decode sizes (T <= 64), in one launch;
    each output bit-identical to ``forward`` of that matrix alone."""
    T, d_in = _act_operands(x_q, absmax)
    items, ys = _decode_items(mats, T, d_in, out_dtype, ys, x_q.device)
    _check(lib.sbl_forward_decode_multi(len(ys), ctypes.c_void_p(ctypes.addressof(items)), _ptr(x_q),
                                        _ptr(absmax), T, d_in, int(out_dtype), _stream(stream)),
           "sbl_forward_decode_multi")
    return ys


def backward(codes: torch.Tensor, gamma: torch.Tensor, x_q: torch.Tensor, absmax: torch.Tensor,
             dY: torch.Tensor, *, need_dx: bool = True, need_dw: bool = True, dx_dtype: int = BF16,
             dX: Optional[torch.Tensor] = None, dW: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, stream=None):
    """Dual-STE gradients: dX = gamma dY W_eff [T, d_in], dW = dY^T x~ [d_out, d_in] (float32)."""
    _as_bits16(dY, "dY")
    T, d_in = _act_operands(x_q, absmax)
    d_out = _code_operands(codes, gamma, d_in, x_q.device)
    flags = (BWD_DX if need_dx else 0) | (BWD_DW if need_dw else 0)
    if dY.device != x_q.device:
        raise ValueError("dY must be on the device of x_q")
    if tuple(dY.shape) != (T, d_out):
        raise ValueError(f"dY has shape {tuple(dY.shape)}, expected {(T, d_out)}")
    if dx_dtype not in (F32, BF16):
        raise ValueError(f"dx_dtype must be F32 or BF16, got {dx_dtype}")
    if need_dx:
        if dX is None:
            dX = torch.empty((T, d_in), dtype=_OUT_TORCH[dx_dtype], device=dY.device)
        _out(dX, (T, d_in), (_OUT_TORCH[dx_dtype],), dY.device, "dX")
    if need_dw:
        if dW is None:
            dW = torch.empty((d_out, d_in), dtype=torch.float32, device=dY.device)
        _out(dW, (d_out, d_in), (torch.float32,), dY.device, "dW")
    need = backward_workspace_size(T, d_in, d_out, flags)
    if need and workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dY.device)
    if workspace is not None:
        _out(workspace, (workspace.numel(),), (torch.uint8,), dY.device, "workspace")
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib.sbl_backward(_ptr(codes), _ptr(gamma), _ptr(x_q), _ptr(absmax), _ptr(dY), T, d_in, d_out,
                            _ptr(dX if need_dx else None), int(dx_dtype), _ptr(dW if need_dw else None), flags,
                            _ptr(workspace), ws_bytes, _stream(stream)), "sbl_backward")
    return (dX if need_dx else None), (dW if need_dw else None)


class SparseBitLinearFunction(torch.autograd.Function):
    """y = Sparse-BitLinear(x; W) with the mask and codes recomputed from W on every call.

    x: bf16 [T, d_in]; W: bf16 master weight [d_out, d_in].  Returns y float32 [T, d_out].
    Backward (Dual STE): grad_x bf16 [T, d_in], grad_W float32 [d_out, d_in] (dense).
    """

    @staticmethod
    def forward(ctx, x: torch.Tensor, W: torch.Tensor, n_keep: int = 6):
        codes, _, gamma = quant_mask_pack(W.contiguous(), n_keep, want_mask=False)
        x_q, absmax = act_quant(x.contiguous())
        y = forward(codes, gamma, x_q, absmax, out_dtype=F32)
        ctx.save_for_backward(codes, gamma, x_q, absmax)
        return y

    @staticmethod
    def backward(ctx, grad_y: torch.Tensor):
        codes, gamma, x_q, absmax = ctx.saved_tensors
        dY = grad_y.to(torch.bfloat16).contiguous()
        dX, dW = backward(codes, gamma, x_q, absmax, dY, need_dx=ctx.needs_input_grad[0],
                          need_dw=ctx.needs_input_grad[1], dx_dtype=BF16)
        return dX, dW, None


def sparse_bitlinear(x: torch.Tensor, W: torch.Tensor, n_keep: int = 6) -> torch.Tensor:
    return SparseBitLinearFunction.apply(x, W, n_keep)
