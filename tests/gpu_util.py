"""Helpers shared by the GPU parity tests: host <-> device marshalling of bit
patterns and the comparison rules of the parity bar."""
import numpy as np
import torch


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (host) -> torch.bfloat16 tensor on cuda:0 with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def bits16(t: torch.Tensor) -> np.ndarray:
    """Device 16-bit tensor -> host uint16 bit patterns."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_y_close(y: np.ndarray, y_ref: np.ndarray, acc_ref: np.ndarray, rtol: float = 1e-5):
    """Forward float32 output: |y - y_ref| <= rtol |y_ref| elementwise, and y == 0 where acc == 0."""
    y = y.astype(np.float64)
    err = np.abs(y - y_ref)
    bad = err > rtol * np.abs(y_ref)
    assert not bad.any(), f"{bad.sum()} elements beyond {rtol} relative; worst {err[bad].max()}"
    assert np.all(y[acc_ref == 0] == 0)


# Second bar, from the arithmetic of the GPU backward: every product is exact in
# float32 and the sums are float32, so the error comes from one bf16 rounding
# per element -- of the output (dX in bf16) or of the scaled operand
# bf16(dY a_t / 127) (dW) -- at most 2^-9 relative, about 2^-9 / sqrt(3) = 1.1e-3
# in a row's L2 norm; float32 dX carries only float32 summation error.
ERR_MODEL_BF16 = 4e-3
ERR_MODEL_F32 = 1e-5


def assert_grad_close(got: np.ndarray, ref: np.ndarray, tol: float = 2e-2, rows=None):
    """Backward outputs: per row ||got - ref||_2 <= tol ||ref||_2, and elementwise
    |got - ref| <= tol * max|ref|."""
    got = got.astype(np.float64)
    diff = got - ref
    rn = np.linalg.norm(ref, axis=1)
    dn = np.linalg.norm(diff, axis=1)
    bad_rows = dn > tol * rn + 1e-30
    assert not bad_rows.any(), f"{bad_rows.sum()} rows beyond {tol} relative L2; worst ratio {(dn / np.maximum(rn, 1e-30)).max()}"
    amax = np.abs(ref).max() if ref.size else 0.0
    assert np.abs(diff).max(initial=0.0) <= tol * amax + 1e-30
