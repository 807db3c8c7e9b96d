"""Seeded synthetic inputs for the Sparse-BitLinear operator.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds NO arithmetic of the method itself: it only draws random
numbers, rounds them to bfloat16 bit patterns, and builds hand-shaped edge-case
tensors.  Both sides of every parity comparison receive the same bit patterns.

Stream layout: ``numpy.random.Generator(PCG64(SeedSequence([cfg, mat, kind, ...])))``
with ``kind`` 0 = W, 1 = x, 2 = dY, 3 = outlier-channel choice; x and dY are
drawn in blocks of ROW_BLOCK token rows, block b from the stream
``[cfg, mat, kind, b]``.

Workloads (all tensors are bfloat16 bit patterns stored as ``uint16``):

* master weights W ~ N(0, 0.02) (std 0.02);
* activations x ~ N(0, 1), or Student-t with 4 degrees of freedom
  (unscaled, variance 2) for the heavy-tailed 3B-like workload, optionally
  with a fraction of outlier channels (columns) scaled by 20;
* upstream gradients dY ~ N(0, 1).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

KIND_W, KIND_X, KIND_DY, KIND_OUTLIER = 0, 1, 2, 3


def rng(cfg: int, mat: int, kind: int, extra: Sequence[int] = ()) -> np.random.Generator:
    """Counter-style seeded generator for tensor ``kind`` of matrix ``mat`` in config ``cfg``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, mat, kind, *extra])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Inputs must be finite; the generators never produce non-finite values.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite float32 bits are <= 0xFF7FFFFF, so the addition cannot wrap in uint32
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal_f32(g: np.random.Generator, shape, std: float) -> np.ndarray:
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def weight(cfg: int, mat: int, d_out: int, d_in: int, std: float = 0.02) -> np.ndarray:
    """Master weight W [d_out, d_in] ~ N(0, std), bf16 bits."""
    return f32_to_bf16_bits(_normal_f32(rng(cfg, mat, KIND_W), (d_out, d_in), std))


ROW_BLOCK = 2048  # token rows per independently seeded block


def _row_blocks(T: int, rows: Optional[np.ndarray]):
    if rows is None:
        return list(range((T + ROW_BLOCK - 1) // ROW_BLOCK))
    return sorted(set(int(r) // ROW_BLOCK for r in np.asarray(rows)))


def _blocked(T: int, ncols: int, fill, rows: Optional[np.ndarray], threads: Optional[int]) -> np.ndarray:
    """Assemble a [T, ncols] bf16 tensor from row blocks of ROW_BLOCK tokens; block b is drawn by
    ``fill(b, nrows)`` from its own seeded stream, so any subset of rows can be regenerated alone
    and blocks can be drawn in parallel threads (numpy releases the GIL while filling)."""
    blocks = _row_blocks(T, rows)
    out = {}

    def work(b):
        n = min(ROW_BLOCK, T - b * ROW_BLOCK)
        out[b] = f32_to_bf16_bits(fill(b, n))

    nthreads = threads if threads is not None else min(16, os.cpu_count() or 1)
    if nthreads > 1 and len(blocks) > 1:
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            list(ex.map(work, blocks))
    else:
        for b in blocks:
            work(b)
    if rows is None:
        if not blocks:
            return np.zeros((0, ncols), np.uint16)
        return np.concatenate([out[b] for b in blocks], axis=0)
    rows = np.asarray(rows)
    res = np.empty((len(rows), ncols), np.uint16)
    for k, r in enumerate(rows):
        res[k] = out[int(r) // ROW_BLOCK][int(r) % ROW_BLOCK]
    return res


def activation(cfg: int, mat: int, T: int, d_in: int, dist: str = "normal",
               outlier_frac: float = 0.0, outlier_scale: float = 20.0,
               rows: Optional[np.ndarray] = None, threads: Optional[int] = None) -> np.ndarray:
    """Activations x [T, d_in] (bf16 bits), drawn in row blocks of ROW_BLOCK tokens.

    ``dist`` is ``"normal"`` (N(0,1)) or ``"student_t4"`` (Student-t, nu = 4).
    ``outlier_frac`` > 0 picks ``max(1, round(frac * d_in))`` seeded columns and
    scales them by ``outlier_scale`` before rounding to bf16.
    ``rows``: optional token indices; only those rows are returned (identical to
    the same rows of the full tensor).
    """
    if dist not in ("normal", "student_t4"):
        raise ValueError(f"unknown activation distribution {dist!r}")
    cols = None
    if outlier_frac > 0.0:
        k = max(1, int(round(outlier_frac * d_in)))
        cols = rng(cfg, mat, KIND_OUTLIER).choice(d_in, size=k, replace=False)

    def fill(b, n):
        g = rng(cfg, mat, KIND_X, (b,))
        if dist == "normal":
            blk = g.standard_normal(size=(n, d_in), dtype=np.float32)
        else:
            blk = g.standard_t(4.0, size=(n, d_in)).astype(np.float32)
        if cols is not None:
            blk[:, cols] *= np.float32(outlier_scale)
        return blk

    return _blocked(T, d_in, fill, rows, threads)


def grad_out(cfg: int, mat: int, T: int, d_out: int, rows: Optional[np.ndarray] = None,
             threads: Optional[int] = None) -> np.ndarray:
    """Upstream gradient dY [T, d_out] ~ N(0, 1), bf16 bits, drawn in row blocks."""
    def fill(b, n):
        return rng(cfg, mat, KIND_DY, (b,)).standard_normal(size=(n, d_out), dtype=np.float32)

    return _blocked(T, d_out, fill, rows, threads)


# ----------------------------------------------------------------------------
# Edge-case tensors
# ----------------------------------------------------------------------------

def tie_heavy_weight(seed: int, d_out: int, d_in: int, alphabet: Sequence[float] = (-2, -1, 0, 1, 2),
                     scale: float = 0.01) -> np.ndarray:
    """W whose entries come from a tiny alphabet (times ``scale``), so groups are full of ties."""
    g = rng(1000 + seed, 0, KIND_W)
    vals = np.asarray(alphabet, dtype=np.float32) * np.float32(scale)
    return f32_to_bf16_bits(vals[g.integers(0, len(vals), size=(d_out, d_in))])


def boundary_row_weight(d_out: int, d_in: int) -> np.ndarray:
    """Rows of alternating 0.5 and 1.5: mean |W| is exactly 1, so |w| = 0.5 sits on the ternary threshold."""
    row = np.tile(np.asarray([0.5, 1.5], dtype=np.float32), d_in // 2)
    sign = np.where((np.arange(d_in) // 3) % 2 == 0, 1.0, -1.0).astype(np.float32)
    return f32_to_bf16_bits(np.tile(row * sign, (d_out, 1)))


@dataclasses.dataclass(frozen=True)
class Linear:
    name: str
    d_out: int
    d_in: int


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark/test workload: a set of linears, a token count, mask patterns."""
    cfg: int
    name: str
    linears: Tuple[Linear, ...]
    T: Tuple[int, ...]
    n_keep: Tuple[int, ...]
    act_dist: str
    outlier_frac: float
    backward: bool


WORKLOADS: Dict[int, Workload] = {
    0: Workload(0, "single linear 256x256, 64 tokens, 6:8, fwd+bwd",
                (Linear("w", 256, 256),), (64,), (6,), "normal", 0.0, True),
    1: Workload(1, "0.5B-like MLP up-projection 896->4864, 512 tokens, 8/6/4/2:8, fwd",
                (Linear("up", 4864, 896),), (512,), (8, 6, 4, 2), "normal", 0.001, False),
    2: Workload(2, "1.5B-like linears q,o 1536->1536, gate,up 1536->8960, down 8960->1536, 8192 tokens, 6:8, fwd+bwd",
                (Linear("q", 1536, 1536), Linear("o", 1536, 1536), Linear("gate", 8960, 1536),
                 Linear("up", 8960, 1536), Linear("down", 1536, 8960)), (8192,), (6,), "normal", 0.0, True),
    3: Workload(3, "3B-like decoder-layer linears (q,k,v,o,gate,up,down), 16x2048 = 32768 tokens, 6:8, fwd+bwd",
                (Linear("q", 2048, 2048), Linear("k", 256, 2048), Linear("v", 256, 2048), Linear("o", 2048, 2048),
                 Linear("gate", 11008, 2048), Linear("up", 11008, 2048), Linear("down", 2048, 11008)),
                (32768,), (6,), "student_t4", 0.0, True),
    4: Workload(4, "3B-like decode on pre-packed weights, 1/8/64 tokens, 6/4/2:8, fwd",
                (Linear("q", 2048, 2048), Linear("k", 256, 2048), Linear("v", 256, 2048), Linear("o", 2048, 2048),
                 Linear("gate", 11008, 2048), Linear("up", 11008, 2048), Linear("down", 2048, 11008)),
                (1, 8, 64), (6, 4, 2), "student_t4", 0.0, False),
}


def sample_rows(cfg: int, mat: int, T: int, count: int) -> np.ndarray:
    """Sorted, seeded sample of ``count`` distinct token indices in [0, T)."""
    g = rng(cfg, mat, 7)
    count = min(count, T)
    return np.sort(g.choice(T, size=count, replace=False))


__all__: List[str] = [
    "rng", "f32_to_bf16_bits", "bf16_bits_to_f32", "weight", "activation", "grad_out",
    "tie_heavy_weight", "boundary_row_weight", "Linear", "Workload", "WORKLOADS", "sample_rows",
]
