"""Seeded synthetic inputs shared by the GPU path's tests and the oracle's.

This module draws random numbers and lays them out; it holds none of the
matrix-multiply arithmetic.  Both sides receive the very same host bits.

Recipe: ``g = torch.Generator().manual_seed(seed)``; A is drawn first, then B,
from the same generator.  Uniform operands are ``torch.rand * 2 - 1``, which
is exact in float32 and lies in [-1, 1 - 2**-23]; normal operands are
``torch.randn``.  Where a leading dimension exceeds the row length, the
padding columns are filled with NaN so that any read of them shows up.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """One SGEMM problem: sizes, leading dimensions, distribution and seed."""
    name: str
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    dist: str  # "uniform" (U[-1,1)), "normal" (N(0,1)) or "int" (integers in [-2, 2])
    seed: int


def _square(name, n, dist, seed):
    return Workload(name, n, n, n, n, n, n, dist, seed)


# The five problem shapes the pages' workload is measured on, largest last.
WORKLOADS = {
    "square256": _square("square256", 256, "uniform", 1),
    "square1024": _square("square1024", 1024, "uniform", 2),
    "square4096": _square("square4096", 4096, "uniform", 3),
    "ragged3001x4099x2047": Workload("ragged3001x4099x2047", 3001, 4099, 2047,
                                     2047, 4099, 4099, "uniform", 4),
    "square8192_normal": _square("square8192_normal", 8192, "normal", 5),
}

COPY_ELEMENTS = 256 * 1024 * 1024  # 1 GiB of float per array
COPY_SEED = 6


def _draw(g: torch.Generator, rows: int, cols: int, dist: str) -> torch.Tensor:
    if dist == "uniform":
        return torch.rand((rows, cols), generator=g, dtype=torch.float32) * 2 - 1
    if dist == "normal":
        return torch.randn((rows, cols), generator=g, dtype=torch.float32)
    if dist == "int":
        return torch.randint(-2, 3, (rows, cols), generator=g).to(torch.float32)
    if dist == "ones":
        return torch.ones((rows, cols), dtype=torch.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def padded(x: torch.Tensor, ld: int) -> torch.Tensor:
    """Place a rows x cols matrix in a buffer with leading dimension ``ld``.

    Returns a view whose stride(0) is ``ld``; the padding columns hold NaN."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    if ld == cols:
        return x.contiguous()
    buf = torch.full((rows, ld), float("nan"), dtype=torch.float32)
    buf[:, :cols] = x
    return buf[:, :cols]


def make_operands(M: int, N: int, K: int, dist: str = "uniform", seed: int = 0,
                  lda: int | None = None, ldb: int | None = None, dist_b: str | None = None):
    """Draw A (M x K) then B (K x N) on the host; returns CPU float32 tensors
    (views with the requested leading dimensions)."""
    g = torch.Generator().manual_seed(seed)
    A = _draw(g, M, K, dist)
    B = _draw(g, K, N, dist_b or dist)
    return padded(A, lda or max(K, 1)), padded(B, ldb or max(N, 1))


def workload_operands(w: Workload):
    """Host operands of a named workload."""
    return make_operands(w.M, w.N, w.K, w.dist, w.seed, w.lda, w.ldb)


def copy_source(n: int = COPY_ELEMENTS, seed: int = COPY_SEED) -> torch.Tensor:
    """The copy probe's source array (uniform [-1, 1))."""
    g = torch.Generator().manual_seed(seed)
    return torch.rand(n, generator=g, dtype=torch.float32) * 2 - 1


def as_numpy(x: torch.Tensor) -> np.ndarray:
    """A numpy view of a CPU float32 tensor that keeps its strides."""
    return x.numpy()


def probe_operands(seed: int = 7, dist: str = "int"):
    """Operand values of the matrix-unit probe: 64 for A, then 64 for B."""
    g = torch.Generator().manual_seed(seed)
    a = _draw(g, 1, 64, dist).reshape(64)
    b = _draw(g, 1, 64, dist).reshape(64)
    return a, b
