"""Helpers for the GPU parity tests: place seeded host operands on the device
with their leading dimensions, run one variant through the C ABI, and check
the output guard band."""
from __future__ import annotations

import numpy as np
import torch

import roofline_sgemm_f32_amd as rs

SENTINEL = 12345.0  # value kept in C's padding and tail; the kernel must not touch it
TAIL = 67           # guard elements after C's last row


def to_device(x: torch.Tensor) -> torch.Tensor:
    """Copy a host row-major view (any row stride) to the device, keeping the
    row stride; padding elements are copied too (NaN from inputs.padded)."""
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else max(cols, 1)
    if rows == 0 or cols == 0:
        return torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    base = torch.as_strided(x, (rows, ld), (ld, 1)) if ld > cols else x
    dev = base.contiguous().cuda()
    return dev[:, :cols]


class Out:
    """A device C buffer (M x N, leading dimension ldc) prefilled with NaN,
    with SENTINEL in the padding columns and in TAIL elements past the end."""

    def __init__(self, M: int, N: int, ldc: int | None = None):
        self.M, self.N = M, N
        self.ldc = ldc or max(N, 1)
        total = M * self.ldc + TAIL
        self.buf = torch.full((total,), SENTINEL, dtype=torch.float32, device="cuda")
        if M and N:
            self.view().fill_(float("nan"))

    def view(self) -> torch.Tensor:
        return torch.as_strided(self.buf, (self.M, self.N), (self.ldc, 1))

    def host(self) -> np.ndarray:
        return self.view().cpu().numpy()

    def guard_intact(self) -> bool:
        full = self.buf.cpu().numpy()
        mask = np.ones(full.size, dtype=bool)
        for i in range(self.M):
            mask[i * self.ldc:i * self.ldc + self.N] = False
        return bool(np.all(full[mask] == SENTINEL))


def run(variant, A_host: torch.Tensor, B_host: torch.Tensor, ldc: int | None = None,
        A_dev=None, B_dev=None) -> tuple[np.ndarray, "Out"]:
    """C = A * B on the GPU with ``variant``; returns (C host copy, Out)."""
    M, K = A_host.shape
    N = B_host.shape[1]
    A = to_device(A_host) if A_dev is None else A_dev
    B = to_device(B_host) if B_dev is None else B_dev
    out = Out(M, N, ldc)
    lda = A.stride(0) if (M > 1 and K > 0) else max(K, 1)
    ldb = B.stride(0) if (K > 1 and N > 0) else max(N, 1)
    aptr = A.data_ptr() if A.numel() else 0
    bptr = B.data_ptr() if B.numel() else 0
    cptr = out.buf.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    st = rs.sgemm_f32_variant(variant, M, N, K, aptr, lda, bptr, ldb, cptr, out.ldc, stream)
    if st != 0:
        raise rs.SgemmError(st, f"variant {variant}")
    torch.cuda.synchronize()
    return out.host(), out
