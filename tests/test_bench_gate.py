"""Host logic of bench.py's row gate, the check that decides whether a timed
GPU product outside the headline leg (a ladder row, a small-shape plan) gets
its throughput printed.  CPU tensors stand in for the GPU result."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _operands(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    A = torch.rand((M, K), generator=g) * 2 - 1
    B = torch.rand((K, N), generator=g) * 2 - 1
    return A, B


def test_row_gate_accepts_fp32_product():
    A, B = _operands(37, 29, 301, 11)
    gate = bench.row_gate(A, B)
    ok, util = gate(A @ B)
    assert ok and 0.0 <= util < 1.0


def test_row_gate_rejects_wrong_gated_row():
    A, B = _operands(37, 29, 301, 12)
    C = A @ B
    # Row M-1 is one of the gate rows: an error of 0.1 there is far above
    # 4 K 2^-24 sum|ab| (about 5e-3 here: sum|ab| is near K/4).
    C[-1, 5] += 0.1
    ok, util = bench.row_gate(A, B)(C)
    assert not ok and util is None


def test_row_gate_rejects_nan_and_accepts_exact_integers():
    g = torch.Generator().manual_seed(13)
    A = torch.randint(-2, 3, (9, 40), generator=g).float()
    B = torch.randint(-2, 3, (40, 7), generator=g).float()
    exact = torch.from_numpy(A.numpy().astype(np.float64) @ B.numpy().astype(np.float64)).float()
    assert bench.row_gate(A, B)(exact) == (True, 0.0)
    exact[0, 0] = float("nan")
    assert bench.row_gate(A, B)(exact)[0] is False


def test_row_gate_single_row():
    A, B = _operands(1, 5, 3, 14)
    assert bench.row_gate(A, B)(A @ B)[0]


def test_row_gate_checks_every_row_of_small_products(monkeypatch):
    """Up to ROW_GATE_FULL_MACS multiply-adds every row is gated: an error in
    a row that is none of the six sampled ones fails; above the limit only
    the sampled rows are."""
    A, B = _operands(37, 29, 301, 16)
    C = A @ B
    C[7, 3] += 0.1        # row 7: not 0, 1, 12, 18, 35 or 36
    assert bench.row_gate(A, B)(C)[0] is False
    monkeypatch.setattr(bench, "ROW_GATE_FULL_MACS", 1)
    assert bench.row_gate(A, B)(C)[0] is True


def test_oracle_gate_checks_every_element():
    """bench.oracle_gate (the CPU leg's full-product gate): a float32 product
    passes, one wrong element anywhere fails."""
    from roofline_sgemm_f32_amd.inputs import Workload
    A, B = _operands(23, 31, 200, 15)
    w = Workload("t", 23, 31, 200, 200, 31, 31, "uniform", 15)
    C = (A @ B).numpy()
    rep = bench.oracle_gate(w, A, B, C)
    assert rep["ok"] and rep["elements_checked"] == 23 * 31
    C[11, 17] += 0.05
    rep = bench.oracle_gate(w, A, B, C)
    assert not rep["ok"] and rep["n_violations"] == 1
