"""GPU special values and determinism, through the C ABI.

NaN and infinity in the operands propagate as IEEE arithmetic says (the
oracle, in double, is the reference): the zero fill the kernels use for
edge tiles, the K tail, split-K and packed operands must neither hide a NaN
nor create one.  Inputs are small, so no finite sum overflows in float.
Every variant and path is run-to-run deterministic (same bits twice)."""
import numpy as np
import pytest
import torch

import oracle
import roofline_sgemm_f32_amd as rs
from roofline_sgemm_f32_amd.inputs import as_numpy, make_operands
from tests.gpu_util import run

pytestmark = pytest.mark.gpu

VARIANTS = ["k1_coalesced", "k2_lds_tiled32", "k3_regtile_db", "k4_mfma", "k4_mfma_tile128",
            "k4_mfma_tile64", "k4_mfma_tile128x256", "auto"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rs.load()
    oracle.load()


def plant(A, B, seed):
    """Put NaN, +inf and -inf at a few places of A and B (host copies)."""
    g = np.random.default_rng(seed)
    A, B = A.clone(), B.clone()
    M, K = A.shape
    N = B.shape[1]
    for val in (float("nan"), float("inf"), float("-inf")):
        A[g.integers(M), g.integers(K)] = val
        B[g.integers(K), g.integers(N)] = val
    # An infinity times a zero: NaN, however the sum is ordered.
    i, k = g.integers(M), g.integers(K)
    A[i, k] = float("inf")
    B[k, :] = 0.0
    return A, B


def masks(C):
    return np.isnan(C), np.isposinf(C), np.isneginf(C)


def check_special(C, ref):
    for got, want, what in zip(masks(C), masks(ref), ("nan", "+inf", "-inf")):
        assert np.array_equal(got, want), f"{what} pattern differs at {np.argwhere(got != want)[:5]}"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(C[fin]))


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", [(33, 65, 17), (129, 257, 131), (300, 260, 170)],
                         ids=lambda s: "x".join(map(str, s)))
def test_nan_inf_propagate(variant, shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, "uniform", seed=M + N)
    A, B = plant(A, B, seed=K)
    C, out = run(rs.VARIANTS[variant], A, B)
    ref, _ = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    check_special(C, ref)
    assert out.guard_intact()


@pytest.mark.parametrize("splits", [2, 7])
@pytest.mark.parametrize("shape", [(64, 96, 2048), (65, 97, 2047)], ids=lambda s: "x".join(map(str, s)))
def test_nan_inf_propagate_split(splits, shape):
    M, N, K = shape
    A, B = make_operands(M, N, K, "uniform", seed=splits)
    A, B = plant(A, B, seed=splits + 1)
    C = rs.sgemm_ex(A.cuda(), B.cuda(), splits=splits)
    torch.cuda.synchronize()
    ref, _ = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    check_special(C.cpu().numpy(), ref)


def test_nan_inf_propagate_packed():
    # Output large enough for packing of both operands (K and N odd).
    M, N, K = 1601, 1283, 97
    A, B = make_operands(M, N, K, "uniform", seed=3)
    A, B = plant(A, B, seed=4)
    C = rs.sgemm_ex(A.cuda(), B.cuda())
    torch.cuda.synchronize()
    ref, _ = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    check_special(C.cpu().numpy(), ref)


@pytest.mark.parametrize("variant", VARIANTS)
def test_run_to_run_deterministic(variant):
    M, N, K = 1000, 777, 1234
    A, B = make_operands(M, N, K, "normal", seed=11)
    C1, _ = run(rs.VARIANTS[variant], A, B)
    C2, _ = run(rs.VARIANTS[variant], A, B)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


@pytest.mark.parametrize("shape,splits", [((128, 128, 4096), 0), ((1601, 1283, 97), 0),
                                          ((200, 120, 3000), 5)], ids=["split", "packed", "split5"])
def test_paths_deterministic(shape, splits):
    M, N, K = shape
    A, B = make_operands(M, N, K, "normal", seed=12)
    Ad, Bd = A.cuda(), B.cuda()
    C1 = rs.sgemm_ex(Ad, Bd, splits=splits)
    C2 = rs.sgemm_ex(Ad, Bd, splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))
