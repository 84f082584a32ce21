"""GPU parity: every ladder variant against the CPU oracle, through the C ABI.

Bar: every element within |C - C_ref| <= 4 K 2^-24 sum_k |a_ik b_kj| of the
double-precision oracle (the checker in oracle.check), every element written
(C is prefilled with NaN), C's padding and the memory after it untouched.
Integer-valued inputs make every partial sum exact in float, so there the
GPU must equal the oracle bit for bit in any summation order.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import check
from roofline_sgemm_f32_amd.inputs import WORKLOADS, as_numpy, make_operands, workload_operands
import roofline_sgemm_f32_amd as rs
from tests.gpu_util import run, to_device

pytestmark = pytest.mark.gpu

ALL = ["k0_naive", "k1_coalesced", "k2_lds_tiled32", "k2_lds_tiled16", "k2_lds_tiled32_pad1", "k2_lds_tiled16_pad1",
       "k3_regtile_db", "k4_mfma", "k4_mfma_tile128", "k4_mfma_tile64", "k4_mfma_tile128x256", "auto"]
FAST = ["k3_regtile_db", "k4_mfma", "k4_mfma_tile128", "k4_mfma_tile64", "k4_mfma_tile128x256", "auto"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rs.load()
    oracle.load()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def full_check(variant, M, N, K, dist="uniform", seed=0, lda=None, ldb=None, ldc=None):
    A, B = make_operands(M, N, K, dist, seed, lda=lda, ldb=ldb)
    C, out = run(variant, A, B, ldc=ldc)
    ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    rep = check.check(C, ref, S, K)
    assert out.guard_intact(), f"{variant} {M}x{N}x{K}: wrote outside C"
    assert rep["ok"], f"{variant} {M}x{N}x{K}: {rep}"
    if dist == "int":
        assert np.array_equal(C.astype(np.float64), ref), f"{variant} {M}x{N}x{K}: not exact"
    return C, rep


SHAPES = [
    (1, 1, 1), (7, 5, 3), (33, 65, 17), (64, 64, 64), (127, 129, 31), (128, 128, 16),
    (129, 257, 33), (200, 300, 1), (256, 256, 256), (96, 160, 1000), (300, 17, 129),
]


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes_uniform(variant, shape):
    M, N, K = shape
    note(f"[parity] {variant} {M}x{N}x{K}")
    full_check(variant, M, N, K, "uniform", seed=M + 3 * N + 7 * K)


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes_integer_exact(variant, shape):
    M, N, K = shape
    note(f"[exact] {variant} {M}x{N}x{K}")
    full_check(variant, M, N, K, "int", seed=11 * M + N + K)


@pytest.mark.parametrize("variant", ALL)
def test_padded_leading_dimensions(variant):
    # lda > K, ldb > N, ldc > N; odd values break 16-byte row alignment.
    for (M, N, K, lda, ldb, ldc) in [(70, 90, 50, 53, 97, 91), (130, 132, 40, 44, 136, 140),
                                     (65, 129, 257, 261, 131, 133)]:
        note(f"[ld] {variant} {M}x{N}x{K} lda={lda} ldb={ldb} ldc={ldc}")
        full_check(variant, M, N, K, "int", seed=5, lda=lda, ldb=ldb, ldc=ldc)
        full_check(variant, M, N, K, "uniform", seed=6, lda=lda, ldb=ldb, ldc=ldc)


@pytest.mark.parametrize("variant", ALL)
def test_k_zero_writes_zeros(variant):
    note(f"[k0] {variant}")
    A = torch.zeros((37, 0))
    B = torch.zeros((0, 41))
    C, out = run(variant, A, B, ldc=45)
    assert np.all(C == 0.0) and out.guard_intact()


@pytest.mark.parametrize("variant", ALL)
def test_empty_output_is_noop(variant):
    assert rs.sgemm_f32_variant(variant, 0, 5, 5, 0, 5, 0, 5, 0, 5, None) == 0
    assert rs.sgemm_f32_variant(variant, 5, 0, 5, 0, 5, 0, 1, 0, 1, None) == 0


@pytest.mark.parametrize("variant", FAST)
def test_edge_sweep_1_to_9(variant):
    # Every (M, N, K) in 1..9: exact integer inputs, bitwise.
    note(f"[sweep9] {variant}")
    for M in range(1, 10):
        for N in range(1, 10):
            for K in range(1, 10):
                full_check(variant, M, N, K, "int", seed=M * 100 + N * 10 + K)


@pytest.mark.parametrize("variant", ["k0_naive", "k1_coalesced", "k2_lds_tiled32", "k2_lds_tiled16",
                                     "k2_lds_tiled32_pad1", "k2_lds_tiled16_pad1"])
def test_edge_sweep_1_to_5(variant):
    note(f"[sweep5] {variant}")
    for M in range(1, 6):
        for N in range(1, 6):
            for K in range(1, 6):
                full_check(variant, M, N, K, "int", seed=M * 100 + N * 10 + K)


@pytest.mark.parametrize("variant", FAST)
def test_tile_boundaries(variant):
    for n in (31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257):
        note(f"[tile] {variant} n={n}")
        full_check(variant, n, n, n, "int", seed=n)
        full_check(variant, n, 2 * n + 1, (n // 2) + 3, "uniform", seed=n + 1)


@pytest.mark.parametrize("variant", FAST)
def test_unaligned_pointers(variant):
    # Operands starting 4 bytes past a 16-byte boundary take the 4-byte load path.
    M, N, K = 100, 132, 68
    A, B = make_operands(M, N, K, "int", seed=9)
    Ad = torch.empty(M * K + 1, device="cuda")[1:].view(M, K)
    Ad.copy_(A.cuda())
    Bd = torch.empty(K * N + 1, device="cuda")[1:].view(K, N)
    Bd.copy_(B.cuda())
    note(f"[unaligned] {variant}")
    C, out = run(variant, A, B, A_dev=Ad, B_dev=Bd)
    ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    assert np.array_equal(C.astype(np.float64), ref) and out.guard_intact()


# --- invariants ----------------------------------------------------------

@pytest.mark.parametrize("variant", FAST)
def test_identity_and_scaling(variant):
    M, N, K = 200, 150, 130
    A, B = make_operands(M, N, K, "uniform", seed=21)
    note(f"[identity] {variant}")
    C_ai, _ = run(variant, A, torch.eye(K))
    assert np.array_equal(C_ai, as_numpy(A)), "A * I != A"
    Bk = make_operands(K, N, K, "uniform", 22)[1]
    C_ib, _ = run(variant, torch.eye(K), Bk)
    assert np.array_equal(C_ib, as_numpy(Bk)), "I * B != B"
    C1, _ = run(variant, A, B)
    C2, _ = run(variant, A * 2, B)
    assert np.array_equal(C2, 2 * C1), "(2A) B != 2 (A B)"
    C3, _ = run(variant, A, B)
    assert np.array_equal(C1, C3), "run-to-run difference"


@pytest.mark.parametrize("variant", FAST)
def test_all_ones_gives_row_sums(variant):
    M, N, K = 77, 300, 513
    A, _ = make_operands(M, N, K, "uniform", seed=31)
    note(f"[ones] {variant}")
    C, _ = run(variant, A, torch.ones((K, N)))
    Ad = as_numpy(A).astype(np.float64)
    rowsum, S = Ad.sum(axis=1), np.abs(Ad).sum(axis=1)
    rep = check.check(C, np.repeat(rowsum[:, None], N, 1), np.repeat(S[:, None], N, 1), K)
    assert rep["ok"], rep
    # Every column sees the same k order, so a row is constant.
    assert np.all(C == C[:, :1])


@pytest.mark.parametrize("variant", ["k4_mfma_tile128", "k4_mfma_tile64", "k4_mfma_tile128x256"])
def test_row_permutation_k4(variant):
    M, N, K = 256, 256, 300
    A, B = make_operands(M, N, K, "normal", seed=41)
    perm = torch.randperm(M, generator=torch.Generator().manual_seed(1))
    C, _ = run(variant, A, B)
    Cp, _ = run(variant, A[perm].contiguous(), B)
    assert np.array_equal(Cp, C[perm.numpy()])


# --- the five workloads ---------------------------------------------------

WL_VARIANTS = ["auto", "k4_mfma_tile128", "k4_mfma_tile64", "k4_mfma_tile128x256"]


class _WorkloadRefs:
    """Host operands and the oracle's full result for one workload at a time
    (the largest, square8192_normal, takes about 1.5 GB of host memory for
    C_ref and S), computed once and reused by every variant's test."""

    def __init__(self):
        self.key = None
        self.val = None

    def get(self, name, dist):
        key = (name, dist)
        if self.key != key:
            self.key, self.val = None, None
            w = WORKLOADS[name]
            if dist == "int":
                A, B = make_operands(w.M, w.N, w.K, "int", seed=w.seed, lda=w.lda, ldb=w.ldb)
            else:
                A, B = workload_operands(w)
            note(f"[workload] oracle {name} {dist} ...")
            ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B), bound=dist != "int")
            self.key, self.val = key, (A, B, ref, S)
        return self.val


@pytest.fixture(scope="module")
def workload_refs():
    return _WorkloadRefs()


# Grouped by workload so that each oracle result is computed once.
WL_CASES = [(name, v) for name in WORKLOADS for v in WL_VARIANTS]


@pytest.mark.parametrize("name,variant", WL_CASES, ids=[f"{n}-{v}" for n, v in WL_CASES])
def test_workload(workload_refs, name, variant):
    """The five workloads at full size, every element of C against the
    oracle's bound; every element written, C's padding and tail untouched."""
    w = WORKLOADS[name]
    A, B, ref, S = workload_refs.get(name, w.dist)
    note(f"[workload] {variant} {name}")
    C, out = run(variant, A, B, ldc=w.ldc)
    assert out.guard_intact(), "wrote outside C"
    rep = check.check(C, ref, S, w.K)
    assert rep["ok"], rep
    assert rep["n"] == w.M * w.N
    note(f"[workload] {variant} {name}: max bound use {rep['max_bound_util']:.3g}, "
         f"page rel err {rep['max_rel_err_page']:.3g}")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_integer_exact(workload_refs, name):
    """The workloads' shapes with integer inputs: every element of the AUTO
    result bit-identical to the oracle (all partial sums exact in float)."""
    w = WORKLOADS[name]
    A, B, ref, _ = workload_refs.get(name, "int")
    note(f"[workload-int] {name}")
    C, out = run("auto", A, B, ldc=w.ldc)
    assert out.guard_intact()
    assert np.array_equal(C.astype(np.float64), ref)


# Narrow outputs where the plan keeps 64 x 64 tiles (128 x 256 or 128 x 128
# ones would be mostly empty), and an output split by the 64 x 64 cost model:
# AUTO against the full oracle, uniform and integer operands.
NARROW = [(65536, 64, 256), (16384, 160, 512), (8192, 320, 300), (192, 2048, 4096)]


@pytest.mark.parametrize("shape", NARROW, ids=lambda s: "x".join(map(str, s)))
def test_narrow_outputs_auto(shape):
    M, N, K = shape
    note(f"[narrow] {M}x{N}x{K} plan {rs.plan_config(M, N, K, A_ptr=1 << 40, B_ptr=1 << 40)}")
    full_check("auto", M, N, K, "uniform", seed=M + N)
    full_check("auto", M, N, K, "int", seed=M + K)


# Thin unaligned operands of large products: the packing pre-pass copies the
# thin one (B with 9 or 13 columns, A with 13 rows and K = 8191) and the
# product runs on 16-byte loads with a K split, all through one workspace.
THIN = [(8192, 13, 8192), (8192, 9, 4096), (13, 8192, 8191)]


@pytest.mark.parametrize("shape", THIN, ids=lambda s: "x".join(map(str, s)))
def test_thin_unaligned_auto(shape):
    M, N, K = shape
    plan = rs.plan_config(M, N, K, A_ptr=1 << 40, B_ptr=1 << 40)
    note(f"[thin] {M}x{N}x{K} plan {plan}")
    assert plan["packed"]
    full_check("auto", M, N, K, "uniform", seed=M + N)
    full_check("auto", M, N, K, "int", seed=M + K)


# Mid-size outputs of 257 to 1024 tiles of 32 x 32 with K <= 2048, which the
# plan runs unsplit on 32 x 32 tiles with 4 K groups (K slabs of 16 in three
# LDS stages, or of 32 in two; more than 768 tiles: slabs of 16 in two
# stages, four workgroups per CU); edges that are not tile multiples
# included, and K from 640 to 2048.
MID = [(640, 640, 640), (300, 1000, 900), (768, 1024, 1024), (1000, 700, 1000),
       (768, 1024, 1280), (1024, 768, 2048), (512, 768, 2048), (700, 900, 1500),
       (896, 896, 896), (1000, 1000, 1024), (800, 1024, 2048)]


@pytest.mark.parametrize("shape", MID, ids=lambda s: "x".join(map(str, s)))
def test_mid_outputs_auto(shape):
    M, N, K = shape
    plan = rs.plan_config(M, N, K, A_ptr=1 << 40, B_ptr=1 << 40)
    note(f"[mid] {M}x{N}x{K} plan {plan}")
    assert plan["tile"] == (32, 32) and plan["k_groups"] == 4 and plan["splits"] == 1, plan
    full_check("auto", M, N, K, "uniform", seed=M + N)
    full_check("auto", M, N, K, "int", seed=M + K)


@pytest.mark.parametrize("shape", MID[4:], ids=lambda s: "x".join(map(str, s)))
def test_mid_outputs_transposed_a(shape):
    """The same plan with A stored K x M (its own occupancy target): every
    element, uniform within the bound and integer bit-exact."""
    M, N, K = shape
    plan = rs.plan_config(M, N, K, transa=True, A_ptr=1 << 40, B_ptr=1 << 40)
    note(f"[mid-tn] {M}x{N}x{K} plan {plan}")
    assert plan["tile"] == (32, 32) and plan["k_groups"] == 4 and plan["splits"] == 1, plan
    for dist in ("uniform", "int"):
        A, B = make_operands(M, N, K, dist, seed=M + 3 * K)
        At = A.t().contiguous()
        C = torch.full((M, N), float("nan"), device="cuda")
        rs.sgemm_ex(At.cuda(), B.cuda(), out=C, transa=True)
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        ref, S, E = oracle.sgemm_ex_f64(True, False, 1.0, as_numpy(At), as_numpy(B), 0.0, None)
        rep = check.check_ex(got, ref, S, E, K)
        assert rep["ok"], (dist, rep)
        if dist == "int":
            assert np.array_equal(got.astype(np.float64), ref)
