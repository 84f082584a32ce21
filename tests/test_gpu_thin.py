"""GPU parity of the thin-product kernels (M <= 8 or N <= 8 with a large
streamed operand), through the C ABI.

Every call goes through the shape-chosen entry point (sgemm_f32_ex) and is
first checked to take the thin path (sgemm_plan_config); the result must meet
the general bound against the CPU oracle (|C - C_ref| <= 4 K 2^-24 |alpha|
sum|ab| + 2 * 2^-24 (|alpha sum ab| + |beta C0|)), and with integer operands
and small integer alpha, beta it must equal the oracle bit for bit.  Shapes
cover M and N from 1 to 8, K chunks split and whole, K not a multiple of
the kernels' pieces, outputs not a multiple of a workgroup's columns or
rows, and A or B stored transposed where the path allows it."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import check
import roofline_sgemm_f32_amd as rs
from roofline_sgemm_f32_amd.inputs import as_numpy, make_operands
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rs.load()
    oracle.load()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_thin(ta, tb, M, N, K, alpha, beta, dist, seed):
    A, B = make_operands(M, N, K, dist, seed)
    C0 = make_operands(M, 1, N, dist, seed + 1)[0]
    As = A.t().contiguous() if ta else A.contiguous()
    Bs = B.t().contiguous() if tb else B.contiguous()
    Ad, Bd = to_device(As), to_device(Bs)
    plan = rs.plan_config(M, N, K, transa=bool(ta), transb=bool(tb), lda=Ad.stride(0),
                          ldb=Bd.stride(0), A_ptr=Ad.data_ptr(), B_ptr=Bd.data_ptr())
    note(f"[thin] {ta}{tb} {M}x{N}x{K} alpha={alpha} beta={beta} {dist} plan={plan}")
    assert plan["engine"] == "thin", plan
    Cbuf = torch.full((M * N + 16,), 777.0, device="cuda")
    Cd = torch.as_strided(Cbuf, (M, N), (N, 1))
    Cd.copy_(C0)
    st = rs.load().sgemm_f32_ex(int(ta), int(tb), M, N, K, alpha, Ad.data_ptr(), Ad.stride(0),
                                Bd.data_ptr(), Bd.stride(0), beta, Cbuf.data_ptr(), N,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0, rs.status_string(st)
    torch.cuda.synchronize()
    assert torch.all(Cbuf[M * N:].cpu() == 777.0), "wrote past C"
    got = Cd.cpu().numpy()
    ref, S, E = oracle.sgemm_ex_f64(ta, tb, alpha, as_numpy(As), as_numpy(Bs), beta,
                                    None if beta == 0 else as_numpy(C0))
    return got, ref, S, E, plan


# (transa, transb, M, N, K).  The streamed operand is 384 MB or more (256 MB
# for 2 to 4 columns, 16 MB for a single column), where the plan takes the
# thin path.  Row counts of the thin_n cases are not multiples of a
# workgroup's rows (32, or 16 for one or two columns with M >= 16384).
THIN_M = [(0, 0, 1, 24576, 4096), (1, 0, 3, 16388, 6147), (0, 0, 8, 8196, 12288)]
THIN_N = [(0, 0, 4096, 1, 1024), (0, 0, 4100, 1, 1028), (0, 1, 16385, 2, 6144), (0, 0, 12289, 5, 8196),
          (0, 1, 8193, 8, 12288), (0, 0, 8200, 3, 8192), (0, 1, 8210, 4, 8196), (0, 0, 16390, 1, 1028),
          (0, 1, 16401, 2, 4100)]
# The large operand stored with K contiguous on the other side (B stored
# N x K with M <= 8, A stored K x M with N <= 8, 384 MB or more): the
# transposed product on the thin kernels, stored transposed, split
# (reduction into C transposed) and whole.
THIN_T = [(0, 1, 1, 24576, 4096), (1, 1, 5, 16388, 6148), (1, 0, 98308, 1, 1028), (1, 0, 16392, 2, 8192),
          (1, 1, 12292, 7, 8200), (0, 1, 1, 24576, 4097)]
# The streamed operand's rows not in 16-byte chunks (K or N odd): thin_n and
# thin_m with 4-byte loads, direct and transposed; from 16 MB for up to 4
# rows or columns of C.
THIN_U = [(0, 0, 16384, 1, 16383), (0, 1, 12289, 3, 8191), (0, 0, 100003, 4, 1023), (0, 0, 1, 16383, 16384),
          (1, 0, 3, 24575, 4097), (1, 0, 16383, 1, 16384), (0, 0, 2, 65535, 4096), (0, 0, 1, 4095, 4096),
          (0, 0, 4096, 3, 2047)]


@pytest.mark.parametrize("case", THIN_M + THIN_N + THIN_T + THIN_U, ids=lambda c: "{}{}-{}x{}x{}".format(*c))
def test_thin_uniform(case):
    ta, tb, M, N, K = case
    for alpha, beta in [(1.0, 0.0), (-1.5, 0.75)]:
        got, ref, S, E, _ = run_thin(ta, tb, M, N, K, alpha, beta, "uniform", seed=M + N + K)
        rep = check.check_ex(got, ref, S, E, K)
        assert rep["ok"], rep


@pytest.mark.parametrize("case", THIN_M + THIN_N + THIN_T + THIN_U, ids=lambda c: "{}{}-{}x{}x{}".format(*c))
def test_thin_integer_exact(case):
    ta, tb, M, N, K = case
    for alpha, beta in [(1.0, 0.0), (2.0, -1.0)]:
        got, ref, _, _, _ = run_thin(ta, tb, M, N, K, alpha, beta, "int", seed=3 * M + K)
        assert np.array_equal(got.astype(np.float64), ref), (case, alpha, beta)


def test_thin_split_and_whole_chunks():
    # The same thin shapes with K split across workgroups and unsplit.
    splits = {}
    for case in [(0, 0, 8, 16384, 8192), (0, 0, 8192, 1, 8192), (0, 0, 100000, 4, 1024)]:
        _, _, M, N, K = case
        got, ref, S, E, plan = run_thin(*case, 1.0, 0.0, "uniform", seed=11)
        splits[(M, N, K)] = plan["splits"]
        assert check.check_ex(got, ref, S, E, K)["ok"]
    assert splits[(8, 16384, 8192)] > 1 and splits[(8192, 1, 8192)] > 1
    assert splits[(100000, 4, 1024)] == 1


def test_thin_repeated_calls_identical():
    A, B = make_operands(4, 16384, 8192, "uniform", 12)
    Ad, Bd = A.cuda(), B.cuda()
    assert rs.plan_config(4, 16384, 8192, A_ptr=Ad.data_ptr(), B_ptr=Bd.data_ptr())["engine"] == "thin"
    outs = []
    for _ in range(3):
        C = torch.empty((4, 16384), device="cuda")
        rs.sgemm(Ad, Bd, out=C)
        outs.append(C)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("case", [(0, 0, 2, 16384, 8192), (0, 0, 8192, 3, 8192), (0, 0, 4100, 1, 1028)],
                         ids=lambda c: "{}{}-{}x{}x{}".format(*c))
def test_thin_padded_ldc(case):
    # C with a leading dimension past N: the padding columns and the tail
    # keep their sentinel; split (workspace, then the reduction) and unsplit
    # thin calls alike.
    ta, tb, M, N, K = case
    A, B = make_operands(M, N, K, "uniform", seed=21)
    C0 = make_operands(M, 1, N, "uniform", seed=22)[0]
    Ad, Bd = to_device(A.contiguous()), to_device(B.contiguous())
    plan = rs.plan_config(M, N, K, A_ptr=Ad.data_ptr(), B_ptr=Bd.data_ptr())
    note(f"[thin-ldc] {M}x{N}x{K} plan={plan}")
    assert plan["engine"] == "thin", plan
    ldc = N + 3
    Cbuf = torch.full((M * ldc + 16,), 555.0, device="cuda")
    Cd = torch.as_strided(Cbuf, (M, N), (ldc, 1))
    Cd.copy_(C0)
    st = rs.load().sgemm_f32_ex(0, 0, M, N, K, 1.25, Ad.data_ptr(), Ad.stride(0), Bd.data_ptr(),
                                Bd.stride(0), -0.5, Cbuf.data_ptr(), ldc,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0, rs.status_string(st)
    torch.cuda.synchronize()
    full = Cbuf[:M * ldc].view(M, ldc).cpu()
    assert torch.all(full[:, N:] == 555.0) and torch.all(Cbuf[M * ldc:].cpu() == 555.0), "wrote outside C"
    ref, S, E = oracle.sgemm_ex_f64(0, 0, 1.25, as_numpy(A), as_numpy(B), -0.5, as_numpy(C0))
    rep = check.check_ex(full[:, :N].numpy(), ref, S, E, K)
    assert rep["ok"], rep


@pytest.mark.parametrize("case", [(0, 1, 2, 16384, 8192), (1, 0, 16392, 3, 8192)],
                         ids=lambda c: "{}{}-{}x{}x{}".format(*c))
def test_thin_transposed_padded_ldc(case):
    # A transposed thin product stores C transposed: into a C whose leading
    # dimension is past N, leaving the padding and the tail untouched.
    ta, tb, M, N, K = case
    A, B = make_operands(M, N, K, "int", seed=31)
    C0 = make_operands(M, 1, N, "int", seed=32)[0]
    As = A.t().contiguous() if ta else A.contiguous()
    Bs = B.t().contiguous() if tb else B.contiguous()
    Ad, Bd = to_device(As), to_device(Bs)
    plan = rs.plan_config(M, N, K, transa=bool(ta), transb=bool(tb), lda=Ad.stride(0), ldb=Bd.stride(0),
                          A_ptr=Ad.data_ptr(), B_ptr=Bd.data_ptr())
    note(f"[thin-t-ldc] {ta}{tb} {M}x{N}x{K} plan={plan}")
    assert plan["engine"] == "thin", plan
    ldc = N + 3
    Cbuf = torch.full((M * ldc + 16,), 555.0, device="cuda")
    Cd = torch.as_strided(Cbuf, (M, N), (ldc, 1))
    Cd.copy_(C0)
    st = rs.load().sgemm_f32_ex(ta, tb, M, N, K, 2.0, Ad.data_ptr(), Ad.stride(0), Bd.data_ptr(),
                                Bd.stride(0), -1.0, Cbuf.data_ptr(), ldc,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0, rs.status_string(st)
    torch.cuda.synchronize()
    full = Cbuf[:M * ldc].view(M, ldc).cpu()
    assert torch.all(full[:, N:] == 555.0) and torch.all(Cbuf[M * ldc:].cpu() == 555.0), "wrote outside C"
    ref, _, _ = oracle.sgemm_ex_f64(ta, tb, 2.0, as_numpy(As), as_numpy(Bs), -1.0, as_numpy(C0))
    assert np.array_equal(full[:, :N].numpy().astype(np.float64), ref)


@pytest.mark.parametrize("shape", [(1, 16384, 16384), (16384, 1, 16384)], ids=["thin_m", "thin_n"])
def test_explicit_k4_mfma_stays_on_matrix_cores(shape):
    """SGEMM_K4_MFMA runs the matrix-core kernel even where AUTO streams the
    product through the thin kernels: both meet the bound (integer operands:
    both exact), and on uniform operands their results differ, as two
    different summation orders do (both kernels are deterministic, so the
    difference is a property of these seeds, not chance)."""
    M, N, K = shape
    assert rs.plan_config(M, N, K, A_ptr=1 << 40, B_ptr=1 << 40)["engine"] == "thin"
    from tests.gpu_util import run
    A, B = make_operands(M, N, K, "int", seed=M + 2)
    ref, _ = oracle.sgemm_f64(as_numpy(A), as_numpy(B), bound=False)
    for v in ("auto", "k4_mfma"):
        note(f"[thin-vs-k4] {v} {M}x{N}x{K} int")
        C, out = run(v, A, B)
        assert out.guard_intact() and np.array_equal(C.astype(np.float64), ref), v
    A, B = make_operands(M, N, K, "uniform", seed=M + 3)
    ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    got = {}
    for v in ("auto", "k4_mfma"):
        note(f"[thin-vs-k4] {v} {M}x{N}x{K} uniform")
        got[v], _ = run(v, A, B)
        assert check.check(got[v], ref, S, K)["ok"], v
    assert not np.array_equal(got["auto"], got["k4_mfma"])
