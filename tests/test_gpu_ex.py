"""GPU parity of the general entry points, through the C ABI:
C = alpha op(A) op(B) + beta C in row-major (sgemm_f32_ex) and column-major
(sgemm_f32_colmajor) storage, against the CPU oracle.

Bar: |C - C_ref| <= 4 K 2^-24 |alpha| sum|ab| + 2 * 2^-24 (|alpha sum ab| +
|beta C0|) per element (oracle.check.check_ex); integer operands with small
integer alpha, beta are exact in float, so there the result must match the
oracle bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from oracle import check
import roofline_sgemm_f32_amd as rs
from roofline_sgemm_f32_amd.inputs import WORKLOADS, as_numpy, make_operands, workload_operands
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rs.load()
    oracle.load()


def stored(X: torch.Tensor, trans: bool, pad: int) -> torch.Tensor:
    """Host storage of a logical operand: X itself or its transpose, with
    `pad` NaN columns of leading-dimension padding."""
    from roofline_sgemm_f32_amd.inputs import padded
    S = X.t().contiguous() if trans else X.contiguous()
    return padded(S, S.shape[1] + pad)


def run_ex(ta, tb, M, N, K, alpha, beta, dist, seed, pad=0, c0_nan=False):
    A, B = make_operands(M, N, K, dist, seed)
    C0 = make_operands(M, 1, N, dist, seed + 1)[0]  # an M x N matrix
    As, Bs = stored(A, ta, pad), stored(B, tb, pad)
    Ad, Bd = to_device(As), to_device(Bs)
    ldc = N + pad
    Cbuf = torch.full((M * ldc + 16,), 777.0, device="cuda")
    Cd = torch.as_strided(Cbuf, (M, N), (ldc, 1))
    Cd.copy_(torch.full((M, N), float("nan")) if c0_nan else C0)
    st = rs.load().sgemm_f32_ex(int(ta), int(tb), M, N, K, alpha, Ad.data_ptr() if Ad.numel() else 0,
                                Ad.stride(0) if M * K else max(1, M if ta else K),
                                Bd.data_ptr() if Bd.numel() else 0,
                                Bd.stride(0) if K * N else max(1, K if tb else N), beta,
                                Cbuf.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream)
    assert st == 0, rs.status_string(st)
    torch.cuda.synchronize()
    got = Cd.cpu().numpy()
    tail = Cbuf[M * ldc:].cpu()
    assert torch.all(tail == 777.0), "wrote past C"
    if pad:
        padv = torch.as_strided(Cbuf, (M, pad), (ldc, 1), N).cpu()
        assert torch.all(padv == 777.0), "wrote into C's padding"
    ref, S, E = oracle.sgemm_ex_f64(ta, tb, alpha, as_numpy(As), as_numpy(Bs), beta,
                                    None if beta == 0 else as_numpy(C0))
    return got, ref, S, E


# With unpadded (16-byte) operands 640 x 576 x 300 runs on 32 x 32 tiles with
# K groups and 1024 x 960 x 300 on 64 x 64 tiles with K groups, in every
# orientation; the padded (4-byte) runs take the 32 x 32 configuration.
SHAPES = [(1, 1, 1), (7, 5, 3), (33, 65, 17), (129, 257, 33), (300, 17, 129), (256, 256, 256),
          (65, 129, 257), (640, 576, 300), (1024, 960, 300)]
COEFS = [(1.0, 0.0), (2.0, 0.5), (-1.5, -2.0), (0.0, 3.0)]


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)], ids=["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ex_uniform(ta, tb, shape):
    M, N, K = shape
    for alpha, beta in COEFS:
        print(f"[ex] {ta}{tb} {M}x{N}x{K} alpha={alpha} beta={beta}", flush=True)
        got, ref, S, E = run_ex(ta, tb, M, N, K, alpha, beta, "uniform", seed=M + N + K, pad=3)
        rep = check.check_ex(got, ref, S, E, K)
        assert rep["ok"], rep


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)], ids=["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ex_integer_exact(ta, tb, shape):
    M, N, K = shape
    for alpha, beta in [(1.0, 0.0), (2.0, -1.0), (-3.0, 0.5)]:
        got, ref, _, _ = run_ex(ta, tb, M, N, K, alpha, beta, "int", seed=7 * M + K)
        assert np.array_equal(got.astype(np.float64), ref), (ta, tb, alpha, beta)


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 1)], ids=["NN", "TT"])
def test_ex_beta_zero_does_not_read_c(ta, tb):
    got, ref, S, E = run_ex(ta, tb, 70, 90, 50, 1.25, 0.0, "uniform", seed=3, c0_nan=True)
    assert np.isfinite(got).all() and check.check_ex(got, ref, S, E, 50)["ok"]


def test_ex_alpha_zero_and_k_zero_scale_c():
    got, ref, S, E = run_ex(0, 0, 40, 30, 20, 0.0, -2.5, "uniform", seed=4)
    assert check.check_ex(got, ref, S, E, 20)["ok"]
    got, ref, S, E = run_ex(0, 0, 40, 30, 0, 1.0, 0.5, "uniform", seed=5)
    assert check.check_ex(got, ref, S, E, 0)["ok"]
    got, ref, _, _ = run_ex(1, 1, 40, 30, 0, 1.0, 0.0, "uniform", seed=6, c0_nan=True)
    assert np.all(got == 0)


def test_ex_offsets_beyond_32_bits_use_the_64_bit_kernel():
    # A stored K x M with a leading dimension whose 31 rows of offsets exceed
    # the matrix-core kernel's 32-bit buffer range: the general 64-bit kernel
    # takes it.
    M, N, K, lda = 50, 40, 3, 20_000_000
    A, B = make_operands(M, N, K, "int", seed=8)
    Abuf = torch.zeros(K * lda, device="cuda")
    Av = torch.as_strided(Abuf, (K, M), (lda, 1))
    Av.copy_(A.t())
    Bd = B.cuda()
    C = torch.empty((M, N), device="cuda")
    st = rs.load().sgemm_f32_ex(1, 0, M, N, K, 1.0, Abuf.data_ptr(), lda, Bd.data_ptr(), N, 0.0,
                                C.data_ptr(), N, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    want = np.matmul(as_numpy(A).astype(np.int64), as_numpy(B).astype(np.int64))
    assert np.array_equal(C.cpu().numpy().astype(np.int64), want)


# --- column-major -----------------------------------------------------------

def colmajor(X: torch.Tensor) -> torch.Tensor:
    """A column-major GPU copy of a logical matrix (stride(0) == 1)."""
    return X.t().contiguous().cuda().t()


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)], ids=["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("shape", [(33, 65, 17), (129, 100, 257), (5, 7, 3)], ids=lambda s: "x".join(map(str, s)))
def test_colmajor(ta, tb, shape):
    m, n, k = shape
    A, B = make_operands(m, n, k, "uniform", seed=m * n)
    C0 = make_operands(m, 1, n, "uniform", seed=9)[0]
    Ag = colmajor(A.t() if ta else A)   # stored k x m when transposed
    Bg = colmajor(B.t() if tb else B)
    Cg = colmajor(C0)
    rs.sgemm_colmajor(Ag, Bg, Cg, transa=bool(ta), transb=bool(tb), alpha=1.5, beta=-0.5)
    torch.cuda.synchronize()
    got = Cg.cpu().numpy()
    ref, S, E = oracle.sgemm_ex_f64(False, False, 1.5, as_numpy(A.contiguous()),
                                    as_numpy(B.contiguous()), -0.5, as_numpy(C0.contiguous()))
    rep = check.check_ex(got, ref, S, E, k)
    assert rep["ok"], rep


def test_colmajor_operand_swap_gives_the_rowmajor_product():
    # The course's trick: a row-major C = A B through the column-major entry
    # point by passing B first.  It must equal the row-major call bit for bit.
    M, N, K = 300, 260, 170
    A, B = make_operands(M, N, K, "uniform", seed=10)
    Ad, Bd = A.cuda(), B.cuda()
    C1 = torch.empty((M, N), device="cuda")
    C2 = torch.empty((M, N), device="cuda")
    lib = rs.load()
    s = torch.cuda.current_stream().cuda_stream
    assert lib.sgemm_f32_colmajor(0, 0, N, M, K, 1.0, Bd.data_ptr(), N, Ad.data_ptr(), K, 0.0,
                                  C1.data_ptr(), N, s) == 0
    assert lib.sgemm_f32_ex(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0,
                            C2.data_ptr(), N, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    assert check.check(C1.cpu().numpy(), ref, S, K)["ok"]


# --- full size, transposed operands ----------------------------------------

@pytest.mark.parametrize("ta,tb", [(0, 1), (1, 0), (1, 1)], ids=["NT", "TN", "TT"])
def test_ex_square4096_sampled(ta, tb):
    w = WORKLOADS["square4096"]
    A, B = workload_operands(w)
    As = A.t().contiguous() if ta else A
    Bs = B.t().contiguous() if tb else B
    print(f"[ex4096] {ta}{tb}", flush=True)
    C = rs.sgemm_ex(As.cuda(), Bs.cuda(), transa=bool(ta), transb=bool(tb))
    torch.cuda.synchronize()
    Cn = C.cpu().numpy()
    assert np.isfinite(Cn).all()
    rows = np.array([0, 1, 127, 128, 2049, 4095])
    ref, S = oracle.sgemm_rows_f64(as_numpy(A), as_numpy(B), rows)
    assert check.check(Cn[rows], ref, S, w.K)["ok"]
    cols = np.array([0, 63, 64, 3000, 4095])
    ref, S = oracle.sgemm_f64(as_numpy(A), np.ascontiguousarray(as_numpy(B)[:, cols]))
    assert check.check(Cn[:, cols], ref, S, w.K)["ok"]


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)], ids=["NN", "NT", "TN", "TT"])
def test_ex_128x256_every_orientation(ta, tb):
    # 512 tiles of 128 x 256 with a short K: the largest tiles in each storage
    # orientation, every element against the oracle, integer-exact and
    # uniform with alpha, beta.
    M, N, K = 2048, 8192, 72
    plan = rs.plan_config(M, N, K, transa=bool(ta), transb=bool(tb), lda=M if ta else K,
                          ldb=K if tb else N, A_ptr=1 << 40, B_ptr=1 << 40)
    print(f"[ex128x256] {ta}{tb} plan {plan}", flush=True)
    assert plan["tile"] == (128, 256), plan
    got, ref, _, _ = run_ex(ta, tb, M, N, K, 1.0, 0.0, "int", seed=11)
    assert np.array_equal(got.astype(np.float64), ref)
    got, ref, S, E = run_ex(ta, tb, M, N, K, -0.75, 1.5, "uniform", seed=12)
    rep = check.check_ex(got, ref, S, E, K)
    assert rep["ok"], rep


# Outputs large enough for 64 x 64 tiles whose operands do not suit 16-byte
# loads are packed into zero-padded aligned copies first: both operands, only
# A (K odd), only B (N odd), in every orientation.
PACKED = [(1601, 1283, 97), (1600, 1283, 96), (1601, 1284, 97)]


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)], ids=["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("shape", PACKED, ids=lambda s: "x".join(map(str, s)))
def test_ex_packed_operands(ta, tb, shape):
    M, N, K = shape
    print(f"[packed] {ta}{tb} {M}x{N}x{K}", flush=True)
    got, ref, _, _ = run_ex(ta, tb, M, N, K, 2.0, -1.0, "int", seed=M + K)
    assert np.array_equal(got.astype(np.float64), ref)
    got, ref, S, E = run_ex(ta, tb, M, N, K, 1.5, 0.5, "uniform", seed=N + K, pad=1)
    rep = check.check_ex(got, ref, S, E, K)
    assert rep["ok"], rep


@pytest.mark.parametrize("shape", [(767, 769, 4095), (513, 511, 8193), (1025, 1025, 2047), (511, 513, 4095),
                                   (600, 601, 1600)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ex_heavy_mid_size_packed(shape):
    # Mid-size outputs with a long K and unaligned operands: 4 GFLOP or more,
    # or 1 GFLOP or more with K >= 1536, so the plan copies both operands and
    # splits K on the copies.
    M, N, K = shape
    plan = rs.plan_config(M, N, K, A_ptr=1 << 40, B_ptr=1 << 40)
    print(f"[heavy packed] {M}x{N}x{K} plan {plan}", flush=True)
    assert plan["packed"] and plan["splits"] > 1
    got, ref, _, _ = run_ex(0, 0, M, N, K, 2.0, -1.0, "int", seed=M + 3)
    assert np.array_equal(got.astype(np.float64), ref)
    got, ref, S, E = run_ex(0, 0, M, N, K, 1.0, 0.5, "uniform", seed=M + 4)
    rep = check.check_ex(got, ref, S, E, K)
    assert rep["ok"], rep


def test_ex_packed_and_split():
    # Unaligned operands whose packed copies get a split plan (600 tiles of
    # 64 x 64, under 4 per CU, K = 4095): packing and split share one
    # workspace.
    M, N, K = 1535, 1537, 4095
    print(f"[packed+split] {M}x{N}x{K}", flush=True)
    got, ref, _, _ = run_ex(0, 0, M, N, K, 2.0, -1.0, "int", seed=5)
    assert np.array_equal(got.astype(np.float64), ref)
    got, ref, S, E = run_ex(0, 0, M, N, K, 1.0, 0.0, "uniform", seed=6)
    rep = check.check_ex(got, ref, S, E, K)
    assert rep["ok"], rep
