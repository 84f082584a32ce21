"""GPU parity of the small-shape path (split-K), through the C ABI.

sgemm_f32_ex_split cuts K into chunks whose partial products a second kernel
adds in chunk order; the result must meet the same per-element bar as every
other path against the CPU oracle (|C - C_ref| <= 4 K 2^-24 |alpha| sum|ab|
+ 2 * 2^-24 (|alpha sum ab| + |beta C0|)), and integer operands, exact in any
order, must match the oracle bit for bit.  Every call here is checked to have
split the way the host plan says (sgemm_split_plan)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import check
import roofline_sgemm_f32_amd as rs
from roofline_sgemm_f32_amd.inputs import as_numpy, make_operands, padded
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


def run_split(ta, tb, M, N, K, alpha, beta, splits, dist="uniform", seed=0, pad=0, c0_nan=False,
              stream=None):
    """C = alpha op(A) op(B) + beta C0 with a split request; returns
    (C, oracle C, S, E, chunks)."""
    A, B = make_operands(M, N, K, dist, seed)
    C0 = make_operands(M, 1, N, dist, seed + 1)[0]
    As = A.t().contiguous() if ta else A
    Bs = B.t().contiguous() if tb else B
    As, Bs = padded(As, As.shape[1] + pad), padded(Bs, Bs.shape[1] + pad)
    Ad, Bd = to_device(As), to_device(Bs)
    ldc = N + pad
    Cbuf = torch.full((M * ldc + 16,), 777.0, device="cuda")
    Cd = torch.as_strided(Cbuf, (M, N), (ldc, 1))
    Cd.copy_(torch.full((M, N), float("nan")) if c0_nan else C0)
    chunks, _ = rs.split_plan(M, N, K, transa=ta, transb=tb, lda=Ad.stride(0), ldb=Bd.stride(0),
                              A_ptr=Ad.data_ptr(), B_ptr=Bd.data_ptr(), splits=splits)
    s = stream if stream is not None else torch.cuda.current_stream()
    torch.cuda.synchronize()
    st = rs.load().sgemm_f32_ex_split(int(ta), int(tb), M, N, K, alpha, Ad.data_ptr(), Ad.stride(0),
                                      Bd.data_ptr(), Bd.stride(0), beta, Cbuf.data_ptr(), ldc,
                                      splits, s.cuda_stream)
    assert st == 0, rs.status_string(st)
    torch.cuda.synchronize()
    got = Cd.cpu().numpy()
    assert torch.all(Cbuf[M * ldc:].cpu() == 777.0), "wrote past C"
    if pad:
        assert torch.all(torch.as_strided(Cbuf, (M, pad), (ldc, 1), N).cpu() == 777.0), "wrote into padding"
    ref, S, E = oracle.sgemm_ex_f64(ta, tb, alpha, as_numpy(As), as_numpy(Bs), beta,
                                    None if beta == 0 else as_numpy(C0))
    return got, ref, S, E, chunks


SHAPES = [(64, 64, 64), (33, 65, 257), (129, 257, 1000), (256, 256, 256), (100, 60, 2047),
          (7, 5, 300), (300, 17, 129)]


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)], ids=["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_split_uniform(ta, tb, shape):
    M, N, K = shape
    for splits in (2, 3, 7, rs.MAX_SPLITS):
        for alpha, beta in [(1.0, 0.0), (-1.5, 2.0)]:
            note(f"[split] {ta}{tb} {M}x{N}x{K} splits={splits} alpha={alpha} beta={beta}")
            got, ref, S, E, chunks = run_split(ta, tb, M, N, K, alpha, beta, splits,
                                               seed=M + K + splits, pad=splits % 3)
            assert chunks > 1 or K <= 32
            rep = check.check_ex(got, ref, S, E, K)
            assert rep["ok"], (splits, chunks, rep)


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 1)], ids=["NN", "TT"])
@pytest.mark.parametrize("shape", [(64, 64, 1024), (129, 257, 1000), (31, 33, 4099)],
                         ids=lambda s: "x".join(map(str, s)))
def test_split_integer_exact(ta, tb, shape):
    M, N, K = shape
    for splits in (2, 5, 16):
        got, ref, _, _, chunks = run_split(ta, tb, M, N, K, 2.0, -1.0, splits, dist="int", seed=splits)
        assert chunks > 1
        assert np.array_equal(got.astype(np.float64), ref), (splits, chunks)


def test_split_beta_zero_does_not_read_c():
    got, ref, S, E, chunks = run_split(0, 0, 70, 90, 500, 1.25, 0.0, 4, c0_nan=True)
    assert chunks == 4 and np.isfinite(got).all()
    assert check.check_ex(got, ref, S, E, 500)["ok"]


def test_split_one_is_the_unsplit_kernel():
    # splits = 1 runs the unsplit kernel; splits = 0 and the plain entry
    # point run the same split plan, bit for bit.
    M, N, K = 128, 128, 4096
    assert rs.split_plan(M, N, K, A_ptr=1 << 40, B_ptr=1 << 40)[0] > 1
    A, B = make_operands(M, N, K, "uniform", 3)
    Ad, Bd = A.cuda(), B.cuda()
    C1 = rs.sgemm_ex(Ad, Bd, splits=1)
    C2 = rs.sgemm_ex(Ad, Bd, splits=0)
    C3 = rs.sgemm_ex(Ad, Bd)
    torch.cuda.synchronize()
    assert torch.equal(C2, C3)
    ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    for C in (C1, C2):
        assert check.check(C.cpu().numpy(), ref, S, K)["ok"]


# Shapes the shape-chosen plan splits, at full size through the plain entry
# point sgemm_f32 (AUTO): every element against the oracle.
AUTO_SPLIT = [(256, 256, 768, 3), (128, 128, 1024, 4), (128, 128, 4096, 16), (256, 256, 16384, 8),
              (256, 256, 2048, 8), (64, 64, 65536, 32), (512, 512, 4096, 2), (200, 120, 3000, 0),
              # 64 x 64 tiles split by the cost model
              (64, 8192, 8192, 8), (192, 8192, 8192, 4), (1536, 1024, 1024, 2), (768, 768, 4096, 7)]


@pytest.mark.parametrize("M,N,K,want", AUTO_SPLIT, ids=lambda v: str(v))
def test_auto_split_full(M, N, K, want):
    A, B = make_operands(M, N, K, "uniform", M + N + K)
    Ad, Bd = A.cuda(), B.cuda()
    chunks, _ = rs.split_plan(M, N, K, A_ptr=Ad.data_ptr(), B_ptr=Bd.data_ptr())
    if want:
        assert chunks == want
    else:
        assert chunks > 1  # unaligned N: the 4-byte-load configuration splits too
    note(f"[auto-split] {M}x{N}x{K} chunks={chunks}")
    C = torch.full((M, N), float("nan"), device="cuda")
    st = rs.sgemm_f32(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, C.data_ptr(), N,
                      torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    rep = check.check(C.cpu().numpy(), ref, S, K)
    assert rep["ok"], rep


def test_workspace_reuse_across_sizes_and_streams():
    # Stream-ordered workspace: back-to-back calls of different sizes on two
    # streams, then every result checked.
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    cases = [(256, 256, 8192, s1), (64, 64, 4096, s2), (512, 512, 1024, s1), (128, 96, 2000, s2),
             (256, 256, 8192, s2)]
    outs = []
    for i, (M, N, K, s) in enumerate(cases):
        A, B = make_operands(M, N, K, "uniform", 40 + i)
        with torch.cuda.stream(s):
            Ad, Bd = A.cuda(), B.cuda()
            C = torch.empty((M, N), device="cuda")
        assert rs.split_plan(M, N, K, A_ptr=Ad.data_ptr(), B_ptr=Bd.data_ptr())[0] > 1
        st = rs.load().sgemm_f32_ex_split(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N,
                                          0.0, C.data_ptr(), N, 0, s.cuda_stream)
        assert st == 0
        outs.append((A, B, Ad, Bd, C))
    torch.cuda.synchronize()
    for A, B, _, _, C in outs:
        ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
        assert check.check(C.cpu().numpy(), ref, S, A.shape[1])["ok"]


def test_split_repeated_calls_identical():
    # Fixed chunk order: the same call twice gives the same bits.
    A, B = make_operands(96, 80, 5000, "normal", 11)
    Ad, Bd = A.cuda(), B.cuda()
    C1 = rs.sgemm_ex(Ad, Bd, splits=8)
    C2 = rs.sgemm_ex(Ad, Bd, splits=8)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


# One shape per tile configuration of the plan, split on request: 64 x 64
# tiles with 4 K groups (16-byte loads, under 256 tiles), 32 x 32 with 4 K
# groups (16-byte loads up to 768 tiles with a short K, and 4-byte loads),
# 64 x 64 (512 tiles and more), with both load widths.
CONFIG_SHAPES = [(1024, 960, 300), (640, 576, 300), (641, 577, 301), (2048, 1024, 256), (2049, 1023, 255)]


@pytest.mark.parametrize("shape", CONFIG_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 1)], ids=["NN", "TT"])
def test_split_every_config(shape, ta, tb):
    M, N, K = shape
    for splits in (2, 5):
        note(f"[split-cfg] {ta}{tb} {M}x{N}x{K} splits={splits}")
        got, ref, _, _, chunks = run_split(ta, tb, M, N, K, 1.0, 0.0, splits, dist="int", seed=splits)
        assert 1 < chunks <= splits  # whole slabs: K = 256 in slabs of 32 takes 4 chunks for 5
        assert np.array_equal(got.astype(np.float64), ref), (splits, chunks)
        got, ref, S, E, _ = run_split(ta, tb, M, N, K, 0.75, -1.25, splits, seed=M + splits)
        rep = check.check_ex(got, ref, S, E, K)
        assert rep["ok"], rep
