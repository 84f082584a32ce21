"""Graph capture of the C ABI entry points.

Every entry point can be captured into a HIP graph (torch.cuda.graph over
the caller's stream): captured calls skip the library workspace (split-K and
operand packing), so they run the unsplit kernel on the operands as stored.
Each graph is replayed several times with eager work in between, and every
replay must equal the eager unsplit call bit for bit (and the oracle within
the bound)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import check
import roofline_sgemm_f32_amd as rs
from roofline_sgemm_f32_amd.inputs import as_numpy, make_operands

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rs.load()
    oracle.load()


# (shape, what the eager AUTO call would do)
CASES = [((1024, 1024, 1024), "32x32 tiles with K groups, four workgroups per CU"),
         ((1024, 1024, 4096), "64x64 tiles with K groups"),
         ((4096, 4096, 1024), "128x256 tiles"),
         ((128, 128, 4096), "split-K when eager"),
         ((1601, 1283, 97), "packed operands when eager"),
         ((300, 260, 170), "32x32 tiles with K groups")]


def call(lib, A, B, C, splits, stream):
    M, K = A.shape
    N = B.shape[1]
    st = lib.sgemm_f32_ex_split(0, 0, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0,
                                C.data_ptr(), N, splits, stream)
    assert st == 0, rs.status_string(st)


@pytest.mark.parametrize("shape,what", CASES, ids=[c[1] for c in CASES])
def test_capture_and_replay(shape, what):
    M, N, K = shape
    lib = rs.load()
    A, B = make_operands(M, N, K, "uniform", seed=M + K)
    Ad, Bd = A.cuda(), B.cuda()
    want = torch.empty((M, N), device="cuda")
    call(lib, Ad, Bd, want, 1, torch.cuda.current_stream().cuda_stream)  # unsplit, unpacked
    other = torch.empty((M, N), device="cuda")
    out = torch.full((M, N), float("nan"), device="cuda")
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        call(lib, Ad, Bd, out, 0, torch.cuda.current_stream().cuda_stream)  # AUTO plan
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))                                   # eager work between replays
        call(lib, Ad, Bd, other, 0, torch.cuda.current_stream().cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r} differs from the eager unsplit call"
    ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    assert check.check(out.cpu().numpy(), ref, S, K)["ok"]
    assert check.check(other.cpu().numpy(), ref, S, K)["ok"]


@pytest.mark.parametrize("shape", [(4096, 1, 1024), (8192, 1, 8192)], ids=lambda s: "x".join(map(str, s)))
def test_capture_thin(shape):
    # Thin products: a captured call runs the thin kernel with one K chunk.
    # (4096, 1, 1024) takes one chunk eagerly too, so replays equal the eager
    # call; (8192, 1, 8192) splits K eagerly, so replays are checked against
    # each other and the oracle.
    M, N, K = shape
    lib = rs.load()
    A, B = make_operands(M, N, K, "uniform", seed=M + K)
    Ad, Bd = A.cuda(), B.cuda()
    plan = rs.plan_config(M, N, K, A_ptr=Ad.data_ptr(), B_ptr=Bd.data_ptr())
    assert plan["engine"] == "thin"
    eager = torch.empty((M, N), device="cuda")
    call(lib, Ad, Bd, eager, 0, torch.cuda.current_stream().cuda_stream)
    out = torch.full((M, N), float("nan"), device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        call(lib, Ad, Bd, out, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    first = None
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        if first is None:
            first = out.clone()
        assert torch.equal(out, first), f"replay {r} differs from the first"
    if plan["splits"] == 1:
        assert torch.equal(first, eager)
    ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
    assert check.check(first.cpu().numpy(), ref, S, K)["ok"]
    assert check.check(eager.cpu().numpy(), ref, S, K)["ok"]
