"""The entry point that allocates nothing (sgemm_f32_ex_split_noalloc)
against the existing entry point it mirrors (sgemm_f32_ex_split), through the
C ABI.

Its kernels are the same, with the library's static device scratch in place
of the pool workspace, so where the plan fits the scratch the two results
must be bit-identical; where it does not (packed copies over 64 MiB) the
product runs unpacked and is checked against the CPU oracle's bound and, on
integer operands, bit for bit against the oracle.  Calls run back to back,
larger then smaller, so that each one reuses scratch contents the previous
call left behind.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import check
from roofline_sgemm_f32_amd.inputs import as_numpy, make_operands
import roofline_sgemm_f32_amd as rs

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


def _pair(M, N, K, dist, seed, splits=0, transa=False, transb=False, alpha=1.0, beta=0.0):
    """(noalloc result, existing entry point's result, host A, B, C0)."""
    A, B = make_operands(M, N, K, dist, seed)
    Ah = A.t().contiguous() if transa else A
    Bh = B.t().contiguous() if transb else B
    Ad, Bd = Ah.cuda(), Bh.cuda()
    C0 = make_operands(M, N, N, dist, seed + 1)[0] if beta else None  # an M x N matrix
    c_new = torch.full((M, N), float("nan"), device="cuda") if C0 is None else C0.cuda()
    c_old = c_new.clone()
    rs.sgemm_ex(Ad, Bd, out=c_new, transa=transa, transb=transb, alpha=alpha, beta=beta,
                splits=splits, noalloc=True)
    rs.sgemm_ex(Ad, Bd, out=c_old, transa=transa, transb=transb, alpha=alpha, beta=beta,
                splits=splits)
    torch.cuda.synchronize()
    return c_new.cpu().numpy(), c_old.cpu().numpy(), A, B


# Shapes whose scratch fits: the packed ragged product (copies about 55 MiB),
# a 16-way split of 32 x 32 tiles, an 8-way explicit split, a thin product
# split 16 ways, a model-split narrow product; largest first.
FITS = [
    ("packed3001x4099x2047", 3001, 4099, 2047, 0),
    ("split128x128x4096", 128, 128, 4096, 0),
    ("explicit256x256x16384", 256, 256, 16384, 8),
    ("thin1x16384x16384", 1, 16384, 16384, 0),
    ("narrow64x8192x8192", 64, 8192, 8192, 0),
    ("small96x80x700", 96, 80, 700, 0),
]


def test_two_calls_larger_then_smaller_bitwise():
    """The ragged packed product, then a smaller split one: both equal the
    existing entry point's result bit for bit and lie within the bound."""
    for name, M, N, K, splits in (FITS[0], FITS[1]):
        note(f"[noalloc] {name} splits={splits}")
        new, old, A, B = _pair(M, N, K, "uniform", seed=M + N + K, splits=splits)
        assert np.array_equal(new, old), f"{name}: differs from sgemm_f32_ex_split"
        ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B))
        rep = check.check(new, ref, S, K)
        assert rep["ok"], (name, rep)


@pytest.mark.parametrize("case", FITS, ids=lambda c: c[0])
def test_fits_bitwise_and_integer_exact(case):
    name, M, N, K, splits = case
    note(f"[noalloc] {name} int splits={splits}")
    new, old, A, B = _pair(M, N, K, "int", seed=3 * M + K, splits=splits)
    assert np.array_equal(new, old), f"{name}: differs from sgemm_f32_ex_split"
    if M * N * K <= 4096 ** 3:
        ref, _ = oracle.sgemm_f64(as_numpy(A), as_numpy(B), bound=False)
        assert np.array_equal(new.astype(np.float64), ref), f"{name}: not exact"


@pytest.mark.parametrize("orient", [(False, True), (True, False), (True, True)])
def test_transposed_alpha_beta_bitwise(orient):
    ta, tb = orient
    note(f"[noalloc] transposed {orient}")
    new, old, A, B = _pair(1000, 700, 3000, "uniform", seed=5, splits=4, transa=ta, transb=tb,
                           alpha=-1.25, beta=0.5)
    assert np.array_equal(new, old)


def test_over_scratch_runs_unpacked_within_bound():
    """Packed copies of 4095 x 4097 x 4093 take about 134 MB, over the static
    scratch: the product runs on 4-byte loads instead, still correct."""
    M, N, K = 4095, 4097, 4093
    assert rs.plan_config(M, N, K, A_ptr=1 << 40, B_ptr=1 << 40)["packed"]
    for dist in ("int", "uniform"):
        note(f"[noalloc] over-scratch {M}x{N}x{K} {dist}")
        new, old, A, B = _pair(M, N, K, dist, seed=7)
        ref, S = oracle.sgemm_f64(as_numpy(A), as_numpy(B), bound=dist != "int")
        if dist == "int":
            assert np.array_equal(new.astype(np.float64), ref)
            assert np.array_equal(new, old)
        else:
            assert check.check(new, ref, S, K)["ok"]
            assert check.check(old, ref, S, K)["ok"]


def test_split_over_scratch_is_refused():
    A = torch.zeros((4096, 8192), device="cuda")
    B = torch.zeros((8192, 4096), device="cuda")
    C = torch.full((4096, 4096), 7.0, device="cuda")
    with pytest.raises(rs.SgemmError) as e:
        rs.sgemm_ex(A, B, out=C, splits=2, noalloc=True)
    assert e.value.status == 9
    torch.cuda.synchronize()
    assert bool((C == 7.0).all()), "a refused call must not write C"


def test_graph_capture_replays_match_eager():
    """Captured, the call still splits (its scratch needs no allocation);
    three replays with eager work in between equal the eager call."""
    M, N, K = 128, 128, 4096
    A, B = make_operands(M, N, K, "uniform", seed=9)
    Ad, Bd = A.cuda(), B.cuda()
    eager = torch.empty((M, N), device="cuda")
    rs.sgemm_ex(Ad, Bd, out=eager, noalloc=True)
    torch.cuda.synchronize()
    out = torch.full((M, N), float("nan"), device="cuda")
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        rs.sgemm_ex(Ad, Bd, out=out, noalloc=True)
    torch.cuda.synchronize()
    other = torch.empty((64, 64), device="cuda")
    for rep in range(3):
        note(f"[noalloc] graph replay {rep}")
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
        # Eager work between replays, including a call that reuses the scratch.
        rs.sgemm_ex(torch.ones((64, 2048), device="cuda"), torch.ones((2048, 64), device="cuda"),
                    out=other, noalloc=True)
        torch.cuda.synchronize()
        assert bool((other == 2048.0).all())
