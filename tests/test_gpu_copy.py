"""GPU: the HBM copy probe copies exactly and touches nothing else."""
import pytest
import torch

import roofline_sgemm_f32_amd as rs
from roofline_sgemm_f32_amd.inputs import copy_source

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("n", [1, 3, 4, 5, 63, 64, 1000, 4097, 1 << 20, (1 << 20) + 3])
@pytest.mark.parametrize("offset", [0, 1])  # 1: 4-byte aligned only
def test_copy_exact(n, offset):
    print(f"[copy] n={n} offset={offset}", flush=True)
    src_h = copy_source(n, seed=n)
    src = torch.empty(n + 2 * offset + 8, device="cuda")
    src[offset:offset + n] = src_h.cuda()
    dst = torch.full((n + offset + 8,), 777.0, device="cuda")
    rs.copy_f32(dst[offset:offset + n], src[offset:offset + n])
    torch.cuda.synchronize()
    assert torch.equal(dst[offset:offset + n].cpu(), src_h)
    assert torch.all(dst[:offset] == 777.0) and torch.all(dst[offset + n:] == 777.0)


@pytest.mark.parametrize("block,grid", [(64, 1), (128, 7), (512, 64), (1024, 1024), (256, 4096)])
def test_copy_launch_shapes(block, grid):
    print(f"[copy-launch] block={block} grid={grid}", flush=True)
    n = 3 * (1 << 18) + 1
    src_h = copy_source(n, seed=3)
    src = src_h.cuda()
    dst = torch.zeros(n + 16, device="cuda")
    rs.copy_f32_launch(dst[:n], src, block, grid)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n].cpu(), src_h) and torch.all(dst[n:] == 0)


def test_copy_full_size_probe():
    # The probe's own size: 256 Mi floats (1 GiB per array).
    n = 256 * 1024 * 1024
    print("[copy] full size", flush=True)
    src = torch.rand(n, device="cuda")
    dst = torch.empty_like(src)
    rs.copy_f32(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
