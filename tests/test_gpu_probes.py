"""GPU: the compute-roof probes against the CPU oracle, through the C ABI.

The multiply-add chain is deterministic IEEE arithmetic (one rounding per
step), so the GPU must equal the oracle bit for bit.  The matrix-unit probe
uses small integer operands, so every partial sum is exact and the 32 x 32
results must equal the oracle exactly; a wrong register-to-(row, column) map
would scramble them."""
import numpy as np
import pytest
import torch

import oracle
import roofline_sgemm_f32_amd as rs
from roofline_sgemm_f32_amd.inputs import probe_operands

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rs.load()
    oracle.load()


@pytest.mark.parametrize("x,y,iters", [(0.999, 0.001, 1000), (1.0, 1.0, 4096), (2.0, 0.0, 30),
                                       (-0.75, 0.25, 777), (1.0001, -0.5, 0)])
@pytest.mark.parametrize("blocks,block", [(1, 64), (7, 256), (64, 1024)])
def test_valu_probe_matches_oracle(x, y, iters, blocks, block):
    print(f"[probe-valu] x={x} y={y} iters={iters} blocks={blocks} block={block}", flush=True)
    out = rs.probe_valu(blocks, block, iters, x, y)
    torch.cuda.synchronize()
    want = oracle.fma_chain_f32(iters, x, y, rs.VALU_CHAINS)
    got = out.cpu().numpy()
    assert got.shape == (blocks * block, rs.VALU_CHAINS)
    assert np.array_equal(got, np.tile(want, (blocks * block, 1)))


@pytest.mark.parametrize("seed,iters,blocks", [(7, 1, 1), (8, 1000, 3), (9, 4096, 16), (10, 0, 2)])
def test_mfma_probe_matches_oracle(seed, iters, blocks):
    print(f"[probe-mfma] seed={seed} iters={iters} blocks={blocks}", flush=True)
    a, b = probe_operands(seed)
    out = rs.probe_mfma(a.cuda(), b.cuda(), blocks, iters)
    torch.cuda.synchronize()
    want = oracle.mfma_probe_f64(iters, a.numpy(), b.numpy())
    got = out.cpu().numpy().astype(np.float64)
    assert got.shape == (blocks * 4, 4, 32, 32)
    assert np.array_equal(got, np.broadcast_to(want, got.shape))


def test_mfma_probe_index_encoded():
    # A[i][0] = i, A[i][1] = 0, B[0][j] = j + 1, B[1][j] = 0: D[i][j] = i (j + 1).
    a = torch.zeros(64); a[:32] = torch.arange(32)
    b = torch.zeros(64); b[:32] = torch.arange(32) + 1
    out = rs.probe_mfma(a.cuda(), b.cuda(), 1, 1)
    torch.cuda.synchronize()
    want = np.outer(np.arange(32), np.arange(32) + 1)
    assert np.array_equal(out[0, 0].cpu().numpy(), want)


def test_probe_argument_errors():
    lib = rs.load()
    assert lib.sgemm_probe_valu_f32(0x1000, 0, 64, 1, 1.0, 1.0, None) == 8
    assert lib.sgemm_probe_valu_f32(0x1000, 1, 100, 1, 1.0, 1.0, None) == 8
    assert lib.sgemm_probe_valu_f32(0x1000, 1, 64, -1, 1.0, 1.0, None) == 8
    assert lib.sgemm_probe_valu_f32(None, 1, 64, 1, 1.0, 1.0, None) == 3
    assert lib.sgemm_probe_mfma_f32(0x1000, None, 0x2000, 1, 1, None) == 3
    assert lib.sgemm_probe_mfma_f32(0x1000, 0x2000, 0x3000, 0, 1, None) == 8
