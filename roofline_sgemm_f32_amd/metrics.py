"""Throughput and roofline arithmetic for SGEMM and the HBM copy probe.

Definitions follow the pages:
* FLOP count, throughput and percent-of-peak: amittech.dev, "3.5 Project:
  tiled matrix multiplication", section "the numeric background" (items 1-3)
  and the reporting routine in section "starter scaffolding".  A product of
  N x N matrices costs 2N per output (N multiplies, N adds) over N^2 outputs;
  for M x K times K x N that is 2MNK.
* Peak from the spec sheet: amittech.dev, "7.3 Bandwidths and peak rate -
  exercises", exercise 1 (units x lanes x 2 FLOP per fused multiply-add x
  clock).
* Copy bandwidth: the same page, exercise 2 (each element is read once and
  written once, so a copy of n floats moves 2 * n * 4 bytes).
* Ridge point: the same page, exercise 3 (arithmetic peak / memory bandwidth).
"""
from __future__ import annotations

FLOAT_BYTES = 4

# The pages' own reference machine (context only): 132 SMs x 128 FP32 lanes x
# 2 FLOP x 1.98 GHz, which the course rounds to 66 900 GFLOP/s.
H100_SMS, H100_FP32_LANES, H100_BOOST_GHZ = 132, 128, 1.98
H100_FP32_PEAK_GFLOPS_PAGE = 66900.0
H100_HBM_GBS = 3350.0

# MI355X (gfx950): 256 compute units, each retiring 128 FP32 fused
# multiply-adds per clock on the matrix cores (and, with packed FP32, on the
# vector ALUs), at a 2.4 GHz peak engine clock.  HBM3E: 8 TB/s.
MI355X_CUS = 256
MI355X_FP32_FMA_PER_CU_CLK = 128
MI355X_PEAK_GHZ = 2.4
MI355X_HBM_GBS = 8000.0


def sgemm_flops(M: int, N: int, K: int) -> int:
    """Floating-point operations of C = A * B (M x K times K x N)."""
    return 2 * int(M) * int(N) * int(K)


def sgemm_min_bytes(M: int, N: int, K: int) -> int:
    """Algorithmic HBM traffic: read A and B once, write C once."""
    return FLOAT_BYTES * (int(M) * int(K) + int(K) * int(N) + int(M) * int(N))


def gflops(flops: float, ms: float) -> float:
    """Throughput in GFLOP/s of ``flops`` done in ``ms`` milliseconds."""
    return flops / (ms / 1000.0) / 1e9


def peak_gflops(units: int, fma_lanes_per_unit: int, clock_ghz: float) -> float:
    """Peak GFLOP/s: units x lanes x 2 FLOP per fused multiply-add x clock."""
    return units * fma_lanes_per_unit * 2 * clock_ghz


def pct_of_peak(gflops_value: float, peak: float) -> float:
    return 100.0 * gflops_value / peak


def speedup(ms_base: float, ms_new: float) -> float:
    return ms_base / ms_new


def copy_bytes(n: int) -> int:
    """Bytes a device-to-device copy of n floats moves (one read, one write)."""
    return 2 * int(n) * FLOAT_BYTES


def gbs(nbytes: float, ms: float) -> float:
    """Bandwidth in GB/s (1e9 bytes per second)."""
    return nbytes / (ms / 1000.0) / 1e9


def ridge_flop_per_byte(peak_gflops_value: float, bw_gbs: float) -> float:
    """Arithmetic intensity at which a kernel moves from the memory roof to
    the compute roof."""
    return peak_gflops_value / bw_gbs


def arithmetic_intensity(flops: float, nbytes: float) -> float:
    return flops / nbytes


# AMD's published FP32 figure, the same for the vector units and the matrix
# cores.  Plain (unpacked) v_fma_f32 on vector-register operands gets close
# to it on MI355X (129-132 TFLOP/s measured by the chain probe, 32 waves per
# CU), so no separate unpacked roof applies.
MI355X_FP32_PEAK_GFLOPS = peak_gflops(MI355X_CUS, MI355X_FP32_FMA_PER_CU_CLK, MI355X_PEAK_GHZ)
