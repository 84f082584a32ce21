"""Throughput and roofline arithmetic against the numbers the pages print."""
import os

import pytest

from roofline_sgemm_f32_amd import metrics as m

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _table():
    rows = []
    with open(os.path.join(GOLDEN, "page_results_table.txt")) as f:
        for ln in f:
            if ln.startswith("#") or not ln.strip():
                continue
            n, name, ms, gf, pct, sp = ln.split()
            rows.append((int(n), name, float(ms), float(gf), float(pct), float(sp)))
    return rows


def test_flop_count_n4096():
    # Printed: 2 * 4096^3 = 2 * 68,719,476,736 ~ 1.374e11, "about 137.4 GFLOP".
    assert 4096 ** 3 == 68_719_476_736
    assert m.sgemm_flops(4096, 4096, 4096) == 137_438_953_472
    assert round(m.sgemm_flops(4096, 4096, 4096) / 1e9, 1) == 137.4


def test_flop_count_is_2mnk_for_rectangles():
    assert m.sgemm_flops(3001, 4099, 2047) == 2 * 3001 * 4099 * 2047 == 50_360_699_306
    assert m.sgemm_flops(0, 5, 7) == 0


def test_h100_peak_formula():
    # 132 SMs x 128 FP32 lanes x 2 FLOP per FFMA x 1.98 GHz ~ 66.9 TFLOP/s.
    peak = m.peak_gflops(m.H100_SMS, m.H100_FP32_LANES, m.H100_BOOST_GHZ)
    assert peak == pytest.approx(66908.16)
    assert round(peak / 100) * 100 == m.H100_FP32_PEAK_GFLOPS_PAGE


def test_forgetting_fma_counts_two_halves_the_peak():
    # The exercise's trap: one FLOP per FMA gives half the true figure (50 % low).
    one = m.H100_SMS * m.H100_FP32_LANES * 1 * m.H100_BOOST_GHZ
    assert one / m.peak_gflops(m.H100_SMS, m.H100_FP32_LANES, m.H100_BOOST_GHZ) == 0.5


@pytest.mark.parametrize("row", _table(), ids=lambda r: r[1])
def test_page_results_table_reproduced(row):
    n, name, ms, gf, pct, sp = row
    flops = m.sgemm_flops(n, n, n)
    g = m.gflops(flops, ms)
    assert round(g) == pytest.approx(gf, abs=1)
    assert round(m.pct_of_peak(g, m.H100_FP32_PEAK_GFLOPS_PAGE), 1) == pct
    assert round(m.speedup(68.0, ms), 1) == sp


def test_mi355x_peak():
    # 256 CUs x 128 FP32 FMA per clock x 2 FLOP x 2.4 GHz = 157.3 TFLOP/s.
    assert m.MI355X_FP32_PEAK_GFLOPS == pytest.approx(157286.4)
    # 70 % of that peak at N = 4096 means at most 1.248 ms per product.
    ms = m.sgemm_flops(4096, 4096, 4096) / (0.7 * m.MI355X_FP32_PEAK_GFLOPS * 1e9) * 1e3
    assert ms == pytest.approx(1.2483, abs=1e-4)


def test_copy_bytes_and_bandwidth():
    # One read and one write per element: 2 x n x sizeof(float).
    n = 256 * 1024 * 1024
    assert m.copy_bytes(n) == 2 * n * 4 == 2 * 1024 ** 3
    # At the H100's 3.35 TB/s that copy would take about 0.64 ms.
    assert m.gbs(m.copy_bytes(n), 0.641) == pytest.approx(3350, rel=2e-3)


def test_ridge_points():
    # BF16 tensor and FP8 tensor peaks over 3.35 TB/s: about 295 and 591 FLOP/B.
    assert m.ridge_flop_per_byte(989e3, 3350) == pytest.approx(295, abs=0.5)
    assert m.ridge_flop_per_byte(1979e3, 3350) == pytest.approx(591, abs=0.5)
    # MI355X FP32 against 8 TB/s.
    assert m.ridge_flop_per_byte(m.MI355X_FP32_PEAK_GFLOPS, m.MI355X_HBM_GBS) == pytest.approx(19.66, abs=0.01)


def test_scalar_times_vector_intensity():
    # y = a * x: one FLOP per 8 bytes moved.
    assert m.arithmetic_intensity(1, 8) == 0.125


def test_sgemm_intensity_n4096():
    ai = m.arithmetic_intensity(m.sgemm_flops(4096, 4096, 4096), m.sgemm_min_bytes(4096, 4096, 4096))
    assert ai == pytest.approx(4096 * 2 / 12)
