"""Roofline report: classification against the ridge point and the 2 x 2
memory/compute table of the bandwidth-and-peak exercises."""
import math

import pytest

from roofline_sgemm_f32_amd import report
from roofline_sgemm_f32_amd import metrics as m

PEAK, BW = m.MI355X_FP32_PEAK_GFLOPS / 1e3, m.MI355X_HBM_GBS


def test_copy_is_memory_bound_and_fma_probe_compute_bound():
    # A copy moves bytes and does no arithmetic: it sits on the slope, with a
    # high memory percentage and ~0 compute; an FMA chain the reverse.
    copy = report.classify(report.Point("copy", 0.33, 0.0, 1073.7, 1073.7), PEAK, BW)
    fma = report.classify(report.Point("fma", 1.0, 1.37e11, 0.0, 33.5), PEAK, BW)
    assert copy["bound"] == "memory" and copy["mem_pct"] > 80 and copy["compute_pct"] == 0
    assert fma["bound"] == "compute" and fma["compute_pct"] > 80 and fma["mem_pct"] < 1


def test_ridge_and_roof():
    ridge = m.ridge_flop_per_byte(PEAK * 1e3, BW)
    # Just below the ridge the roof is the slope, just above it the flat roof.
    below = report.classify(report.Point("a", 1.0, ridge * 0.5 * 1e9, 1e3, 0.0), PEAK, BW)
    above = report.classify(report.Point("b", 1.0, ridge * 2 * 1e9, 1e3, 0.0), PEAK, BW)
    assert below["bound"] == "memory" and below["roof_tflops"] == pytest.approx(PEAK / 2)
    assert above["bound"] == "compute" and above["roof_tflops"] == pytest.approx(PEAK)


def test_sgemm_intensity_from_counts():
    # 137.4 GFLOP over 201.3 MB (A, B read once, C written once) = 683 FLOP/B.
    p = report.Point("sgemm", 1.0, 2 * 4096 ** 3, 134.2, 67.1)
    assert p.intensity == pytest.approx(2 * 4096 ** 3 / 201.3e6, rel=1e-3)
    assert report.classify(p, PEAK, BW)["bound"] == "compute"


def test_parse_and_render(tmp_path):
    t = tmp_path / "t.txt"
    t.write_text("# comment\nkernel ms TFLOP/s clk FLOP MOPS FMA util rd wr\n"
                 "k4 1.0 137 2.3 1.3744e+11 1.3744e+11 0 87.0% 735.4 77.6 169 1 0% 64 0 33280\n"
                 "copy_vec4 0.326 0.00 2.399 0.0 0.0 0.0 0.0% 1073.7 1073.7 0.0 0 0% 8 0 0\n")
    pts = report.parse_counter_table(str(t))
    assert [p.kernel for p in pts] == ["k4", "copy_vec4"]
    rows = [report.classify(p, PEAK, BW) for p in pts]
    md = report.markdown(rows, PEAK, BW, "t")
    assert "| k4 |" in md and "compute" in md and "memory" in md
    s = report.svg(rows, PEAK, BW, "t")
    assert s.startswith("<svg") and s.count("<circle") == 4


def test_small_shape_points():
    line = {"small_shapes": [
        {"shape": "square256", "M": 256, "N": 256, "K": 256, "chunks": 1, "us_per_call": 5.0,
         "unsplit_us_per_call": 5.0},
        {"shape": "kheavy", "M": 128, "N": 128, "K": 4096, "chunks": 16, "us_per_call": 13.0,
         "unsplit_us_per_call": 30.0},
        {"shape": "failed", "M": 64, "N": 64, "K": 64, "gate": False},
        {"shape": "thin", "M": 1, "N": 4096, "K": 4096, "chunks": 4, "engine": "thin",
         "us_per_call": 20.0, "unsplit_us_per_call": 30.0}]}
    pts = report.small_shape_points(line)
    assert [p.kernel for p in pts] == ["square256 (1 chunk)", "kheavy (16 chunks)", "kheavy unsplit",
                                       "thin (thin kernel, 4 chunks)", "thin matrix cores, unsplit"]
    # 2 * 256^3 FLOP in 5 us; algorithmic bytes 4 * 3 * 256^2.
    assert pts[0].tflops == pytest.approx(2 * 256 ** 3 / 5e-6 / 1e12)
    assert pts[0].intensity == pytest.approx(2 * 256 ** 3 / (12 * 256 ** 2))
    assert pts[2].ms == pytest.approx(0.030)
