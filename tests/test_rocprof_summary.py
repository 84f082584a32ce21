"""The rocprofv3 CSV -> profiles/ summary step on tiny hand-made fixtures
(no GPU): copy-probe calibration, counted FLOP and bytes, the traffic file
bench.py reads, the wave-cycle breakdown and the headline's timed dispatches
in the kernel trace."""
import csv
import json
import os

import pytest

from roofline_sgemm_f32_amd import report, rocprof

HEAD = ("void sgemm::k4_mfma<sgemm::k4::Cfg<2, 2, 2, 4, 16, true, true, false, 2>, 2, 8, true, false, "
        "false, 1, true>(int, int, int, float const*, int, float const*, int, float*, long, float, float, "
        "int, int, int, int)")
COPY = "sgemm::copy_vec4(float*, float const*, long)"
GIB = 1 << 30


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp", "VGPR_Count", "Accum_VGPR_Count", "LDS_Block_Size"]
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for i, (kern, counters, ns) in enumerate(rows):
            for c, v in counters.items():
                w.writerow([i, kern, c, v, 1000, 1000 + ns, 128, 0, 49664])


def _fixture(out):
    # Copy probe: 1 GiB read and 1 GiB written; FETCH_SIZE reads half of it
    # (KiB), WRITE_SIZE all of it, so the scales are 2.0 and 1.0.
    copy_fetch, copy_write = GIB / 2 / 1024, GIB / 1024
    # Headline kernel: 1 ms, 137438953472 FLOP = 268435456 MOPS x 512,
    # 200 MiB fetched (counted 100 MiB x 2) and 64 MiB written.
    k_fetch, k_write = 100 * 1024, 64 * 1024
    _counter_csv(os.path.join(out, "fetch"), [(HEAD, {"FETCH_SIZE": k_fetch}, 1_000_000),
                                               (COPY, {"FETCH_SIZE": copy_fetch}, 300_000)])
    _counter_csv(os.path.join(out, "write"), [(HEAD, {"WRITE_SIZE": k_write}, 1_000_000),
                                               (COPY, {"WRITE_SIZE": copy_write}, 300_000)])
    # 8 XCDs x 2.0e6 busy clocks in 1 ms: 2.0 GHz.  MFMA busy cycles are
    # 90 % of 2.0e6 x 1024 SIMDs.
    sq = {"SQ_INSTS_VALU_MFMA_MOPS_F32": 268435456, "SQ_VALU_MFMA_BUSY_CYCLES": 0.9 * 2.0e6 * 1024,
          "SQ_LDS_BANK_CONFLICT": 0, "SQ_LDS_IDX_ACTIVE": 100, "SQ_INSTS_VALU_FMA_F32": 0, "SQ_WAVES": 2048,
          "SQ_BUSY_CYCLES": 1, "SQ_INSTS_LDS": 1e7, "GRBM_GUI_ACTIVE": 8 * 2.0e6}
    sq_copy = dict(sq, SQ_INSTS_VALU_MFMA_MOPS_F32=0, SQ_VALU_MFMA_BUSY_CYCLES=0, SQ_INSTS_LDS=0)
    _counter_csv(os.path.join(out, "sq"), [(HEAD, sq, 1_000_000), (COPY, sq_copy, 300_000)])
    # Stall pass: 2 waves per SIMD resident the whole time (wave-cycles in
    # quad-cycles: 2 x 2.0e6 x 1024 / 4), 30 % of them waiting on anything.
    wc = 2 * 2.0e6 * 1024 / 4
    st = {"SQ_WAVE_CYCLES": wc, "SQ_WAIT_ANY": 0.3 * wc, "SQ_WAIT_INST_ANY": 0.1 * wc,
          "SQ_WAIT_INST_LDS": 0.01 * wc, "SQ_ACTIVE_INST_VALU": 0.5 * wc, "SQ_ACTIVE_INST_LDS": 0.05 * wc,
          "SQ_ACTIVE_INST_VMEM": 0.02 * wc, "SQ_ACTIVE_INST_SCA": 0.03 * wc, "GRBM_GUI_ACTIVE": 8 * 2.0e6}
    _counter_csv(os.path.join(out, "stall"), [(HEAD, st, 1_000_000)])
    with open(os.path.join(out, "source_hash.txt"), "w") as f:
        f.write("0123456789abcdef\n")
    # Kernel trace of the bench: 4 square4096 dispatches (grid 512) of which
    # the last 2 are the timed ones (1.0 and 0.98 ms), 1 square8192 (2048).
    tr = os.path.join(out, "trace")
    os.makedirs(tr)
    with open(os.path.join(tr, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X",
                    "Grid_Size_Y"])
        t = 0
        for dur, grid in ((1_200_000, 512), (7_600_000, 2048), (1_100_000, 512), (1_000_000, 512),
                          (980_000, 512)):
            w.writerow([HEAD, t, t + dur, grid * 256, 256, 1])
            t += dur + 10
    with open(os.path.join(tr, "run_kernel_stats.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([HEAD, 5, 11880000, 2376000.0, 100.0, 980000, 7600000, 1.0])
    line = {"metric": "m", "value": 140000.0, "steps": 2, "ms_per_step": 0.99,
            "roofline": {"achieved": 138.8}, "hbm_copy": {"ms": 0.33, "gbs": 6500.0},
            "small_shapes": [{"shape": "square256", "M": 256, "N": 256, "K": 256, "chunks": 1,
                              "us_per_call": 5.0, "unsplit_us_per_call": 5.0}]}
    with open(os.path.join(out, "trace.log"), "w") as f:
        f.write("noise\n" + json.dumps(line) + "\n")


@pytest.fixture
def summary(tmp_path):
    out, prof = tmp_path / "out", tmp_path / "profiles"
    out.mkdir()
    prof.mkdir()
    _fixture(str(out))
    written = rocprof.summarize(str(out), str(prof))
    return prof, {os.path.basename(p) for p in written}


def test_files_written(summary):
    prof, names = summary
    assert {"ladder_square4096_counters.txt", "k4_mfma_square4096_traffic.txt",
            "k4_mfma_square4096_kernel_trace.txt", "roofline_square4096.md", "roofline_square4096.svg",
            "roofline_small_shapes.md", "roofline_small_shapes.svg"} <= names


def test_traffic_file_scaled_by_copy_probe(summary):
    prof, _ = summary
    rec = dict(ln.split(": ", 1) for ln in open(prof / "k4_mfma_square4096_traffic.txt").read().splitlines()
               if not ln.startswith("#"))
    assert float(rec["fetch_scale"]) == pytest.approx(2.0)
    assert float(rec["write_scale"]) == pytest.approx(1.0)
    # 100 MiB x 2 read + 64 MiB written.
    assert int(rec["bytes_per_launch"]) == 264 * (1 << 20)
    assert rec["source_sha256_16"] == "0123456789abcdef"
    assert int(rec["algorithmic_bytes_per_launch"]) == 12 * 4096 ** 2


def test_counter_table_row(summary):
    prof, _ = summary
    pts = {p.kernel: p for p in report.parse_counter_table(str(prof / "ladder_square4096_counters.txt"))}
    head = [p for k, p in pts.items() if k.startswith("k4_mfma")][0]
    assert head.ms == pytest.approx(1.0)
    assert head.flop == pytest.approx(2 * 4096 ** 3, rel=1e-4)
    assert head.read_mb == pytest.approx(200 * (1 << 20) / 1e6, rel=1e-3)
    assert head.write_mb == pytest.approx(64 * (1 << 20) / 1e6, rel=1e-3)
    text = open(prof / "ladder_square4096_counters.txt").read()
    row = [ln for ln in text.splitlines() if ln.startswith("k4_mfma")][0].split()
    assert float(row[3]) == pytest.approx(2.0)        # clock, GHz
    assert row[7] == "90.0%"                          # MFMA util
    assert "python -m roofline_sgemm_f32_amd.rocprof summarize OUT" in text


def test_stall_breakdown(summary):
    prof, _ = summary
    text = open(prof / "ladder_square4096_counters.txt").read().split("Wave-cycle breakdown")[1]
    row = [ln for ln in text.splitlines() if ln.startswith("k4_mfma")][0].split()
    assert float(row[1]) == pytest.approx(2.0)        # resident waves per SIMD
    assert row[2] == "30.0%" and row[3] == "10.0%" and row[5] == "50.0%"


def test_headline_trace_averages_the_timed_dispatches(summary):
    prof, _ = summary
    text = open(prof / "k4_mfma_square4096_kernel_trace.txt").read()
    # The last 2 of the 4 grid-512 dispatches: (1.0 + 0.98) / 2 ms.
    assert "average 0.99000 ms" in text
    assert "grid    512 x   1  n=    4" in text and "grid   2048 x   1  n=    1" in text
