"""rocprofv3 runs over bench.py, and the text summaries under profiles/ made
from their CSV output.

amittech.dev, "7.3 Bandwidths and peak rate - exercises", exercises 4 and 6:
read each kernel's achieved rate against both roofs from profiler metrics
(here rocprofv3's counters on MI355X: HBM bytes from FETCH_SIZE and
WRITE_SIZE, matrix-core busy cycles, LDS bank conflicts, where the waves
wait), and place the kernels on the roofline.

    python -m roofline_sgemm_f32_amd.rocprof collect OUT     # on one MI355X
    python -m roofline_sgemm_f32_amd.rocprof summarize OUT   # anywhere

``collect`` runs every pass below as its own rocprofv3 process over
``python3 bench.py`` (counters in separate runs, at most 8 SQ counters each;
no pass combines counters with a trace), each under a time limit, and stops
at the first failure.  ``summarize`` writes:

  profiles/ladder_square4096_counters.txt   per-kernel counter table (ladder,
                                            probes) and the wave-cycle
                                            breakdown of the matrix-core kernels
  profiles/k4_mfma_square4096_traffic.txt   HBM bytes per launch of the
                                            headline kernel (bench.py reads it)
  profiles/k4_mfma_square4096_kernel_trace.txt  kernel-trace summary of the
                                            default bench command
  profiles/small_shapes_kernel_trace.txt    one kernel trace per small shape
  profiles/thin_kernels_..._traffic.txt     HBM bytes of the thin kernels
  profiles/roofline_square4096.{md,svg}     the roofline report (report.py)

Every summary's header names the command that made its data.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import subprocess
import sys

from . import metrics as m
from . import report

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")

# bench.py arguments of the counter passes: the ladder on square4096 (every
# variant twice after one warm-up), a short headline, the copy probe and the
# compute probes; no CPU leg, configs or small shapes.
PMC_ARGS = ["--cpu-seconds", "0", "--copy-steps", "3", "--steps", "2", "--warmup", "1", "--ladder",
            "--ladder-reps", "2", "--ladder-workloads", "square4096", "--small-reps", "0",
            "--configs-seconds", "0"]
SQ_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT",
               "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_VALU_FMA_F32", "SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_INSTS_LDS",
               "GRBM_GUI_ACTIVE"]
# Where a wave's cycles go: SQ_WAVE_CYCLES (all resident wave-cycles),
# SQ_WAIT_ANY (waiting on anything: s_waitcnt, s_barrier, dependencies),
# SQ_WAIT_INST_ANY (an instruction ready but not issued), SQ_WAIT_INST_LDS,
# and the cycles spent issuing each kind of instruction.  All in quad-cycles.
STALL_COUNTERS = ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
                  "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_SCA",
                  "GRBM_GUI_ACTIVE"]
SMALL = ["square256", "square512", "square1024", "kheavy128x128x4096", "kheavy256x256x16384",
         "kheavy1024x1024x4096", "skinny64x8192x8192", "thin1x16384x16384", "column16384x1x16384",
         "mid768x1024x1024"]
THIN = {"thin1x16384x16384": (1, 16384, 16384), "column16384x1x16384": (16384, 1, 16384)}
COPY_BYTES = 268435456 * 4  # the copy probe reads and writes 1 GiB per dispatch
N4096 = 4096


def passes() -> list[tuple[str, list[str], list[str], int]]:
    """(name, rocprofv3 options, bench.py arguments, time limit in s)."""
    out = [("fetch", ["--pmc", "FETCH_SIZE"], PMC_ARGS, 200),
           ("write", ["--pmc", "WRITE_SIZE"], PMC_ARGS, 200),
           ("sq", ["--pmc", *SQ_COUNTERS], PMC_ARGS, 200),
           ("stall", ["--pmc", *STALL_COUNTERS], PMC_ARGS, 200),
           ("trace", ["--kernel-trace", "--stats"], [], 400)]
    for s in SMALL:
        out.append((f"small_{s}", ["--kernel-trace", "--stats"], ["--small-only", s, "--small-reps", "200"], 150))
    for s in THIN:
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            out.append((f"thin_{s}_{c}", ["--pmc", c], ["--small-only", s, "--small-reps", "20"], 150))
    return out


def command(name, opts, args, out) -> list[str]:
    return ["rocprofv3", *opts, "-f", "csv", "-d", os.path.join(out, name), "-o", "run", "--",
            "python3", os.path.join(ROOT, "bench.py"), *args]


def shown(name, opts, args) -> str:
    """The command as a summary header shows it (run from the repository root)."""
    return " ".join(["rocprofv3", *opts, "-f", "csv", "-d", f"OUT/{name}", "-o", "run", "--",
                     "python3", "bench.py", *args])


def collect(out: str) -> int:
    """Run every pass (one GPU); returns 0, or the exit status of the first
    pass that failed.  rocprofv3 may end with a segmentation fault after the
    program has finished and written its results; such a pass counts as
    done when its CSV output is there."""
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    with open(os.path.join(out, "source_hash.txt"), "w") as f:
        sys.path.insert(0, ROOT)
        import bench
        f.write(bench.kernel_source_hash() + "\n")
    for name, opts, args, limit in passes():
        print(f"[rocprof] {name}", flush=True)
        with open(os.path.join(out, f"{name}.log"), "w") as log:
            r = subprocess.run(["timeout", "-s", "KILL", str(limit), *command(name, opts, args, out)],
                               stdout=log, stderr=subprocess.STDOUT, cwd="/tmp", env=env)
        done = any(f.endswith(".csv") for _, _, fs in os.walk(os.path.join(out, name)) for f in fs)
        if r.returncode != 0 and not (r.returncode == 139 and done):
            print(f"[rocprof] {name}: exit status {r.returncode}", flush=True)
            return r.returncode or 1
    print("[rocprof] done", flush=True)
    return 0


# ---------------------------------------------------------------- summaries

def short(name: str) -> str | None:
    """Kernel name without namespaces and argument list (None: not ours)."""
    if "sgemm::" not in name:
        return None
    return name.split("(")[0].replace("void ", "").replace("sgemm::", "").replace("k4::Cfg", "Cfg")


def read_counters(*dirs) -> dict:
    """Per kernel: counter -> list of per-dispatch values, plus the dispatch
    durations (ms) and the launch resources."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                k = short(r["Kernel_Name"])
                if not k:
                    continue
                a = agg[k]
                a[r["Counter_Name"]].append(float(r["Counter_Value"]))
                a["dur_ms"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
                a["vgpr"] = [int(r["VGPR_Count"])]
                a["agpr"] = [int(r["Accum_VGPR_Count"])]
                a["lds"] = [int(r["LDS_Block_Size"])]
    return agg


def means(agg: dict) -> dict:
    return {k: {c: sum(v) / len(v) for c, v in d.items() if v} for k, d in agg.items()}


def copy_scales(avg: dict) -> tuple[float, float]:
    """FETCH_SIZE and WRITE_SIZE (KiB) scale factors from the copy probe,
    which reads and writes COPY_BYTES per dispatch."""
    c = avg["copy_vec4"]
    return COPY_BYTES / (c["FETCH_SIZE"] * 1024), COPY_BYTES / (c["WRITE_SIZE"] * 1024)


def counter_row(k: str, a: dict, fscale: float, wscale: float) -> dict:
    dur = a["dur_ms"]
    xcd_clk = a["GRBM_GUI_ACTIVE"] / 8  # GRBM_GUI_ACTIVE sums the 8 XCDs' busy clocks
    f = a["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512 + a["SQ_INSTS_VALU_FMA_F32"] * 128
    rd = a["FETCH_SIZE"] * 1024 * fscale / 1e6
    wr = a["WRITE_SIZE"] * 1024 * wscale / 1e6
    return {
        "kernel": k, "ms": dur, "tflops": f / (dur * 1e-3) / 1e12, "clk": xcd_clk / (dur * 1e-3) / 1e9,
        "flop": f, "mops512": a["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512, "fma": a["SQ_INSTS_VALU_FMA_F32"],
        "util": a["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_clk * 1024) * 100, "rd": rd, "wr": wr,
        "ai": f / ((rd + wr) * 1e6) if f else 0.0, "lds": a["SQ_INSTS_LDS"],
        "confl": a["SQ_LDS_BANK_CONFLICT"] / a["SQ_LDS_IDX_ACTIVE"] * 100 if a["SQ_LDS_IDX_ACTIVE"] else 0.0,
        "vgpr": int(a["vgpr"]), "agpr": int(a["agpr"]), "lds_b": int(a["lds"]),
    }


LADDER_ORDER = ["k0_naive", "k1_coalesced", "k2_lds<16, 0>", "k2_lds<16, 1>", "k2_lds<32, 0>",
                "k2_lds<32, 1>", "k3_regtile<true>"]


def counters_table(out: str) -> tuple[list[str], dict, float, float]:
    agg = read_counters(*(os.path.join(out, p) for p in ("fetch", "write", "sq")))
    avg = means(agg)
    fscale, wscale = copy_scales(avg)
    L = ["# Counters per dispatch, square4096 (M=N=K=4096): every ladder kernel, the compute probes and the copy probe",
         "# Commands (from the repository root on one MI355X; one rocprofv3 run per pass):",
         f"#   {shown('fetch', ['--pmc', 'FETCH_SIZE'], PMC_ARGS)}",
         f"#   {shown('write', ['--pmc', 'WRITE_SIZE'], PMC_ARGS)}",
         f"#   {shown('sq', ['--pmc', *SQ_COUNTERS], PMC_ARGS)}",
         f"#   {shown('stall', ['--pmc', *STALL_COUNTERS], PMC_ARGS)}",
         "#   python -m roofline_sgemm_f32_amd.rocprof summarize OUT",
         "# Values are means over each kernel's dispatches in those runs (counter runs serialise dispatches;",
         "# durations under the profiler run slower than the bench's).",
         f"# HBM calibration with the copy probe (reads 1 GiB, writes 1 GiB per dispatch): FETCH_SIZE scale "
         f"{fscale:.4f}, WRITE_SIZE scale {wscale:.4f}",
         "# MFMA util = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs * 1024 SIMDs); clock = GRBM_GUI_ACTIVE / 8 / duration",
         "# (SQ_VALU_MFMA_BUSY_CYCLES reads 8 x SQ_INSTS_VALU_MFMA_MOPS_F32 on the matrix kernels, 64 busy cycles per",
         "#  v_mfma_f32_32x32x2_f32: MFMA util is the matrix work over the SIMD-cycles elapsed at the measured clock)",
         "# LDS conflict rate = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
         f"{'kernel':36s} {'ms':>8s} {'TFLOP/s':>8s} {'clk GHz':>7s} {'FLOP':>11s} {'MOPS*512':>11s} "
         f"{'FMA instr':>11s} {'MFMA util':>9s} {'HBM rd MB':>9s} {'HBM wr MB':>9s} {'AI FLOP/B':>9s} "
         f"{'LDS instr':>11s} {'LDS confl':>9s} {'VGPR':>5s} {'AGPR':>5s} {'LDS B':>6s}"]
    keys = [k for k in LADDER_ORDER if k in avg]
    keys += sorted(k for k in avg if k not in LADDER_ORDER and k != "copy_vec4") + ["copy_vec4"]
    for k in keys:
        r = counter_row(k, avg[k], fscale, wscale)
        L.append(f"{k.replace(', ', ','):36s} {r['ms']:8.3f} {r['tflops']:8.2f} {r['clk']:7.3f} {r['flop']:11.4e} "
                 f"{r['mops512']:11.4e} {r['fma']:11.4e} {r['util']:8.1f}% {r['rd']:9.1f} {r['wr']:9.1f} "
                 f"{r['ai']:9.1f} {r['lds']:11.4e} {r['confl']:8.2f}% {r['vgpr']:5d} {r['agpr']:5d} {r['lds_b']:6d}")
    L.append(f"# algorithmic: {2 * N4096 ** 3} FLOP and {12 * N4096 ** 2 / 1e6:.1f} MB (A, B read once, C written once) "
             "per SGEMM dispatch;")
    L.append("# FLOP = SQ_INSTS_VALU_MFMA_MOPS_F32*512 + SQ_INSTS_VALU_FMA_F32*64 lanes*2 (counted, not assumed);")
    L.append("# probe_valu / probe_mfma are the compute-roof probes (FMA chains / back-to-back FP32 MFMA), "
             "copy_vec4 the HBM probe.")
    stall_dir = os.path.join(out, "stall")
    if os.path.exists(os.path.join(stall_dir, "run_counter_collection.csv")):
        L += stall_table(means(read_counters(stall_dir)))
    return L, avg, fscale, wscale


def stall_table(avg: dict) -> list[str]:
    """Where the resident wave-cycles of each matrix-core kernel (and the
    probes) go, as fractions of SQ_WAVE_CYCLES."""
    L = ["#",
         "# Wave-cycle breakdown (stall pass): fractions of SQ_WAVE_CYCLES, the cycles waves are resident.",
         "#   wait any  = SQ_WAIT_ANY (waiting on s_waitcnt, s_barrier or a dependency)",
         "#   wait issue = SQ_WAIT_INST_ANY (an instruction ready, not issued: the unit busy with other waves)",
         "#   wait LDS issue = SQ_WAIT_INST_LDS; VALU / LDS / VMEM / scalar = SQ_ACTIVE_INST_* (issuing those)",
         "#   (MFMA instructions issue as VALU; the counters sample every wave of every SIMD, so on a SIMD with",
         "#    two waves, one waiting while the other issues is normal overlap, not lost time)",
         f"{'kernel':36s} {'waves/SIMD':>10s} {'wait any':>9s} {'wait issue':>10s} {'wait LDS iss':>12s} "
         f"{'VALU':>7s} {'LDS':>7s} {'VMEM':>7s} {'scalar':>7s}"]
    for k in sorted(avg):
        a = avg[k]
        if not (k.startswith("k4_mfma") or k.startswith("probe")) or not a.get("SQ_WAVE_CYCLES"):
            continue
        wc = a["SQ_WAVE_CYCLES"]
        # Wave-cycles over SIMD-cycles: the average number of resident waves per SIMD.
        simd_q = a["GRBM_GUI_ACTIVE"] / 8 * 1024 / 4
        L.append(f"{k.replace(', ', ','):36s} {wc / simd_q:10.2f} {100 * a['SQ_WAIT_ANY'] / wc:8.1f}% "
                 f"{100 * a['SQ_WAIT_INST_ANY'] / wc:9.1f}% {100 * a['SQ_WAIT_INST_LDS'] / wc:11.1f}% "
                 f"{100 * a['SQ_ACTIVE_INST_VALU'] / wc:6.1f}% {100 * a['SQ_ACTIVE_INST_LDS'] / wc:6.1f}% "
                 f"{100 * a['SQ_ACTIVE_INST_VMEM'] / wc:6.1f}% {100 * a['SQ_ACTIVE_INST_SCA'] / wc:6.1f}%")
    return L


def headline_instance(avg: dict) -> str:
    """The 128 x 256 matrix-core kernel on A and B as stored (16-byte loads):
    the one AUTO runs for square4096."""
    cands = [k for k in avg if k.startswith("k4_mfma<Cfg<2, 2, 2, 4, 16, true, true, false")]
    if not cands:
        raise SystemExit("no 128 x 256 matrix-core kernel in the counter data")
    return max(cands, key=lambda k: len(avg[k]))


def traffic_file(out: str, agg_avg: dict, fscale: float, wscale: float) -> list[str]:
    k = headline_instance(agg_avg)
    a = agg_avg[k]
    c = agg_avg["copy_vec4"]
    tb = a["FETCH_SIZE"] * 1024 * fscale + a["WRITE_SIZE"] * 1024 * wscale
    alg = 12 * N4096 ** 2
    src = open(os.path.join(out, "source_hash.txt")).read().strip()
    return [
        "# HBM traffic of the matrix-core kernel on square4096, from two rocprofv3 counter runs",
        f"#   {shown('fetch', ['--pmc', 'FETCH_SIZE'], PMC_ARGS)}",
        f"#   {shown('write', ['--pmc', 'WRITE_SIZE'], PMC_ARGS)}",
        "#   python -m roofline_sgemm_f32_amd.rocprof summarize OUT",
        "# scaled by what the same counters read for the copy probe (1 GiB read + 1 GiB written per dispatch).",
        "# bench.py reports bytes_per_launch as roofline.traffic only while source_sha256_16 matches the kernel",
        "# code and its plan (k4_mfma.hip, k4_layout.h and k4_plan.hip, comments excluded: bench.kernel_source_hash).",
        "kernel: k4_mfma",
        "workload: square4096",
        f"source_sha256_16: {src}",
        f"kernel_instance: {k}",
        f"fetch_kib_per_dispatch: {a['FETCH_SIZE']:.1f}",
        f"write_kib_per_dispatch: {a['WRITE_SIZE']:.1f}",
        f"copy_fetch_kib_per_dispatch: {c['FETCH_SIZE']:.1f}",
        f"copy_write_kib_per_dispatch: {c['WRITE_SIZE']:.1f}",
        f"copy_bytes_read_per_dispatch: {COPY_BYTES}",
        f"copy_bytes_written_per_dispatch: {COPY_BYTES}",
        f"fetch_scale: {fscale:.5f}",
        f"write_scale: {wscale:.5f}",
        f"bytes_per_launch: {int(tb)}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {tb / alg:.3f}",
    ]


def thin_traffic(out: str, fscale: float, wscale: float) -> list[str]:
    L = ["# HBM traffic of the thin-product kernels (and of the matrix-core kernel on the same shapes, which the",
         "# bench times as the 'unsplit' call), from rocprofv3 counter runs, one per shape and counter:"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        L.append(f"#   {shown(f'thin_<shape>_{c}', ['--pmc', c], ['--small-only', '<shape>', '--small-reps', '20'])}")
    L += ["#   python -m roofline_sgemm_f32_amd.rocprof summarize OUT",
          f"# scaled by the copy-probe calibration of the square4096 counter runs (FETCH_SIZE x {fscale:.4f}, "
          f"WRITE_SIZE x {wscale:.4f}).",
          "# Algorithmic bytes of a product: 4 (MK + KN + MN); a split thin call also writes S partial slabs of M x N",
          "# floats, which splitk_reduce reads back before writing C.  Means over each kernel's dispatches.",
          f"{'shape':22s} {'kernel':62s} {'n':>5s} {'read MB':>9s} {'written MB':>10s} {'alg MB':>9s} {'read/alg':>8s}"]
    for sh, (M, N, K) in THIN.items():
        dirs = [os.path.join(out, f"thin_{sh}_{c}") for c in ("FETCH_SIZE", "WRITE_SIZE")]
        if not all(os.path.exists(os.path.join(d, "run_counter_collection.csv")) for d in dirs):
            L.append(f"{sh:22s} no counter data")
            continue
        agg = read_counters(*dirs)
        alg = 4 * (M * K + K * N + M * N)
        for k, d in agg.items():
            rd = sum(d["FETCH_SIZE"]) / len(d["FETCH_SIZE"]) * 1024 * fscale / 1e6
            wr = sum(d["WRITE_SIZE"]) / len(d["WRITE_SIZE"]) * 1024 * wscale / 1e6
            L.append(f"{sh:22s} {k.replace(', ', ','):62s} {len(d['FETCH_SIZE']):5d} {rd:9.2f} {wr:10.2f} "
                     f"{alg / 1e6:9.2f} {rd / (alg / 1e6):8.3f}")
    return L


def bench_line(path: str, key: str = "metric") -> dict | None:
    line = None
    with open(path) as f:
        for ln in f:
            if ln.startswith("{") and f'"{key}"' in ln:
                line = json.loads(ln)
    return line


def trace_rows(d: str) -> list[dict]:
    with open(os.path.join(d, "run_kernel_trace.csv")) as f:
        return list(csv.DictReader(f))


def by_kernel_grid(rows: list[dict]) -> "collections.OrderedDict":
    """(kernel, workgroups x, grid y) -> durations in us, in first-launch order."""
    g = collections.OrderedDict()
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        k = short(r["Kernel_Name"])
        if not k:
            continue
        wg = int(r["Workgroup_Size_X"])
        key = (k, int(r["Grid_Size_X"]) // wg, int(r["Grid_Size_Y"]))
        g.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return g


def small_traces(out: str) -> list[str]:
    L = ["# Small-shape path: rocprofv3 kernel traces, one run per shape (200 timed calls with the K split the",
         "# library chooses, then 200 unsplit, each after about 50 ms of warm-up calls).  Commands, from the",
         "# repository root on one MI355X:",
         f"#   {shown('small_<shape>', ['--kernel-trace', '--stats'], ['--small-only', '<shape>', '--small-reps', '200'])}",
         "#   python -m roofline_sgemm_f32_amd.rocprof summarize OUT",
         "# Per shape: the bench's own JSON (us per call, split and unsplit), then each sgemm kernel dispatched:",
         "# grid (workgroups x, y), dispatches, mean and min duration in us (device time, from the trace)."]
    for sh in SMALL:
        d = os.path.join(out, f"small_{sh}")
        if not os.path.exists(os.path.join(d, "run_kernel_trace.csv")):
            L.append(f"## {sh}: no trace")
            continue
        js = bench_line(os.path.join(out, f"small_{sh}.log"), "small_shapes")["small_shapes"][0]
        L.append(f"## {sh}: M={js['M']} N={js['N']} K={js['K']} chunks={js['chunks']} kchunk={js['kchunk']}: "
                 f"{js['us_per_call']} us/call ({js['gflops']} GFLOP/s); unsplit {js['unsplit_us_per_call']} us/call "
                 f"({js['unsplit_gflops']} GFLOP/s); x{js['speedup_vs_unsplit']}")
        for (k, gx, gy), v in by_kernel_grid(trace_rows(d)).items():
            L.append(f"   {k.replace(', ', ','):70s} grid {gx:6d} x {gy:3d}  n={len(v):4d}  "
                     f"mean {sum(v) / len(v):8.2f} us  min {min(v):8.2f} us")
    return L


def headline_trace(out: str) -> list[str]:
    d = os.path.join(out, "trace")
    line = bench_line(os.path.join(out, "trace.log"))
    rows = trace_rows(d)
    groups = by_kernel_grid(rows)
    steps = line["steps"]
    head = [key for key in groups if key[0].startswith("k4_mfma<Cfg<2, 2, 2, 4, 16, true, true, false")
            and key[1] == (N4096 // 128) * (N4096 // 256)]
    T = ["# rocprofv3 --kernel-trace --stats summary of the default benchmark (copy and compute probes, the",
         "# five configs through AUTO, then square4096: 100 warm-up + 100 timed products, small shapes, CPU leg).",
         "# Command, from the repository root on one MI355X:",
         f"#   {shown('trace', ['--kernel-trace', '--stats'], [])}",
         "#   python -m roofline_sgemm_f32_amd.rocprof summarize OUT",
         f"# The bench line of that same run: value {line['value']} GFLOP/s, ms_per_step {line['ms_per_step']} ms "
         f"({line['roofline']['achieved']} TFLOP/s), hbm_copy {line['hbm_copy']['ms']} ms "
         f"({line['hbm_copy']['gbs']} GB/s)."]
    if head:
        v = groups[head[0]]
        timed = v[-steps:]
        T.append(f"# The headline kernel runs square4096 on a grid of {head[0][1]} workgroups (the configs section's")
        T.append(f"# square4096 calls included): {len(v)} dispatches; the last {steps}, the timed ones, average "
                 f"{sum(timed) / len(timed) / 1e3:.5f} ms")
        T.append(f"# (bench: {line['ms_per_step']} ms per step, from events around the timed launches).  The same kernel")
        T.append("# also runs square8192 in the configs section (grid 2048), so the stats row below mixes both sizes.")
    T.append("#")
    T.append("# Per kernel and grid (workgroups x, y): dispatches, mean and min duration in us:")
    for (k, gx, gy), v in groups.items():
        T.append(f"#   {k.replace(', ', ','):74s} grid {gx:6d} x {gy:3d}  n={len(v):5d}  "
                 f"mean {sum(v) / len(v):10.2f}  min {min(v):10.2f}")
    T.append("# rocprofv3 --stats table (names of torch's own kernels shortened):")
    T.append("# Name | Calls | TotalDurationNs | AverageNs | Percentage | MinNs | MaxNs | StdDev")
    with open(os.path.join(d, "run_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            n = r["Name"]
            if "sgemm::" not in n:
                n = re.sub(r"<.*", "", n)[:70]
            T.append(f"{n} | {r['Calls']} | {r['TotalDurationNs']} | {float(r['AverageNs']):.1f} | "
                     f"{r['Percentage']} | {r['MinNs']} | {r['MaxNs']} | {float(r['StdDev']):.1f}")
    return T


def summarize(out: str, profiles: str = PROFILES) -> list[str]:
    """Write every summary whose data is under ``out``; returns the paths."""
    written = []

    def put(name, lines):
        p = os.path.join(profiles, name)
        with open(p, "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append(p)

    if os.path.exists(os.path.join(out, "sq", "run_counter_collection.csv")):
        L, avg, fscale, wscale = counters_table(out)
        table = os.path.join(profiles, "ladder_square4096_counters.txt")
        put("ladder_square4096_counters.txt", L)
        put("k4_mfma_square4096_traffic.txt", traffic_file(out, avg, fscale, wscale))
        put("thin_kernels_thin1x16384x16384_column16384x1x16384_traffic.txt", thin_traffic(out, fscale, wscale))
        pts = report.parse_counter_table(table)
        rows = [report.classify(p, m.MI355X_FP32_PEAK_GFLOPS / 1e3, m.MI355X_HBM_GBS) for p in pts]
        title = "MI355X FP32 roofline, square4096 ladder"
        md = report.markdown(rows, m.MI355X_FP32_PEAK_GFLOPS / 1e3, m.MI355X_HBM_GBS, title).split("\n")
        md[1:1] = ["", "From `profiles/ladder_square4096_counters.txt` by "
                   "`python -m roofline_sgemm_f32_amd.rocprof summarize OUT` (the same as "
                   "`python -m roofline_sgemm_f32_amd.report profiles/ladder_square4096_counters.txt`)."]
        put("roofline_square4096.md", md)
        put("roofline_square4096.svg", [report.svg(rows, m.MI355X_FP32_PEAK_GFLOPS / 1e3, m.MI355X_HBM_GBS,
                                                   title).rstrip("\n")])
    if os.path.exists(os.path.join(out, "trace", "run_kernel_trace.csv")):
        put("k4_mfma_square4096_kernel_trace.txt", headline_trace(out))
        line = bench_line(os.path.join(out, "trace.log"))
        if line and line.get("small_shapes"):
            rows = [report.classify(p, m.MI355X_FP32_PEAK_GFLOPS / 1e3, m.MI355X_HBM_GBS)
                    for p in report.small_shape_points(line)]
            title = "MI355X FP32 roofline, small-shape path (time per call)"
            md = report.markdown(rows, m.MI355X_FP32_PEAK_GFLOPS / 1e3, m.MI355X_HBM_GBS, title,
                                 report.ALGORITHMIC).split("\n")
            md[1:1] = ["", "The small-shape section of the bench line of the trace run "
                       f"(`{shown('trace', ['--kernel-trace', '--stats'], [])}`), placed by "
                       "`python -m roofline_sgemm_f32_amd.rocprof summarize OUT`."]
            put("roofline_small_shapes.md", md)
            put("roofline_small_shapes.svg", [report.svg(rows, m.MI355X_FP32_PEAK_GFLOPS / 1e3, m.MI355X_HBM_GBS,
                                                         title).rstrip("\n")])
    if any(os.path.exists(os.path.join(out, f"small_{s}")) for s in SMALL):
        put("small_shapes_kernel_trace.txt", small_traces(out))
    return written


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("collect", help="run every rocprofv3 pass over bench.py (one GPU)")
    c.add_argument("out")
    s = sub.add_parser("summarize", help="write the profiles/ summaries from collected CSV output")
    s.add_argument("out")
    s.add_argument("--profiles", default=PROFILES)
    sub.add_parser("commands", help="print the rocprofv3 commands collect runs")
    a = ap.parse_args(argv)
    if a.cmd == "collect":
        sys.exit(collect(os.path.abspath(a.out)))
    if a.cmd == "summarize":
        for p in summarize(os.path.abspath(a.out), a.profiles):
            print(p)
    else:
        for name, opts, args, _ in passes():
            print(shown(name, opts, args))


if __name__ == "__main__":
    main()
