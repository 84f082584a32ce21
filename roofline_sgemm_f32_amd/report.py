"""Roofline report: place every ladder kernel and probe on the MI355X roofline.

amittech.dev, "7.3 Bandwidths and peak rate - exercises", exercise 6: for
each kernel record (arithmetic intensity, achieved FLOP/s), draw the compute
roof and the memory slope, and classify kernels with a two-column table of
memory-throughput and compute-throughput percentages (a kernel on the slope
shows a high memory figure and a low compute one, and the reverse on the flat
roof).  Exercise 3 of the same page defines the ridge point as peak FLOP/s
over bandwidth.

Input is a counter summary written from rocprofv3 runs (the table in
``profiles/ladder_<workload>_counters.txt``: per-kernel duration, counted
FLOP, HBM bytes read and written), or with ``--small`` a bench.py JSON line
whose small-shape section is placed at algorithmic intensity and measured
time per call.  Output: a markdown table and an SVG plot.

    python -m roofline_sgemm_f32_amd.report profiles/ladder_square4096_counters.txt \\
        --md profiles/roofline_square4096.md --svg profiles/roofline_square4096.svg
    python -m roofline_sgemm_f32_amd.report bench.out --small \\
        --md profiles/roofline_small_shapes.md --svg profiles/roofline_small_shapes.svg
"""
from __future__ import annotations

import argparse
import math
from dataclasses import dataclass

from . import metrics as m


@dataclass
class Point:
    kernel: str
    ms: float
    flop: float
    read_mb: float
    write_mb: float

    @property
    def bytes(self) -> float:
        return (self.read_mb + self.write_mb) * 1e6

    @property
    def tflops(self) -> float:
        return self.flop / (self.ms * 1e-3) / 1e12

    @property
    def gbs(self) -> float:
        return self.bytes / (self.ms * 1e-3) / 1e9

    @property
    def intensity(self) -> float:
        return self.flop / self.bytes if self.bytes else math.inf


def parse_counter_table(path: str) -> list[Point]:
    """Rows of the counter summary: kernel, ms, TFLOP/s, clock, FLOP (counted),
    MFMA ops x 512, FMA instructions, MFMA util, HBM rd MB, HBM wr MB, ..."""
    pts = []
    with open(path) as f:
        for ln in f:
            if ln.startswith("# Wave-cycle breakdown"):
                break  # the stall section that follows has columns of its own
            if ln.startswith("#") or ln.startswith("kernel") or not ln.strip():
                continue
            cols = ln.split()
            pts.append(Point(kernel=cols[0], ms=float(cols[1]), flop=float(cols[4]),
                             read_mb=float(cols[8]), write_mb=float(cols[9])))
    return pts


def classify(p: Point, peak_tflops: float, bw_gbs: float) -> dict:
    """Memory- or compute-bound by intensity against the ridge point, plus the
    two utilisation percentages of the exercise's 2 x 2 table."""
    ridge = m.ridge_flop_per_byte(peak_tflops * 1e3, bw_gbs)
    mem_pct = 100.0 * p.gbs / bw_gbs
    cmp_pct = 100.0 * p.tflops / peak_tflops
    bound = "memory" if p.intensity < ridge else "compute"
    roof = min(peak_tflops, p.intensity * bw_gbs / 1e3)
    return {"kernel": p.kernel, "ms": p.ms, "intensity": p.intensity, "tflops": p.tflops,
            "gbs": p.gbs, "mem_pct": mem_pct, "compute_pct": cmp_pct, "bound": bound,
            "roof_tflops": roof, "pct_of_roof": 100.0 * p.tflops / roof if roof else 0.0}


COUNTED = "Intensity and bandwidth use counted HBM bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated)."
ALGORITHMIC = ("Intensity and bandwidth use algorithmic bytes (A and B read once, C written once); "
               "times are per call, back-to-back, host launch cost included.")


def markdown(rows: list[dict], peak_tflops: float, bw_gbs: float, title: str, note: str = COUNTED) -> str:
    ridge = m.ridge_flop_per_byte(peak_tflops * 1e3, bw_gbs)
    out = [f"# {title}", "",
           f"Roofs: FP32 {peak_tflops:.1f} TFLOP/s, HBM {bw_gbs / 1e3:.1f} TB/s; ridge {ridge:.1f} FLOP/B.",
           note, "",
           "| kernel | ms | FLOP/B | TFLOP/s | GB/s | HBM % | FP32 % | bound | % of its roof |",
           "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        ai = "inf" if math.isinf(r["intensity"]) else f"{r['intensity']:.1f}"
        out.append(f"| {r['kernel']} | {r['ms']:.4f} | {ai} | {r['tflops']:.2f} | {r['gbs']:.0f} | "
                   f"{r['mem_pct']:.1f} | {r['compute_pct']:.1f} | {r['bound']} | {r['pct_of_roof']:.1f} |")
    return "\n".join(out) + "\n"


def svg(rows: list[dict], peak_tflops: float, bw_gbs: float, title: str) -> str:
    """Log-log roofline: x = FLOP/B (0.01 .. 1e4), y = TFLOP/s (0.01 .. 1e3)."""
    W, H, L, R, T, B = 760, 500, 70, 20, 40, 60
    x0, x1, y0, y1 = -2.0, 4.0, -2.0, 3.0

    def X(ai):
        return L + (math.log10(ai) - x0) / (x1 - x0) * (W - L - R)

    def Y(tf):
        return H - B - (math.log10(tf) - y0) / (y1 - y0) * (H - T - B)

    ridge = m.ridge_flop_per_byte(peak_tflops * 1e3, bw_gbs)
    s = [f'<svg xmlns="http://www.w3.org/2000/svg" width="{W}" height="{H}" font-family="sans-serif" font-size="11">',
         f'<rect width="{W}" height="{H}" fill="white"/>',
         f'<text x="{W / 2}" y="20" text-anchor="middle" font-size="14">{title}</text>']
    for e in range(int(x0), int(x1) + 1):
        s.append(f'<line x1="{X(10 ** e):.1f}" y1="{T}" x2="{X(10 ** e):.1f}" y2="{H - B}" stroke="#ddd"/>')
        s.append(f'<text x="{X(10 ** e):.1f}" y="{H - B + 15}" text-anchor="middle">1e{e}</text>')
    for e in range(int(y0), int(y1) + 1):
        s.append(f'<line x1="{L}" y1="{Y(10 ** e):.1f}" x2="{W - R}" y2="{Y(10 ** e):.1f}" stroke="#ddd"/>')
        s.append(f'<text x="{L - 5}" y="{Y(10 ** e) + 4:.1f}" text-anchor="end">1e{e}</text>')
    s.append(f'<text x="{W / 2}" y="{H - 20}" text-anchor="middle">arithmetic intensity (FLOP per HBM byte)</text>')
    s.append(f'<text x="18" y="{H / 2}" text-anchor="middle" transform="rotate(-90 18 {H / 2})">TFLOP/s</text>')
    lo_ai = 10 ** x0
    s.append(f'<polyline fill="none" stroke="black" stroke-width="2" points="'
             f'{X(lo_ai):.1f},{Y(lo_ai * bw_gbs / 1e3):.1f} {X(ridge):.1f},{Y(peak_tflops):.1f} '
             f'{X(10 ** x1):.1f},{Y(peak_tflops):.1f}"/>')
    s.append(f'<text x="{X(ridge) + 5:.1f}" y="{Y(peak_tflops) - 6:.1f}">FP32 {peak_tflops:.1f} TFLOP/s, '
             f'HBM {bw_gbs / 1e3:.1f} TB/s, ridge {ridge:.1f} FLOP/B</text>')
    colors = ["#1f77b4", "#ff7f0e", "#2ca02c", "#d62728", "#9467bd", "#8c564b", "#e377c2", "#7f7f7f",
              "#bcbd22", "#17becf", "#000080", "#800000", "#008000"]
    ly = T + 10
    for i, r in enumerate(rows):
        c = colors[i % len(colors)]
        ai = min(max(r["intensity"], 10 ** x0), 10 ** x1)
        tf = min(max(r["tflops"], 10 ** y0), 10 ** y1)
        if r["tflops"] <= 0:  # the copy probe does no arithmetic: place it on the x axis floor
            tf = 10 ** y0
        s.append(f'<circle cx="{X(ai):.1f}" cy="{Y(tf):.1f}" r="5" fill="{c}"/>')
        s.append(f'<circle cx="{W - R - 250}" cy="{ly + 12 * i:.1f}" r="4" fill="{c}"/>')
        s.append(f'<text x="{W - R - 240}" y="{ly + 12 * i + 4:.1f}">{r["kernel"]}</text>')
    s.append("</svg>")
    return "\n".join(s) + "\n"


def small_shape_points(bench_line: dict) -> list[Point]:
    """Points of the small-shape section of a bench.py JSON line: per shape,
    the plan the library chose and the unsplit one, at their measured time
    per call (back-to-back calls, so host launch cost included) and the
    algorithmic traffic (A and B read once, C written once)."""
    pts = []
    for r in bench_line.get("small_shapes") or []:
        if r.get("gate") is False:
            continue  # no throughput was measured for a failed result
        M, N, K = r["M"], r["N"], r["K"]
        flop = m.sgemm_flops(M, N, K)
        rd = 4.0 * (M * K + K * N) / 1e6
        wr = 4.0 * M * N / 1e6
        kind = "thin kernel, " if r.get("engine") == "thin" else ""
        pts.append(Point(f"{r['shape']} ({kind}{r['chunks']} chunk{'s' if r['chunks'] > 1 else ''})",
                         r["us_per_call"] / 1e3, flop, rd, wr))
        if r["chunks"] > 1 or kind:
            other = "matrix cores, unsplit" if kind else "unsplit"
            pts.append(Point(f"{r['shape']} {other}", r["unsplit_us_per_call"] / 1e3, flop, rd, wr))
    return pts


def main(argv=None):
    ap = argparse.ArgumentParser(description="roofline report from a counter summary")
    ap.add_argument("table", help="counter summary, or a bench.py JSON line file with --small")
    ap.add_argument("--small", action="store_true",
                    help="the table is bench.py output: report its small-shape section")
    ap.add_argument("--md")
    ap.add_argument("--svg")
    ap.add_argument("--peak-tflops", type=float, default=m.MI355X_FP32_PEAK_GFLOPS / 1e3)
    ap.add_argument("--bw-gbs", type=float, default=m.MI355X_HBM_GBS)
    ap.add_argument("--title", default="MI355X FP32 roofline, square4096 ladder")
    a = ap.parse_args(argv)
    if a.small:
        import json
        line = None
        for ln in open(a.table):
            if ln.lstrip().startswith("{") and '"small_shapes"' in ln:
                line = json.loads(ln)
        if line is None:
            raise SystemExit(f"{a.table}: no bench.py line with a small-shape section")
        pts = small_shape_points(line)
    else:
        pts = parse_counter_table(a.table)
    rows = [classify(p, a.peak_tflops, a.bw_gbs) for p in pts]
    md = markdown(rows, a.peak_tflops, a.bw_gbs, a.title, ALGORITHMIC if a.small else COUNTED)
    if a.md:
        open(a.md, "w").write(md)
    else:
        print(md)
    if a.svg:
        open(a.svg, "w").write(svg(rows, a.peak_tflops, a.bw_gbs, a.title))


if __name__ == "__main__":
    main()
