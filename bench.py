#!/usr/bin/env python3
"""Benchmark: SGEMM GFLOP/s at N = 4096 (FP32) and its fraction of the
MI355X FP32 peak, on one GPU.

One step is one C = A * B of the square 4096 workload (A, B uniform [-1, 1)
from seed 3) through the C ABI, inputs resident in HBM.  Timing follows
amittech.dev, "3.5 Project: tiled matrix multiplication", section "starter
scaffolding" (the event timer): untimed warm-up launches, then back-to-back
timed launches bracketed by events on the launch stream, mean per launch.

Prints ONE JSON line on stdout; the ladder table and the copy-probe sweep
(--ladder, --copy-sweep) go to stderr and to --out as JSON lines.

Legs, in the order they run:
  * hbm_copy: the copy probe (256 Mi floats, 2 GiB moved) against 8 TB/s,
    and compute_probe: register-only FMA chains and back-to-back FP32 matrix
    instructions, the two roofs the kernels are measured against.
  * configs: each of the five workloads through AUTO (time per call,
    GFLOP/s, fraction of the FP32 peak).
  * GPU product (the headline): value = 2 M N K / mean step time.
  * roofline: the matrix-core kernel's achieved TFLOP/s against 157.3, from
    the events around the timed launches on the launch stream; ``traffic``
    is read from a committed counter summary when it was taken on the
    current kernel source.
  * small_shapes: the small-shape path, split as chosen and unsplit.
  * cpu_baseline: the CPU oracle timed on this host on a bounded sample of
    the headline product; the oracle's full results then gate every element
    of the headline product and of each config's result.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SGEMM GFLOP/s at N=4096 FP32 and % of MI355X FP32 peak"
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(files=("k4_mfma.hip", "k4_layout.h", "k4_plan.hip")) -> str:
    """Hash of the matrix-core kernel's code and of the plan that picks its
    configuration (comments and blank lines dropped, so that editing a
    comment keeps recorded counters valid)."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "roofline_sgemm_f32_amd", "csrc", f)) as fh:
            for ln in fh:
                code = re.sub(r"//.*", "", ln).strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary (key: value
    lines), if it was taken on the current kernel source; else None."""
    p = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(p):
        return None
    rec = {}
    with open(p) as f:
        for ln in f:
            if ln.startswith("#") or ":" not in ln:
                continue
            k, v = ln.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_sha256_16") != kernel_source_hash():
        return None
    return int(rec["bytes_per_launch"]) if "bytes_per_launch" in rec else None


def time_launches(fn, steps: int, warmup: int, per_launch: bool = True):
    """Warm up, then time ``steps`` back-to-back launches on the current
    stream; returns (mean ms per step, mean ms per launch from per-launch
    event pairs, or None without them)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    n = steps if per_launch else 0
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    if per_launch:
        for i in range(steps):
            starts[i].record()
            fn()
            ends[i].record()
    else:
        for _ in range(steps):
            fn()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1) / steps
    per = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / steps if per_launch else None
    return total, per


def launch_times(fn, steps: int, warmup: int):
    """Per-launch durations (ms) of ``steps`` back-to-back launches, each
    between its own pair of events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def run_gemm_factory(variant, A, B, C):
    import roofline_sgemm_f32_amd as rs
    import torch
    M, K = A.shape
    N = B.shape[1]
    lda, ldb, ldc = A.stride(0), B.stride(0), C.stride(0)
    a, b, c = A.data_ptr(), B.data_ptr(), C.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    vid = rs.VARIANTS[variant]
    lib = rs.load()

    def fn():
        st = lib.sgemm_f32_variant(vid, M, N, K, a, lda, b, ldb, c, ldc, stream)
        if st != 0:
            raise rs.SgemmError(st, variant)
    return fn


def device_operands(w):
    import torch
    from roofline_sgemm_f32_amd.inputs import workload_operands
    A_h, B_h = workload_operands(w)
    A = torch.as_strided(torch.empty(w.M * w.lda, device="cuda"), (w.M, w.K), (w.lda, 1))
    B = torch.as_strided(torch.empty(w.K * w.ldb, device="cuda"), (w.K, w.N), (w.ldb, 1))
    A.copy_(A_h)
    B.copy_(B_h)
    C = torch.as_strided(torch.full((w.M * w.ldc,), float("nan"), device="cuda"), (w.M, w.N), (w.ldc, 1))
    return A_h, B_h, A, B, C


def cpu_baseline_leg(w, A_h, B_h, C, budget_s: float, threads: int | None = None):
    """Time the CPU oracle on a bounded sample of rows of the same product,
    and check the GPU's rows against it (C: the GPU result, a host array or
    a device tensor)."""
    import numpy as np
    import oracle
    from oracle import check
    from roofline_sgemm_f32_amd import metrics as m
    from roofline_sgemm_f32_amd.inputs import as_numpy
    An, Bn = as_numpy(A_h), as_numpy(B_h)
    threads = threads or oracle.default_threads()
    oracle.load()
    rng = np.random.default_rng(0)
    # Calibrate on one row per thread, then size the sample to the budget:
    # a random subset of rows, or every row repeated when the whole product
    # takes less than the budget.
    cal = np.sort(rng.choice(w.M, size=min(threads, w.M), replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.sgemm_rows_f64(An, Bn, cal, bound=False, threads=threads)
    t_cal = max(time.perf_counter() - t0, 1e-6)
    n = int(budget_s / t_cal * len(cal))
    if n >= w.M:
        rows = np.arange(w.M, dtype=np.int64)
        reps = max(1, int(budget_s / (t_cal * w.M / len(cal))))
    else:
        n = max(len(cal), (n // threads) * threads)
        rows = np.sort(rng.choice(w.M, size=n, replace=False)).astype(np.int64)
        reps = 1
    t0 = time.perf_counter()
    for _ in range(reps):
        ref, _ = oracle.sgemm_rows_f64(An, Bn, rows, bound=False, threads=threads)
    dt = time.perf_counter() - t0
    flops = m.sgemm_flops(len(rows), w.N, w.K) * reps
    # Gate: the GPU rows against the oracle rows, with the bound matrix
    # (untimed).
    _, S = oracle.sgemm_rows_f64(An, Bn, rows, bound=True, threads=threads)
    Cr = C[rows] if isinstance(C, np.ndarray) else C[rows.tolist()].cpu().numpy()
    rep = check.check(Cr, ref, S, w.K)
    base = {
        "value": round(m.gflops(flops, dt * 1e3), 3),
        "unit": "GFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{reps} x {len(rows)} of {w.M} rows of the {w.name} product "
                  f"({reps}*2*{len(rows)}*{w.N}*{w.K} FLOP, fp64 accumulate), {dt:.2f} s "
                  f"on {threads} host threads",
    }
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
        if model:
            base["cpu"] = model
    except OSError:
        pass
    # The oracle runs `cores` POSIX threads whatever OpenMP is set to; the
    # environment's OpenMP setting is recorded for context.
    base["omp_num_threads_env"] = os.environ.get("OMP_NUM_THREADS")
    gate = {"rows_checked": len(rows), "ok": rep["ok"], "max_bound_util": rep["max_bound_util"],
            "max_rel_err_page": rep["max_rel_err_page"], "n_violations": rep["n_violations"]}
    return base, gate


def oracle_gate(w, A_h, B_h, C_host):
    """Every element of a GPU result against the CPU oracle's bound (part
    of the CPU leg: the oracle runs on this host's threads, untimed here)."""
    import oracle
    from oracle import check
    from roofline_sgemm_f32_amd.inputs import as_numpy
    ref, S = oracle.sgemm_f64(as_numpy(A_h), as_numpy(B_h))
    rep = check.check(C_host, ref, S, w.K)
    return {"elements_checked": rep["n"], "ok": rep["ok"], "max_bound_util": rep["max_bound_util"],
            "max_rel_err_page": rep["max_rel_err_page"], "n_violations": rep["n_violations"]}


def configs_leg(budget_s: float):
    """The five workloads through AUTO: back-to-back calls for about
    ``budget_s`` (at least 20, after as many warm-ups), mean per call.
    Returns the records and, per workload, the host operands and the
    (device) result of the timed launches, for the CPU leg's gate."""
    import torch
    import roofline_sgemm_f32_amd as rs
    from roofline_sgemm_f32_amd import metrics as m
    from roofline_sgemm_f32_amd.inputs import WORKLOADS
    rows, keep = [], {}
    for name, w in WORKLOADS.items():
        A_h, B_h, A, B, C = device_operands(w)
        fn = run_gemm_factory("auto", A, B, C)
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        steps = int(max(20, min(2000, budget_s / max(time.perf_counter() - t0, 1e-6))))
        ms, _ = time_launches(fn, steps, steps, per_launch=False)
        plan = rs.plan_config(w.M, w.N, w.K, lda=w.lda, ldb=w.ldb, A_ptr=A.data_ptr(),
                              B_ptr=B.data_ptr())
        g = m.gflops(m.sgemm_flops(w.M, w.N, w.K), ms)
        rec = {"workload": name, "M": w.M, "N": w.N, "K": w.K, "dist": w.dist, "seed": w.seed,
               "variant": "auto", "engine": plan["engine"], "tile": list(plan["tile"]),
               "k_groups": plan["k_groups"], "packed": plan["packed"], "chunks": plan["splits"],
               "ms": round(ms, 5), "gflops": round(g, 1),
               "pct_peak": round(m.pct_of_peak(g, m.MI355X_FP32_PEAK_GFLOPS), 2), "steps": steps}
        rows.append(rec)
        keep[name] = (w, A_h, B_h, C)
        log(f"  config {name:22s} {ms:9.4f} ms {g:10.1f} GFLOP/s {rec['pct_peak']:6.2f}% "
            f"tile {plan['tile']} x{plan['k_groups']} packed={plan['packed']} chunks={plan['splits']}")
        del A, B
    return rows, keep


def copy_probe(steps: int, block=None, grid=None):
    import torch
    import roofline_sgemm_f32_amd as rs
    from roofline_sgemm_f32_amd import metrics as m
    from roofline_sgemm_f32_amd.inputs import COPY_ELEMENTS
    n = COPY_ELEMENTS
    from roofline_sgemm_f32_amd.inputs import COPY_SEED
    g = torch.Generator(device="cuda")
    g.manual_seed(COPY_SEED)
    src = torch.rand(n, device="cuda", generator=g)
    dst = torch.empty_like(src)
    if block is None:
        fn = lambda: rs.copy_f32(dst, src)  # noqa: E731
    else:
        fn = lambda: rs.copy_f32_launch(dst, src, block, grid)  # noqa: E731
    total, per = time_launches(fn, steps, 1)
    ok = bool(torch.equal(dst, src))
    gbs = m.gbs(m.copy_bytes(n), per)
    return {"n": n, "bytes": m.copy_bytes(n), "ms": round(per, 5), "gbs": round(gbs, 1),
            "frac": round(gbs / m.MI355X_HBM_GBS, 4), "exact": ok,
            "block": block or 64, "grid": grid}


def compute_probe(valu_iters=4096, mfma_iters=4096, steps=30, warmup=10):
    """Sustained FP32 rate of register-only multiply-add chains (vector ALU)
    and of back-to-back FP32 matrix instructions, for the compute roof: mean
    over the timed launches, and the fastest launch (the chip's clock, and so
    these rates, drop when it runs into its power limit)."""
    import statistics
    import torch
    import roofline_sgemm_f32_amd as rs
    from roofline_sgemm_f32_amd.inputs import probe_operands
    blocks, block = 256 * 8, 256  # 32 waves per CU
    out_v = torch.empty((blocks * block, rs.VALU_CHAINS), device="cuda")
    tv = launch_times(lambda: rs.probe_valu(blocks, block, valu_iters, 0.999, 0.001, out_v), steps, warmup)
    fv = blocks * block * valu_iters * rs.VALU_CHAINS * 2
    a, b = probe_operands(7)
    a, b = a.cuda(), b.cuda()
    # 8 waves per CU (2 per SIMD): with 4 per SIMD the back-to-back MFMA
    # chains of the probe run at 88-104 TFLOP/s, with 1 or 2 per SIMD at
    # 150-154 (measured on MI355X), so the roof is taken at 2.
    mblocks = 256 * 2
    out_m = torch.empty((mblocks * 4, 4, 32, 32), device="cuda")
    tm = launch_times(lambda: rs.probe_mfma(a, b, mblocks, mfma_iters, out_m), steps, warmup)
    fm = mblocks * 16 * mfma_iters * 4096
    tf = lambda f, ms: round(f / (ms * 1e-3) / 1e12, 2)
    return {"valu_fma_tflops": tf(fv, statistics.mean(tv)), "valu_fma_tflops_best": tf(fv, min(tv)),
            "mfma_f32_tflops": tf(fm, statistics.mean(tm)), "mfma_f32_tflops_best": tf(fm, min(tm)),
            "valu_ms": round(statistics.mean(tv), 4), "mfma_ms": round(statistics.mean(tm), 4),
            "launches": steps}


# Products up to this many multiply-adds are gated on every row of C, as far
# as the rows of A checked hold at most ROW_GATE_A_ELEMS elements (evenly
# spaced rows beyond that); larger products (the ladder rows at square4096)
# on six rows.
ROW_GATE_FULL_MACS = 2 ** 33
ROW_GATE_A_ELEMS = 2 ** 24


def row_gate(A_h, B_h):
    """Correctness gate for a timed GPU product outside the headline leg (a
    ladder row, a small-shape plan): the rows of C (all of them for products
    of up to ROW_GATE_FULL_MACS multiply-adds and ROW_GATE_A_ELEMS elements
    of A, evenly spaced ones up to that many elements for a larger A, else a
    few: first, last and some between), against numpy's float64 product of
    the same host operands, with the binary32 dot-product bound
    4 K 2^-24 sum|a b| per element.  Its throughput is printed only when the
    result passes."""
    import numpy as np
    from roofline_sgemm_f32_amd.inputs import as_numpy
    M, K = A_h.shape
    N = B_h.shape[1]
    sentinel = {0, 1 % M, M // 3, M // 2, max(M - 2, 0), M - 1}
    if M * N * K <= ROW_GATE_FULL_MACS:
        n = max(1, min(M, ROW_GATE_A_ELEMS // max(K, 1)))
        rows = sorted(sentinel | {i * M // n for i in range(n)})
    else:
        rows = sorted(sentinel)
    A64 = as_numpy(A_h)[rows].astype(np.float64)
    B64 = as_numpy(B_h).astype(np.float64)
    ref = A64 @ B64
    tol = 4.0 * K * 2.0 ** -24 * (np.abs(A64) @ np.abs(B64))

    def check(C):
        got = C[rows].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        ok = bool(np.all(err <= tol))  # False on any NaN
        util = float(np.max(err / np.where(tol > 0, tol, 1.0))) if ok else None
        return ok, (round(util, 4) if util is not None else None)
    return check


def ladder(args, out):
    """Every variant on every selected workload: the results table."""
    import torch
    from roofline_sgemm_f32_amd import metrics as m
    from roofline_sgemm_f32_amd.inputs import WORKLOADS
    import roofline_sgemm_f32_amd as rs
    names = args.ladder_workloads.split(",")
    variants = ["k0_naive", "k1_coalesced", "k2_lds_tiled16", "k2_lds_tiled32", "k2_lds_tiled32_pad1", "k2_lds_tiled16_pad1",
                "k3_regtile_db", "k4_mfma_tile64", "k4_mfma_tile128", "k4_mfma_tile128x256", "k4_mfma",
                "auto"]
    rows = []
    for name in names:
        w = WORKLOADS[name]
        A_h, B_h, A, B, C = device_operands(w)
        flops = m.sgemm_flops(w.M, w.N, w.K)
        gate = row_gate(A_h, B_h)
        base_ms = None
        for v in variants:
            fn = run_gemm_factory(v, A, B, C)
            fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            one = time.perf_counter() - t0
            reps = int(max(1, min(args.ladder_reps, 3.0 / max(one, 1e-6))))
            total, per = time_launches(fn, reps, 1)
            ok, util = gate(C)
            if not ok:
                log(f"  {name:22s} {v:22s} outside the error bound on the gate rows: no throughput")
                rows.append({"workload": name, "variant": v, "gate": False, "bound_util": util})
                continue
            g = m.gflops(flops, per)
            if v == "k0_naive":
                base_ms = per
            rec = {"workload": name, "variant": v, "gate": True, "bound_util": util,
                   "ms": round(per, 4), "gflops": round(g, 1),
                   "pct_peak": round(m.pct_of_peak(g, m.MI355X_FP32_PEAK_GFLOPS), 2),
                   "speedup_vs_naive": round(base_ms / per, 2) if base_ms else None, "reps": reps}
            rows.append(rec)
            log(f"  {name:22s} {v:22s} {per:9.3f} ms {g:10.1f} GFLOP/s {rec['pct_peak']:6.2f}% "
                f"x{rec['speedup_vs_naive']}")
            if out:
                out.write(json.dumps({"ladder": rec}) + "\n")
        del A, B, C
        torch.cuda.empty_cache()
    return rows


# Small-shape path: shapes whose 64 x 64 tiles underfill the 256 compute
# units (the two small workloads plus K-heavy and skinny outputs), and one
# thin product (a single row of C, 1 GiB of B streamed), timed with the K
# split the library chooses and unsplit.
SMALL_SHAPES = {
    "square256": None,
    "square512": (512, 512, 512),
    "square1024": None,
    "kheavy128x128x4096": (128, 128, 4096),
    "kheavy256x256x16384": (256, 256, 16384),
    "kheavy1024x1024x4096": (1024, 1024, 4096),
    "skinny64x8192x8192": (64, 8192, 8192),
    "thin1x16384x16384": (1, 16384, 16384),
    "column16384x1x16384": (16384, 1, 16384),
    "mid768x1024x1024": (768, 1024, 1024),
}


def small_shapes(reps: int, only=None):
    """Per shape: chunks chosen, us per call split (as chosen) and unsplit:
    back-to-back calls on one stream (best of three rounds), so a call's time
    is the larger of its device time and its host launch cost."""
    import torch
    import roofline_sgemm_f32_amd as rs
    from roofline_sgemm_f32_amd import metrics as m
    from roofline_sgemm_f32_amd.inputs import WORKLOADS, make_operands
    lib = rs.load()
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for name, dims in SMALL_SHAPES.items():
        if only and name not in only:
            continue
        if dims is None:
            w = WORKLOADS[name]
            A_h, B_h, A, B, C = device_operands(w)
        else:
            M, N, K = dims
            A_h, B_h = make_operands(M, N, K, "uniform", seed=100 + len(rows))
            A, B = A_h.cuda(), B_h.cuda()
            C = torch.full((M, N), float("nan"), device="cuda")
        M, K = A.shape
        N = B.shape[1]
        args = (M, N, K, 1.0, A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0), 0.0,
                C.data_ptr(), C.stride(0))
        chunks, kchunk = rs.split_plan(M, N, K, lda=A.stride(0), ldb=B.stride(0),
                                       A_ptr=A.data_ptr(), B_ptr=B.data_ptr())
        plan = rs.plan_config(M, N, K, lda=A.stride(0), ldb=B.stride(0), A_ptr=A.data_ptr(),
                              B_ptr=B.data_ptr())

        def call(splits):
            def fn():
                st = lib.sgemm_f32_ex_split(0, 0, *args, splits, stream)
                if st != 0:
                    raise rs.SgemmError(st, "sgemm_f32_ex_split")
            return fn
        flops = m.sgemm_flops(M, N, K)
        # Warm up for about 50 ms per plan (the clock settles over tens of ms).
        t0 = time.perf_counter()
        call(1)()
        torch.cuda.synchronize()
        warm = int(min(5000, max(20, 0.05 / max(time.perf_counter() - t0, 1e-6))))
        # Three alternating rounds, best of each: these calls take a few us,
        # so host-side jitter would otherwise decide which plan looks faster.
        t_auto = t_one = float("inf")
        gate = row_gate(A_h, B_h)
        ok = True
        for _ in range(3):
            t_auto = min(t_auto, time_launches(call(0), reps, warm, per_launch=False)[0])
            ok = ok and gate(C)[0]
            t_one = min(t_one, time_launches(call(1), reps, warm, per_launch=False)[0])
            ok = ok and gate(C)[0]
        if not ok:
            log(f"  small {name:22s} outside the error bound on the gate rows: no throughput")
            rows.append({"shape": name, "M": M, "N": N, "K": K, "gate": False})
            del A, B, C
            continue
        rec = {"shape": name, "gate": True, "engine": plan["engine"], "tile": list(plan["tile"]), "M": M, "N": N, "K": K, "chunks": chunks, "kchunk": kchunk,
               "us_per_call": round(1e3 * t_auto, 2), "gflops": round(m.gflops(flops, t_auto), 1),
               "unsplit_us_per_call": round(1e3 * t_one, 2),
               "unsplit_gflops": round(m.gflops(flops, t_one), 1),
               "speedup_vs_unsplit": round(t_one / t_auto, 3)}
        rows.append(rec)
        log(f"  small {name:22s} {plan['engine']:4s} chunks={chunks:2d} {rec['us_per_call']:9.2f} us "
            f"{rec['gflops']:9.1f} GFLOP/s (unsplit {rec['unsplit_us_per_call']:9.2f} us) "
            f"x{rec['speedup_vs_unsplit']}")
        del A, B, C
    return rows


def cpu_all(seconds: float):
    """Every workload: the AUTO product on the GPU (mean of back-to-back
    launches) beside the CPU oracle on a bounded sample of the same product
    (all host threads; one thread too for the two small squares), with the
    oracle's rows gating the GPU's.  One JSON line per workload."""
    import torch
    from roofline_sgemm_f32_amd import metrics as m
    from roofline_sgemm_f32_amd.inputs import WORKLOADS
    rows = []
    for name, w in WORKLOADS.items():
        A_h, B_h, A, B, C = device_operands(w)
        fn = run_gemm_factory("auto", A, B, C)
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        # Back-to-back calls for about 0.5 s (at least 5), after as many warm-ups.
        steps = int(max(5, min(2000, 0.5 / max(time.perf_counter() - t0, 1e-6))))
        ms, _ = time_launches(fn, steps, steps, per_launch=False)
        gpu = m.gflops(m.sgemm_flops(w.M, w.N, w.K), ms)
        cpu, gate = cpu_baseline_leg(w, A_h, B_h, C, seconds)
        rec = {"workload": name, "gpu_gflops": round(gpu, 1), "gpu_ms": round(ms, 5),
               "cpu": cpu, "gpu_over_cpu": round(gpu / cpu["value"], 1), "gate": gate}
        if w.M <= 1024:
            one, _ = cpu_baseline_leg(w, A_h, B_h, C, seconds / 2, threads=1)
            rec["cpu_single_thread"] = one
        rows.append(rec)
        log(f"  {name:22s} GPU {gpu:10.1f} GFLOP/s  CPU {cpu['value']:8.2f} GFLOP/s ({cpu['cores']} threads)"
            f"  x{rec['gpu_over_cpu']}  gate {'ok' if gate['ok'] else 'FAILED'}"
            + (f"  1 thread {rec['cpu_single_thread']['value']:.2f}" if "cpu_single_thread" in rec else ""))
        print(json.dumps({"cpu_all": rec}), flush=True)
        del A, B, C
        torch.cuda.empty_cache()
    return rows


def main():
    from roofline_sgemm_f32_amd.inputs import WORKLOADS
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="square4096", choices=sorted(WORKLOADS))
    p.add_argument("--variant", default="auto")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target duration of the CPU oracle sample (0 skips the leg)")
    p.add_argument("--copy-steps", type=int, default=50)
    p.add_argument("--copy-sweep", action="store_true", help="block x grid sweep of the copy probe")
    p.add_argument("--no-compute-probe", dest="compute_probe", action="store_false",
                   help="skip the register-only FMA / MFMA rate probe")
    p.add_argument("--ladder", action="store_true", help="time every variant (table on stderr)")
    p.add_argument("--ladder-workloads", default="square4096")
    p.add_argument("--ladder-reps", type=int, default=20)
    p.add_argument("--out", default=None, help="append extra JSON lines (ladder, sweep) here")
    p.add_argument("--small-reps", type=int, default=200,
                   help="calls timed per small shape (0 skips the small-shape section)")
    p.add_argument("--small-only", default=None,
                   help="comma-separated small shapes: time only these and print their JSON")
    p.add_argument("--cpu-all", action="store_true",
                   help="only: every workload on the GPU beside the CPU oracle (one JSON line each)")
    p.add_argument("--configs-seconds", type=float, default=0.2,
                   help="timed calls per workload in the configs section (0 skips it)")
    args = p.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: this SGEMM runs on a single MI355X and has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import roofline_sgemm_f32_amd as rs
    from roofline_sgemm_f32_amd import metrics as m
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rs.load()  # raises when the HIP library is missing: no fallback
    out = open(args.out, "a") if args.out else None
    if args.cpu_all:
        ok = all(r["gate"]["ok"] for r in cpu_all(args.cpu_seconds))
        sys.exit(0 if ok else 3)
    if args.small_only:
        print(json.dumps({"small_shapes": small_shapes(max(args.small_reps, 1),
                                                       args.small_only.split(","))}), flush=True)
        return

    # The headline's operands are drawn and placed first, so that no host
    # work separates the probe legs from its launches.
    w = WORKLOADS[args.workload]
    A_h, B_h, A, B, C = device_operands(w)
    variant = args.variant
    resolved = variant
    if variant == "auto":
        resolved = rs.variant_name(rs.load().sgemm_auto_variant(
            w.M, w.N, w.K, A.data_ptr(), w.lda, B.data_ptr(), w.ldb, C.data_ptr(), w.ldc))
    fn = run_gemm_factory(variant, A, B, C)

    # The roofs first: the copy probe and the compute probes calibrate the
    # denominators the kernels are measured against.  Then the configs
    # section (the five workloads through AUTO), and the headline directly
    # after it.  The order matters for a headline of few warm-ups: square4096
    # launches settle at 0.961 ms, but start at 1.12-1.19 ms after 1 s of GPU
    # idleness (the clock ramps up over ~25 ms of load) and at 1.07 ms right
    # after the matrix-core probe (it runs the chip harder than the product
    # does, and the clock recovers over ~25 launches), while right after
    # other products of this kind the first launch already takes 0.966 ms
    # (MI355X, fresh processes).  The first launch of a kernel in a process
    # also carries its code object's loading (about 3 ms), which the
    # configs section pays instead of the headline's warm-ups.
    copy = copy_probe(args.copy_steps) if args.copy_steps > 0 else None
    probe = compute_probe() if args.compute_probe else None
    configs, keep = (configs_leg(args.configs_seconds) if args.configs_seconds > 0 else (None, {}))
    log(f"[bench] {w.name} {w.M}x{w.N}x{w.K} variant={variant} ({resolved}) "
        f"warmup={args.warmup} steps={args.steps}")
    # The timed region is the K back-to-back launches between two events on
    # the launch stream; the average launch duration is the step time.
    ms_step, _ = time_launches(fn, args.steps, args.warmup, per_launch=False)
    ms_launch = ms_step
    flops = m.sgemm_flops(w.M, w.N, w.K)
    value = m.gflops(flops, ms_step)
    achieved_tf = flops / (ms_launch / 1e3) / 1e12
    peak_tf = m.MI355X_FP32_PEAK_GFLOPS / 1e3
    log(f"[bench] {ms_step:.4f} ms/step, {value:.1f} GFLOP/s, "
        f"{m.pct_of_peak(value, m.MI355X_FP32_PEAK_GFLOPS):.2f}% of FP32 peak")
    if copy:
        log(f"[bench] copy probe {copy['gbs']} GB/s ({100 * copy['frac']:.1f}% of 8 TB/s)")
    if probe:
        log(f"[bench] compute probe: FP32 FMA chains {probe['valu_fma_tflops']} TFLOP/s "
            f"(best {probe['valu_fma_tflops_best']}), FP32 MFMA {probe['mfma_f32_tflops']} TFLOP/s "
            f"(best {probe['mfma_f32_tflops_best']})")
    # The timed launches' result, checked by the CPU leg.
    C_host = C.cpu().numpy()
    del A, B, C
    torch.cuda.empty_cache()

    if args.copy_sweep:
        from roofline_sgemm_f32_amd.inputs import COPY_ELEMENTS  # noqa: F401
        for block in (64, 128, 256, 512, 1024):
            for grid in (256, 1024, 4096, 16384, 65536):
                r = copy_probe(max(10, args.copy_steps // 2), block, grid)
                log(f"  copy block={block:5d} grid={grid:6d} {r['gbs']:8.1f} GB/s")
                if out:
                    out.write(json.dumps({"copy_sweep": r}) + "\n")
    if args.ladder:
        ladder(args, out)
    small = small_shapes(args.small_reps) if args.small_reps > 0 else None

    # The CPU leg runs last: the GPU clock falls during its seconds of GPU
    # idleness, which would slow GPU work timed after it.  The oracle's
    # results gate the headline product and every config's.
    cpu, gate = None, None
    if args.cpu_seconds > 0:
        log(f"[bench] cpu baseline leg (~{args.cpu_seconds:.0f} s, then the full-product gates)")
        cpu, gate = cpu_baseline_leg(w, A_h, B_h, C_host, args.cpu_seconds)
        log(f"[bench] oracle {cpu['value']} GFLOP/s; gate {gate}")
        for rec in configs or []:
            cw, ca, cb, cc = keep[rec["workload"]]
            rec["gate"] = oracle_gate(cw, ca, cb, cc.cpu().numpy())
            if not rec["gate"]["ok"]:
                rec["gflops"] = rec["pct_peak"] = None
            log(f"  gate {rec['workload']:22s} {rec['gate']}")
        keep.clear()

    traffic = read_traffic(resolved, w.name)
    kernel = resolved
    line = {
        "metric": METRIC,
        "value": round(value, 1) if (gate is None or gate["ok"]) else None,
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "lda": w.lda, "ldb": w.ldb,
                   "ldc": w.ldc, "dist": w.dist, "seed": w.seed, "variant": variant,
                   "kernel": kernel, "parallelism": "single_gpu"},
        "pct_of_fp32_peak": round(m.pct_of_peak(value, m.MI355X_FP32_PEAK_GFLOPS), 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved_tf, 3), "peak": round(peak_tf, 1),
                     "unit": "TFLOP/s", "frac": round(achieved_tf / peak_tf, 4),
                     "traffic": traffic, "kernel": kernel,
                     "flops_per_launch": flops, "ms_per_launch": round(ms_launch, 5)},
        "cpu_baseline": cpu,
        "gate": gate,
        "headline_preceded_by": ["hbm_copy", "compute_probe"] + (["configs"] if configs else []),
        "hbm_copy": copy,
        "compute_probe": probe,
        "configs": configs,
        "small_shapes": small,
    }
    if out:
        out.write(json.dumps({"bench": line}) + "\n")
        out.close()
    print(json.dumps(line), flush=True)
    if gate is not None and not gate["ok"]:
        sys.exit(3)
    if any(not r.get("gate", {"ok": True})["ok"] for r in configs or []):
        sys.exit(3)


if __name__ == "__main__":
    main()
