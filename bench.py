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

Legs:
  * GPU product: value = 2 M N K / mean step time.
  * roofline: the matrix-core kernel's achieved TFLOP/s against 157.3, from
    per-launch events on the launch stream; ``traffic`` is read from a
    committed counter summary when it was taken on the current kernel source.
  * hbm_copy: the copy probe (256 Mi floats, 2 GiB moved) against 8 TB/s.
  * cpu_baseline: the CPU oracle timed on this host on a bounded sample of
    rows of the same product; its rows also gate the GPU result.
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


def kernel_source_hash(files=("k4_mfma.hip",)) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "roofline_sgemm_f32_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
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


def time_launches(fn, steps: int, warmup: int):
    """Warm up, then time ``steps`` back-to-back launches on the current
    stream; returns (mean ms per step, mean ms per launch from per-launch
    event pairs)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1) / steps
    per = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / steps
    return total, per


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


def cpu_baseline_leg(w, A_h, B_h, C_dev, budget_s: float):
    """Time the CPU oracle on a bounded sample of rows of the same product,
    and check the GPU's rows against it."""
    import numpy as np
    import oracle
    from oracle import check
    from roofline_sgemm_f32_amd import metrics as m
    from roofline_sgemm_f32_amd.inputs import as_numpy
    An, Bn = as_numpy(A_h), as_numpy(B_h)
    threads = oracle.default_threads()
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
    rep = check.check(C_dev[rows.tolist()].cpu().numpy(), ref, S, w.K)
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
    gate = {"rows_checked": len(rows), "ok": rep["ok"], "max_bound_util": rep["max_bound_util"],
            "max_rel_err_page": rep["max_rel_err_page"], "n_violations": rep["n_violations"]}
    return base, gate


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


def compute_probe(valu_iters=4096, mfma_iters=2048):
    """Sustained FP32 rate of register-only multiply-add chains (vector ALU)
    and of back-to-back FP32 matrix instructions, for the compute roof."""
    import torch
    import roofline_sgemm_f32_amd as rs
    from roofline_sgemm_f32_amd.inputs import probe_operands
    blocks, block = 256 * 8, 256  # 32 waves per CU
    out_v = torch.empty((blocks * block, 16), device="cuda")
    _, per_v = time_launches(lambda: rs.probe_valu(blocks, block, valu_iters, 0.999, 0.001, out_v), 5, 1)
    valu_tf = blocks * block * valu_iters * 16 * 2 / (per_v * 1e-3) / 1e12
    a, b = probe_operands(7)
    a, b = a.cuda(), b.cuda()
    mblocks = 256 * 4  # 16 waves per CU
    out_m = torch.empty((mblocks * 4, 4, 32, 32), device="cuda")
    _, per_m = time_launches(lambda: rs.probe_mfma(a, b, mblocks, mfma_iters, out_m), 5, 1)
    mfma_tf = mblocks * 16 * mfma_iters * 4096 / (per_m * 1e-3) / 1e12
    return {"valu_fma_tflops": round(valu_tf, 2), "mfma_f32_tflops": round(mfma_tf, 2),
            "valu_ms": round(per_v, 4), "mfma_ms": round(per_m, 4)}


def ladder(args, out):
    """Every variant on every selected workload: the results table."""
    import torch
    from roofline_sgemm_f32_amd import metrics as m
    from roofline_sgemm_f32_amd.inputs import WORKLOADS
    import roofline_sgemm_f32_amd as rs
    names = args.ladder_workloads.split(",")
    variants = ["k0_naive", "k1_coalesced", "k2_lds_tiled16", "k2_lds_tiled32", "k2_lds_tiled32_pad1", "k2_lds_tiled16_pad1",
                "k3_regtile_db", "k4_mfma_tile64", "k4_mfma_tile128", "k4_mfma", "auto"]
    rows = []
    for name in names:
        w = WORKLOADS[name]
        A_h, B_h, A, B, C = device_operands(w)
        flops = m.sgemm_flops(w.M, w.N, w.K)
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
            g = m.gflops(flops, per)
            if v == "k0_naive":
                base_ms = per
            rec = {"workload": name, "variant": v, "ms": round(per, 4), "gflops": round(g, 1),
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


def main():
    from roofline_sgemm_f32_amd.inputs import WORKLOADS
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
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

    w = WORKLOADS[args.workload]
    A_h, B_h, A, B, C = device_operands(w)
    variant = args.variant
    resolved = variant
    if variant == "auto":
        resolved = rs.variant_name(rs.load().sgemm_auto_variant(
            w.M, w.N, w.K, A.data_ptr(), w.lda, B.data_ptr(), w.ldb, C.data_ptr(), w.ldc))
    fn = run_gemm_factory(variant, A, B, C)
    log(f"[bench] {w.name} {w.M}x{w.N}x{w.K} variant={variant} ({resolved}) "
        f"warmup={args.warmup} steps={args.steps}")
    ms_step, ms_launch = time_launches(fn, args.steps, args.warmup)
    flops = m.sgemm_flops(w.M, w.N, w.K)
    value = m.gflops(flops, ms_step)
    achieved_tf = flops / (ms_launch / 1e3) / 1e12
    peak_tf = m.MI355X_FP32_PEAK_GFLOPS / 1e3
    log(f"[bench] {ms_step:.4f} ms/step, {value:.1f} GFLOP/s, "
        f"{m.pct_of_peak(value, m.MI355X_FP32_PEAK_GFLOPS):.2f}% of FP32 peak")

    cpu, gate = None, None
    if args.cpu_seconds > 0:
        log(f"[bench] cpu baseline leg (~{args.cpu_seconds:.0f} s)")
        cpu, gate = cpu_baseline_leg(w, A_h, B_h, C, args.cpu_seconds)
        log(f"[bench] oracle {cpu['value']} GFLOP/s; gate {gate}")

    copy = copy_probe(args.copy_steps) if args.copy_steps > 0 else None
    if copy:
        log(f"[bench] copy probe {copy['gbs']} GB/s ({100 * copy['frac']:.1f}% of 8 TB/s)")
    probe = compute_probe() if args.compute_probe else None
    if probe:
        log(f"[bench] compute probe: FP32 FMA chains {probe['valu_fma_tflops']} TFLOP/s, "
            f"FP32 MFMA {probe['mfma_f32_tflops']} TFLOP/s")
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
        "hbm_copy": copy,
        "compute_probe": probe,
    }
    if out:
        out.write(json.dumps({"bench": line}) + "\n")
        out.close()
    print(json.dumps(line), flush=True)
    if gate is not None and not gate["ok"]:
        sys.exit(3)


if __name__ == "__main__":
    main()
