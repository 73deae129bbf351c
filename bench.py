#!/usr/bin/env python3
"""Benchmark of the swizzled tiled GEMM on one MI355X.

A step is one pass of the whole hot path -- one persistent GEMM launch: the
swizzled task -> tile map, the global -> LDS pipeline, the MFMA K loop, the
tail masks, the K-split fix-up and the epilogue -- over the resident
synthetic operands of the workload.  The headline workload is the fp16
1024 x 1024 x 2048 GEMM (row-major A, B ~ U[-1, 1], fp32 accumulate, fp16
out); the MX-fp8 1024 x 2048 x 4096 GEMM is timed the same way and reported
under "mxfp8".

Prints ONE JSON line.  `roofline` uses the average duration of the timed
launches (HIP events on the launch stream) against the fp16 dense MFMA peak
of MI355X (2.5 PFLOP/s; 5.0 for fp8); `cpu_baseline` times the CPU oracle
(fp64, OpenMP) on the same workload on this host.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"f16": 2500.0, "bf16": 2500.0, "e4m3": 5000.0, "i8": 5000.0}   # TFLOP/s (TOP/s) dense


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("block_swizzle_tile_amd/csrc/bst.hip", "block_swizzle_tile_amd/csrc/bst_device.hpp"):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(name, launches_bytes_alg):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--tile", default="128x128")
    p.add_argument("--split", type=int, default=0)
    p.add_argument("--offset", type=int, default=2)
    p.add_argument("--direction", default="zn")
    p.add_argument("--remap", type=int, default=1)
    p.add_argument("--grid", type=int, default=0)
    p.add_argument("--mx-tile", default="128x128")
    p.add_argument("--mx-split", type=int, default=0)
    p.add_argument("--no-mx", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = auto)")
    return p.parse_args()


def time_launches(fn, steps, warmup):
    """Run fn() warmup times, then steps times between a start and an end
    event, with an event pair around every launch; returns (total ms,
    mean per-launch ms)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(st)
    for a, b in ev:
        a.record(st)
        fn()
        b.record(st)
    t1.record(st)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    per = [a.elapsed_time(b) for a, b in ev]
    return total, sum(per) / len(per), sorted(per)[len(per) // 2]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the GEMM would shard by tiles / batches / groups with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_swizzle_tile_amd as bst
    from block_swizzle_tile_amd import inputs as I

    def gpu(arr, kind):
        a = np.ascontiguousarray(arr)
        if kind == "f16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
        if kind == "e4m3":
            return torch.from_numpy(a.view(np.uint8)).cuda().view(torch.float8_e4m3fn)
        return torch.from_numpy(a).cuda()

    # ---------------------------------------------------------- fp16 2k --
    w = I.workload("fp16_2k")
    M, N, K = w["M"], w["N"], w["K"]
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    tm, tn = map(int, args.tile.split("x"))
    sched = bst.make_sched(tile=(tm, tn), offset=args.offset, direction=args.direction,
                           split_k=args.split, xcd_remap=args.remap, grid=args.grid)
    eff = bst.effective_sched(0, bst.F16, 1, M, N, K, sched)
    nb = bst.workspace_bytes(0, bst.F16, 1, M, N, K, sched)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")

    def step():
        bst.gemm(A, B, C, sched=sched, workspace=ws)

    total_ms, mean_ms, med_ms = time_launches(step, args.steps, args.warmup)
    flop = 2.0 * M * N * K
    ms_per_step = total_ms / args.steps
    value = flop * args.steps / (total_ms * 1e-3) / 1e12
    achieved = flop / (mean_ms * 1e-3) / 1e12

    # spot check of the timed configuration against the oracle (4 rows)
    import oracle
    rows = np.array([0, 1, M // 2, M - 1], np.int64)
    ref, den = oracle.gemm(oracle.F16, w["A"], w["B"], tile=(tm, tn), rows=rows)
    got = oracle.decode("f16", C.cpu().view(torch.int16).numpy().view(np.uint16)[rows])
    err, _ = oracle.compare(got, ref, den)
    if not err <= 2.0 ** -9:
        print("parity check failed: %g" % err, file=sys.stderr)
        sys.exit(1)

    traffic = traffic_from_profile("fp16_2k", None)
    out = {
        "metric": "TFLOP/s and % of MFMA peak, fp16 1024x1024x2048 & mxfp8 1024x2048x4096",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded U[-1,1] fp16 operands)",
        "config": {
            "workload": "fp16 GEMM M=1024 N=1024 K=2048, row-major A/B, fp32 accumulate, fp16 out",
            "tile": [eff.tile_m, eff.tile_n, eff.tile_k], "split_k": eff.split_k,
            "swizzle": {"offset": eff.swizzle_offset,
                        "direction": ["zn", "nz", "raster"][eff.swizzle_direction]},
            "xcd_remap": eff.xcd_remap, "grid": eff.grid,
        },
        "pct_of_peak": round(100.0 * value / PEAK["f16"], 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK["f16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK["f16"], 4),
                     "traffic": traffic, "kernel_ms_mean": round(mean_ms, 5),
                     "kernel_ms_median": round(med_ms, 5),
                     "flop_per_launch": flop},
        "parity_max_norm_err": err,
    }

    # ---------------------------------------------------------- MX-fp8 --
    if not args.no_mx:
        x = I.workload("mxfp8_4k")
        Mx, Nx, Kx = x["M"], x["N"], x["K"]
        Ax, Bx = gpu(x["A"], "e4m3"), gpu(x["B"], "e4m3")
        sa, sb = gpu(x["scale_a"], "u8"), gpu(x["scale_b"], "u8")
        Cx = torch.empty((Mx, Nx), dtype=torch.bfloat16, device="cuda")
        xm, xn = map(int, args.mx_tile.split("x"))
        sx = bst.make_sched(tile=(xm, xn), offset=args.offset, direction=args.direction,
                            split_k=args.mx_split, xcd_remap=args.remap)
        effx = bst.effective_sched(0, bst.MXE4M3, 1, Mx, Nx, Kx, sx)
        nbx = bst.workspace_bytes(0, bst.MXE4M3, 1, Mx, Nx, Kx, sx)
        wsx = torch.zeros(max(nbx, 16), dtype=torch.uint8, device="cuda")

        def stepx():
            bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=sx, workspace=wsx)

        tot, mean_x, med_x = time_launches(stepx, args.steps, args.warmup)
        fx = 2.0 * Mx * Nx * Kx
        vx = fx * args.steps / (tot * 1e-3) / 1e12
        out["mxfp8"] = {
            "workload": "MX-fp8 GEMM M=1024 N=2048 K=4096, e4m3 + e8m0 per-32 scales, bf16 out",
            "value": round(vx, 2), "unit": "TFLOP/s",
            "pct_of_peak": round(100.0 * vx / PEAK["e4m3"], 2),
            "ms_per_step": round(tot / args.steps, 5),
            "kernel_ms_mean": round(mean_x, 5), "kernel_ms_median": round(med_x, 5),
            "achieved": round(fx / (mean_x * 1e-3) / 1e12, 2), "peak": PEAK["e4m3"],
            "tile": [effx.tile_m, effx.tile_n, effx.tile_k], "split_k": effx.split_k,
        }

    # ---------------------------------------------------- CPU baseline --
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        nrows = args.cpu_rows or M
        rows = None if nrows >= M else np.linspace(0, M - 1, nrows).astype(np.int64)
        t = time.perf_counter()
        oracle.gemm(oracle.F16, w["A"], w["B"], tile=(tm, tn), rows=rows)
        dt = time.perf_counter() - t
        omp = int(os.environ.get("OMP_NUM_THREADS", cores))
        out["cpu_baseline"] = {
            "value": round(2.0 * nrows * N * K / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": min(omp, cores), "kind": "oracle",
            "sample": "%d of %d output rows of the fp16 1024x1024x2048 workload (fp64 oracle, "
                      "%.2f s)" % (nrows, M, dt),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
