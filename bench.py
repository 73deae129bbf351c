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
launches (one HIP-graph replay of them between two events on the launch
stream) against the fp16 dense MFMA peak
of MI355X (2.5 PFLOP/s; 5.0 for fp8); `cpu_baseline` times the CPU oracle
(fp64, OpenMP) on the same workload on this host.

Other modes (one JSON line per measurement): --all-configs (every workload
configuration), --l2-sweep (every swizzle setting, for rocprofv3 counters),
--sweep-configs (every configuration's schedules, for rocprofv3 counters),
--summarize (the table of a sweep's rocprofv3 runs),
--large (4096^3 and 8192x8192x4096 beside the library GEMMs torch calls),
--clock (shader clock under each workload, with the cycle-accounting build),
--calib-copy and --traffic-from (HBM traffic calibration and summary).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CALIB_BYTES = 256 << 20   # the calibration copy moves this many bytes each way
PEAK = {"f16": 2500.0, "bf16": 2500.0, "e4m3": 5000.0, "i8": 5000.0}   # TFLOP/s (TOP/s) dense


def kernel_source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "block_swizzle_tile_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(open(os.path.join(d, f), "rb").read())
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


def _pmc_values(d, counter, name_part):
    """Per-dispatch values of one counter from a rocprofv3 --pmc CSV run under d,
    for kernels whose name contains name_part (case-insensitive)."""
    import csv
    import glob
    vals = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"].lower():
                vals.append(float(r["Counter_Value"]))
    return vals


def traffic_summary(d, calib_bytes):
    """HBM bytes per launch of the fp16 workload from four PMC runs under d:
    fetch/ and write/ (FETCH_SIZE, WRITE_SIZE of the bench's fp16 launches),
    calib_fetch/ and calib_write/ (the same counters on --calib-copy, a plain
    copy of calib_bytes bytes).  Each counter is scaled by what it reads for
    the copy; the result goes to profiles/traffic_fp16_2k.json with the
    kernel source hash it was taken on."""
    def med(v):
        v = sorted(v[1:] if len(v) > 2 else v)   # the first launch is cold
        return v[len(v) // 2]
    fk = _pmc_values(os.path.join(d, "fetch"), "FETCH_SIZE", "gemm_dma_kernel")
    wk = _pmc_values(os.path.join(d, "write"), "WRITE_SIZE", "gemm_dma_kernel")
    cf = _pmc_values(os.path.join(d, "calib_fetch"), "FETCH_SIZE", "copy")
    cw = _pmc_values(os.path.join(d, "calib_write"), "WRITE_SIZE", "copy")
    if not (fk and wk and cf and cw):
        sys.exit("traffic: missing PMC values under %s" % d)
    ff = calib_bytes / (med(cf) * 1024.0)
    fw = calib_bytes / (med(cw) * 1024.0)
    fetch_b, write_b = med(fk) * 1024.0 * ff, med(wk) * 1024.0 * fw
    res = {"kernel_hash": kernel_source_hash(),
           "hbm_bytes_per_launch": round(fetch_b + write_b),
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "fetch_kib_raw": med(fk), "write_kib_raw": med(wk),
           "copy_scale_fetch": round(ff, 4), "copy_scale_write": round(fw, 4),
           "dispatches": [len(fk), len(wk), len(cf), len(cw)]}
    with open(os.path.join(ROOT, "profiles", "traffic_fp16_2k.json"), "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res), flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--tile", default="64x64")
    p.add_argument("--split", type=int, default=1)
    p.add_argument("--offset", type=int, default=8)
    p.add_argument("--direction", default="zn")
    p.add_argument("--remap", type=int, default=1)
    p.add_argument("--grid", type=int, default=0)
    p.add_argument("--shuffle-k", type=int, default=1,
                   help="fp16 workload: 1 = ShuffleK, each task's K loop starts at a rotated "
                        "stage (2-4%% faster here), 0 = in order")
    p.add_argument("--mx-shuffle-k", type=int, default=1,
                   help="MX-fp8 workload: ShuffleK (the start stage rounded down to a group of "
                        "four stages of A's block scales; 2-4%% faster here)")
    p.add_argument("--mx-tile", default="64x128")
    p.add_argument("--mx-split", type=int, default=1)
    p.add_argument("--no-mx", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = auto)")
    p.add_argument("--l2-sweep", action="store_true",
                   help="only run the fp16 and MX-fp8 workloads under every swizzle setting (Zn / "
                        "Nz offsets 1, 2, 4, 8 and RASTER, XCD remap off / on) at their named and "
                        "fastest tiles, --steps launches each, for per-setting rocprofv3 counters")
    p.add_argument("--all-configs", action="store_true",
                   help="time every workload configuration (one JSON line per schedule)")
    p.add_argument("--traffic-from", default="",
                   help="write profiles/traffic_fp16_2k.json from the PMC runs under this folder")
    p.add_argument("--large", action="store_true",
                   help="time fp16 and MX-fp8 GEMMs at 4096^3 and 8192x8192x4096 (256x256 tiles) "
                        "and the library GEMMs torch calls for the same shapes")
    p.add_argument("--clock", action="store_true",
                   help="with the cycle-accounting build (python -m block_swizzle_tile_amd.build "
                        "--trace): the shader clock each workload's workgroups ran at")
    p.add_argument("--phases", action="store_true",
                   help="with the cycle-accounting build (python -m block_swizzle_tile_amd.build "
                        "--trace): where a work unit's cycles go, per workload")
    p.add_argument("--wg-times", action="store_true",
                   help="per-workgroup start / end times of one launch of C5 and the slice-K "
                        "workload per schedule, from the production kernels' clock record")
    p.add_argument("--sweep-configs", action="store_true",
                   help="launch every configuration's named and fastest schedules --steps times "
                        "each, eagerly and in a fixed order, for per-dispatch rocprofv3 counters")
    p.add_argument("--plan-out", default="",
                   help="with --l2-sweep / --sweep-configs: write the launch plan here")
    p.add_argument("--summarize", default="",
                   help="print the per-setting table of the rocprofv3 runs of a sweep under this "
                        "folder (plan.json, trace/, tcc/, fetch/, write/, sq/, calib_*/)")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run plain 256 MiB device copies (the known-size reference that "
                        "scales the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def time_launches(fn, steps, warmup, min_warm_s=0.1):
    """Run fn() `warmup` times eagerly, capture `steps` calls of fn() in one
    HIP graph (so host launch overhead does not enter the timing), replay it
    untimed until at least min_warm_s of GPU work has run (an idle GPU's
    clock takes that long to ramp up; the first workload of a process was
    otherwise measured up to 15% slow), then time one replay between two
    events on the launch stream.  Returns (total ms, ms per launch)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            fn()
    t_end = time.perf_counter() + min_warm_s
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    st = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(st)
    g.replay()
    t1.record(st)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    return total, total / steps


def median_launch(bst, fn, n=50):
    """Median over n launches of fn() of each launch's span on the device: from its first
    workgroup's start to its last workgroup's end, read from the production kernels'
    clock record (100 MHz reference counter, 10 ns steps).  Launches run eagerly one after
    another; the span leaves out the host's launch overhead and the dispatch before the
    first workgroup starts.  Returns ms (after at least 0.1 s of warm-up launches)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.1:
        fn()
        torch.cuda.synchronize()
    nwg = 1024
    buf = torch.zeros((n, nwg, 4), dtype=torch.int64, device="cuda")
    try:
        for i in range(n):
            bst.clock_record(buf[i], nwg)
            fn()
    finally:
        bst.clock_record()
    torch.cuda.synchronize()
    t = buf.cpu()
    spans = []
    for i in range(n):
        r = t[i][t[i][:, 3] == 1]
        spans.append(float(r[:, 1].max() - r[:, 0].min()) / 100.0 / 1e3)   # ms
    spans.sort()
    return spans[len(spans) // 2]


def shader_clock(bst, fn):
    """Shader clock (MHz) the workgroups of one launch of fn() ran at, from the production
    kernels' clock record (bst_set_clock_record): median, min and max over the recorded
    workgroups, after at least 0.1 s of warm-up launches."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.1:
        fn()
        torch.cuda.synchronize()
    buf = torch.zeros(4 * 1024, dtype=torch.int64, device="cuda")
    bst.clock_record(buf, 1024)
    try:
        fn()
        torch.cuda.synchronize()
    finally:
        bst.clock_record()
    t = buf.cpu().view(1024, 4)
    t = t[t[:, 3] == 1].double()
    ticks = (t[:, 1] - t[:, 0]).clamp(min=1)
    mhz = t[:, 2] / (ticks / 100.0)
    return {"sclk_mhz_median": round(float(mhz.median()), 0),
            "sclk_mhz_min": round(float(mhz.min()), 0),
            "sclk_mhz_max": round(float(mhz.max()), 0), "workgroups": int(t.shape[0])}


def _run_plan(args, plan, runners, torch):
    """Launch every planned setting args.steps times (eager, in plan order), after writing the
    plan (label, workload, schedule, flop and MFMA cycles per launch) to args.plan_out, so a
    rocprofv3 run can attribute its per-dispatch records to settings."""
    bst = sys.modules["block_swizzle_tile_amd"]
    print(json.dumps({"plan": plan, "launches_each": args.steps}), flush=True)
    if args.plan_out:
        with open(args.plan_out, "w") as f:
            json.dump({"plan": plan, "launches_each": args.steps}, f, indent=1)
    for c in plan:
        kw = dict(c["sched"])
        kw["tile"] = tuple(kw["tile"])
        s = bst.make_sched(**kw)
        for _ in range(args.steps):
            runners[c["workload"]](s)
        torch.cuda.synchronize()


# flop per MFMA cycle of one SIMD, per operand type: 32x32x16 f16 / bf16 every 32 cycles, i8
# 32x32x32 every 32, scaled f8f6f4 32x32x64 every 64
MFMA_FLOP_PER_CLK = {"f16": 1024, "bf16": 1024, "i8": 2048, "e4m3": 2048}


def l2_sweep(args, bst, I, gpu, torch):
    """Every swizzle setting on the fp16 1024x1024x2048 workload (tiles 256x128 and 64x64)
    and on the MX-fp8 1024x2048x4096 one (256x256 and 64x128): Zn / Nz with offsets 1, 2,
    4, 8 and RASTER, each with the XCD remap off and on, split 1."""
    w = I.workload("fp16_2k")
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    x = I.workload("mxfp8_4k")
    Ax, Bx = gpu(x["A"], "e4m3"), gpu(x["B"], "e4m3")
    sa, sb = gpu(x["scale_a"], "u8"), gpu(x["scale_b"], "u8")
    Cx = torch.empty((x["M"], x["N"]), dtype=torch.bfloat16, device="cuda")
    runners = {"fp16_2k": lambda s: bst.gemm(A, B, C, sched=s),
               "mxfp8_4k": lambda s: bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=s)}
    f2, f3 = 2.0 * 1024 * 1024 * 2048, 2.0 * 1024 * 2048 * 4096
    plan = []
    for wl, dt, flop, tiles in (("fp16_2k", "f16", f2, ((256, 128), (64, 64))),
                                ("mxfp8_4k", "e4m3", f3, ((256, 256), (64, 128)))):
        for tile in tiles:
            for remap in (0, 1):
                orders = [(d, off) for d in ("zn", "nz") for off in (1, 2, 4, 8)] + [("raster", 1)]
                for d, off in orders:
                    label = "%s %dx%d remap%d %s" % (wl, tile[0], tile[1], remap,
                                                     "RASTER" if d == "raster" else "%s%d" % (d.capitalize(), off))
                    plan.append({"label": label, "workload": wl, "dtype": dt, "flop": flop,
                                 "mfma_cycles": flop / MFMA_FLOP_PER_CLK[dt],
                                 "alg_bytes": 10485760 if wl == "fp16_2k" else 17170432,
                                 "sched": {"tile": list(tile), "offset": off, "direction": d,
                                           "xcd_remap": remap}})
    _run_plan(args, plan, runners, torch)


def sweep_configs(args, bst, I, gpu, torch):
    """Each workload configuration at its named tile and at its fastest schedules (the
    --all-configs set, padding matmul aside), for per-dispatch rocprofv3 counters."""
    w = I.workload("tails")
    A1, B1 = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C1 = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    w = I.workload("fp16_2k")
    A2, B2 = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C2 = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    x = I.workload("mxfp8_4k")
    Ax, Bx = gpu(x["A"], "e4m3"), gpu(x["B"], "e4m3")
    sa, sb = gpu(x["scale_a"], "u8"), gpu(x["scale_b"], "u8")
    Cx = torch.empty((x["M"], x["N"]), dtype=torch.bfloat16, device="cuda")
    b = I.workload("bf16_batch")
    Ab, Bb = gpu(b["A"], "bf16"), gpu(b["B"], "bf16")
    Cb = torch.empty((b["batch"], b["M"], b["N"]), dtype=torch.bfloat16, device="cuda")
    g = I.workload("int8_groups")
    Ag, Bg, gm = gpu(g["A"], "i8"), gpu(g["B"], "i8"), gpu(g["group_m"], "i32")
    rs, cs = gpu(g["row_scale"], "f32"), gpu(g["col_scale"], "f32")
    Cg = torch.empty((g["total_m"], g["N"]), dtype=torch.bfloat16, device="cuda")
    k = I.workload("int8_slice_k")
    Ak, Bk, gk = gpu(k["A"], "i8"), gpu(k["B"], "i8"), gpu(k["group_k"], "i32")
    rk, ck = gpu(k["row_scale"], "f32"), gpu(k["col_scale"], "f32")
    Ck = torch.empty((k["G"], k["M"], k["N"]), dtype=torch.bfloat16, device="cuda")
    runners = {
        "C1": lambda s: bst.gemm(A1, B1, C1, sched=s),
        "C2": lambda s: bst.gemm(A2, B2, C2, sched=s),
        "C3": lambda s: bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=s),
        "C4": lambda s: bst.batched_gemm(Ab, Bb, Cb, sched=s),
        "C5": lambda s: bst.grouped_gemm_slice_m(Ag, Bg, gm, Cg, row_scale=rs, col_scale=cs,
                                                 sched=s),
        "SK": lambda s: bst.grouped_gemm_slice_k(Ak, Bk, gk, Ck, row_scale=rk, col_scale=ck,
                                                 sched=s),
    }
    info = {  # workload: (name, dtype, flop, algorithmic bytes)
        "C1": ("C1 fp16 200x136x256", "f16", 2.0 * 200 * 136 * 256, 226432),
        "C2": ("C2 fp16 1024x1024x2048", "f16", 2.0 * 1024 * 1024 * 2048, 10485760),
        "C3": ("C3 MX-fp8 1024x2048x4096", "e4m3", 2.0 * 1024 * 2048 * 4096, 17170432),
        "C4": ("C4 bf16 16x512x768x1024", "bf16", 2.0 * 16 * 512 * 768 * 1024, 54525952),
        "C5": ("C5 int8 grouped 8192x4096x2048 dequant", "i8", 2.0 * 8192 * 4096 * 2048,
               151158816),
        "SK": ("int8 slice-K 8x(1024x2048) K 8192 dequant", "i8", 2.0 * 1024 * 2048 * 8192,
               1024 * 8192 + 8192 * 2048 + 8 * 1024 * 2048 * 2 + 8 * (1024 + 2048) * 4),
    }
    scheds = [
        ("C1", dict(tile=[64, 64], offset=3, direction="zn")),
        ("C2", dict(tile=[256, 128], offset=4, direction="zn")),
        ("C2", dict(tile=[64, 64], offset=8, direction="zn", xcd_remap=1, shuffle_k=1)),
        ("C3", dict(tile=[256, 256], offset=4, direction="zn")),
        ("C3", dict(tile=[64, 128], offset=8, direction="zn", xcd_remap=1)),
        ("C4", dict(tile=[128, 192], offset=1, direction="zn")),
        ("C4", dict(tile=[128, 192], offset=1, direction="zn", xcd_remap=1)),
        ("C4", dict(tile=[128, 128], offset=4, direction="zn", xcd_remap=1, path=3)),
        ("C5", dict(tile=[256, 256], offset=1, direction="zn")),
        ("C5", dict(tile=[128, 128], offset=4, direction="zn", xcd_remap=1, path=2)),
        ("C5", dict(tile=[128, 128], offset=4, direction="zn", xcd_remap=1, path=2, dynamic=1)),
        ("C5", dict(tile=[128, 128], offset=4, direction="zn", xcd_remap=1, path=3)),
        ("C5", dict(tile=[128, 128], offset=4, direction="zn", xcd_remap=1, path=3, dynamic=1)),
        ("SK", dict(tile=[128, 128], offset=4, direction="zn", xcd_remap=1)),
    ]
    plan = []
    for wl, kw in scheds:
        name, dt, flop, alg = info[wl]
        label = "%s %dx%d %s%s" % (name, kw["tile"][0], kw["tile"][1],
                                   "%s%d" % (kw["direction"].capitalize(), kw["offset"]),
                                   "".join(" %s" % k for k in ("xcd_remap", "shuffle_k", "dynamic")
                                           if kw.get(k)) +
                                   (" path%d" % kw["path"] if kw.get("path") else ""))
        plan.append({"label": label, "workload": wl, "dtype": dt, "flop": flop,
                     "mfma_cycles": flop / MFMA_FLOP_PER_CLK[dt], "alg_bytes": alg, "sched": kw})
    _run_plan(args, plan, runners, torch)


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        rows.extend(csv.DictReader(open(f)))
    return rows


def _ours(name):
    return "bst::gemm" in name


def summarize(d):
    """Markdown table of a sweep's rocprofv3 runs under d: plan.json (from --plan-out),
    trace/ (--kernel-trace), tcc/ (TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum), fetch/
    (FETCH_SIZE), write/ (WRITE_SIZE), sq/ (SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT
    SQ_INSTS_LDS) and, for the copy calibration, calib_fetch/ and calib_write/ (FETCH_SIZE /
    WRITE_SIZE of --calib-copy).  Per setting, medians over its launches after the first."""
    plan = json.load(open(os.path.join(d, "plan.json")))
    n, settings = plan["launches_each"], plan["plan"]

    def per_dispatch(sub, counter):
        rows = [r for r in _csv_rows(os.path.join(d, sub), "counter_collection.csv")
                if r["Counter_Name"] == counter and _ours(r["Kernel_Name"])]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return [float(r["Counter_Value"]) for r in rows]

    def med(v):
        v = sorted(v[1:] if len(v) > 2 else v)   # the first launch of a setting is cold
        return v[len(v) // 2] if v else float("nan")

    def chunks(vals):
        if len(vals) != n * len(settings):
            return None
        return [vals[i * n:(i + 1) * n] for i in range(len(settings))]

    tr = [r for r in _csv_rows(os.path.join(d, "trace"), "kernel_trace.csv") if _ours(r["Kernel_Name"])]
    tr.sort(key=lambda r: int(r["Dispatch_Id"]))
    dur = chunks([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in tr])
    hit, miss, rdreq = (chunks(per_dispatch("tcc", c)) for c in ("TCC_HIT_sum", "TCC_MISS_sum",
                                                                "TCC_EA0_RDREQ_sum"))
    fetch, write = chunks(per_dispatch("fetch", "FETCH_SIZE")), chunks(per_dispatch("write", "WRITE_SIZE"))
    mfma, conf = (chunks(per_dispatch("sq", c)) for c in ("SQ_VALU_MFMA_BUSY_CYCLES",
                                                        "SQ_LDS_BANK_CONFLICT"))
    cal = 256 << 20
    cf = [float(r["Counter_Value"]) for r in _csv_rows(os.path.join(d, "calib_fetch"), "counter_collection.csv")
          if r["Counter_Name"] == "FETCH_SIZE" and "copy" in r["Kernel_Name"].lower()]
    cw = [float(r["Counter_Value"]) for r in _csv_rows(os.path.join(d, "calib_write"), "counter_collection.csv")
          if r["Counter_Name"] == "WRITE_SIZE" and "copy" in r["Kernel_Name"].lower()]
    sf = cal / (med(cf) * 1024.0) if cf else float("nan")
    sw = cal / (med(cw) * 1024.0) if cw else float("nan")
    print("Copy calibration: FETCH_SIZE scale %.4f, WRITE_SIZE scale %.4f (bytes per KiB counted "
          "/ 1024)\n" % (sf, sw))
    print("| setting | median us | TFLOP/s | L2 hit % | fabric rd req (x1000) | HBM MB "
          "(alg MB) | HBM GB/s | MFMA busy / needed | LDS conflicts |")
    print("|---|---|---|---|---|---|---|---|---|")
    for i, c in enumerate(settings):
        us = med(dur[i]) if dur else float("nan")
        h = med(hit[i]) if hit else float("nan")
        m = med(miss[i]) if miss else float("nan")
        hb = (med(fetch[i]) * 1024 * sf + med(write[i]) * 1024 * sw) if (fetch and write) else float("nan")
        print("| %s | %.2f | %.1f | %.1f | %.0f | %.1f (%.1f) | %.0f | %s | %s |" % (
            c["label"], us, c["flop"] / (us * 1e-6) / 1e12, 100.0 * h / (h + m),
            (med(rdreq[i]) / 1000.0) if rdreq else float("nan"), hb / 1e6, c["alg_bytes"] / 1e6,
            hb / (us * 1e-6) / 1e9,
            ("%.3f" % (med(mfma[i]) / c["mfma_cycles"])) if mfma else "-",
            ("%.0f" % med(conf[i])) if conf else "-"))


def cold_launch(torch, fn, n=20, scrub_bytes=512 << 20):
    """Median ms of n launches of fn(), each timed alone right after a 512 MiB scrub write
    (a fill kernel over a buffer twice the size of the MALL), so that its operands come
    from HBM rather than the caches."""
    scrub = torch.empty(scrub_bytes, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()
    ms = []
    fn()
    for i in range(n):
        scrub.fill_(i & 0xff)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fn()
        e1.record(st)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    del scrub
    ms.sort()
    return ms[len(ms) // 2]


def oracle_time(orc, name, flop_per_row, nrows_total, run_rows, threads=0, budget_s=6.0):
    """The oracle on whole output rows of one workload: the largest sample of evenly spread
    rows (doubling from 1) whose pass takes under budget_s, timed once; returns a
    cpu_baseline-style record in TFLOP/s (threads: 0 = the oracle's default)."""
    import numpy as np
    prev = orc.threads()
    used = orc.threads(threads) if threads > 0 else prev
    try:
        n = 1
        while True:
            rows = np.linspace(0, nrows_total - 1, min(n, nrows_total)).astype(np.int64)
            t0 = time.perf_counter()
            run_rows(rows)
            dt = time.perf_counter() - t0
            if dt * 2.2 > budget_s or n >= nrows_total:
                break
            n *= 2
    finally:
        orc.threads(prev)
    rec = {"config": name, "cpu_baseline": {
        "value": round(flop_per_row * len(rows) / dt / 1e12, 6), "unit": "TFLOP/s",
        "cores": used, "kind": "oracle",
        "sample": "%d of %d output rows (fp64 / int64 oracle, %.2f s)" % (len(rows), nrows_total, dt)}}
    print(json.dumps(rec), flush=True)
    return rec


def all_configs(args, bst, I, gpu, torch):
    """Every configuration of the workload set, at its stated tile and at the
    faster schedules, timed like the headline (warm, graph replay of
    args.steps launches); one JSON line per (config, schedule).  Each
    configuration's fastest schedule also gets its shader clock; C4 and C5
    (whose operands exceed the L2s) also a cold figure; and the oracle is
    timed on a sample of each configuration's rows on this host (C1 and C2
    also on one thread)."""
    import numpy as np
    import oracle as orc
    out = []

    def run(name, flop, dtype, sched_kw, fn, cold=False, clock=False):
        s = bst.make_sched(**sched_kw)
        tot, per = time_launches(lambda: fn(s), args.steps, args.warmup)
        tf = flop / (per * 1e-3) / 1e12
        rec = {"config": name, "sched": {k: list(v) if isinstance(v, tuple) else v
                                         for k, v in sched_kw.items()},
               "us_per_launch": round(per * 1e3, 3), "tflops": round(tf, 2),
               "pct_of_peak": round(100.0 * tf / PEAK[dtype], 2)}
        if cold:
            cms = cold_launch(torch, lambda: fn(s))
            rec["cold_us"] = round(cms * 1e3, 3)
            rec["cold_tflops"] = round(flop / (cms * 1e-3) / 1e12, 2)
        if clock:
            clk = shader_clock(bst, lambda: fn(s))
            rec["sclk_mhz"] = clk["sclk_mhz_median"]
            rec["pct_at_measured_clock"] = round(
                100.0 * tf / (PEAK[dtype] * clk["sclk_mhz_median"] / 2400.0), 2)
        out.append(rec)
        print(json.dumps(rec), flush=True)

    w = I.workload("tails")
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    f1 = 2.0 * w["M"] * w["N"] * w["K"]
    run("C1 fp16 200x136x256", f1, "f16", dict(tile=(64, 64), offset=3, direction="zn"),
        lambda s: bst.gemm(A, B, C, sched=s), clock=True)
    for thr in (0, 1):
        oracle_time(orc, "C1 fp16 200x136x256" + (" (1 thread)" if thr else ""),
                    2.0 * w["N"] * w["K"], w["M"],
                    lambda rows: orc.gemm(orc.F16, w["A"], w["B"], tile=(64, 64), off=3,
                                          rows=rows), threads=thr)

    w = I.workload("fp16_2k")
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    f2 = 2.0 * w["M"] * w["N"] * w["K"]
    for kw in (dict(tile=(256, 128), offset=1, direction="zn", xcd_remap=1),
               dict(tile=(256, 128), offset=4, direction="zn", xcd_remap=0),
               dict(tile=(64, 64), offset=8, direction="zn", xcd_remap=1)):
        run("C2 fp16 1024x1024x2048", f2, "f16", kw, lambda s: bst.gemm(A, B, C, sched=s))
    run("C2 fp16 1024x1024x2048", f2, "f16",
        dict(tile=(64, 64), offset=8, direction="zn", xcd_remap=1, shuffle_k=1),
        lambda s: bst.gemm(A, B, C, sched=s), clock=True)
    for thr in (0, 1):
        oracle_time(orc, "C2 fp16 1024x1024x2048" + (" (1 thread)" if thr else ""),
                    2.0 * w["N"] * w["K"], w["M"],
                    lambda rows: orc.gemm(orc.F16, w["A"], w["B"], tile=(64, 64), rows=rows),
                    threads=thr)

    # matmul-add on the same workload: C = A.B + X with a seeded fp16 addend
    X = gpu(I.uniform_f16((w["M"], w["N"]), I.WORKLOAD_IDS["fp16_2k"], 7, -4.0, 4.0), "f16")
    run("C2 fp16 1024x1024x2048 matmul-add (+X)", f2, "f16",
        dict(tile=(64, 64), offset=8, direction="zn", xcd_remap=1, shuffle_k=1),
        lambda s: bst.gemm(A, B, C, sched=s, add=X))

    # padding matmul on the same workload, with operands whose rows are 2 bytes longer
    # (odd strides): repacked into the workspace, then multiplied
    Ao = torch.zeros((w["M"], w["K"] + 1), dtype=torch.float16, device="cuda")
    Bo = torch.zeros((w["K"], w["N"] + 1), dtype=torch.float16, device="cuda")
    Ao[:, :w["K"]] = A
    Bo[:, :w["N"]] = B
    Ao, Bo = Ao[:, :w["K"]], Bo[:, :w["N"]]
    run("C2 fp16 1024x1024x2048 padding matmul (odd strides)", f2, "f16",
        dict(tile=(64, 64), offset=8, direction="zn", xcd_remap=1, shuffle_k=1),
        lambda s: bst.gemm_padded(Ao, Bo, C, sched=s))

    x = I.workload("mxfp8_4k")
    Ax, Bx = gpu(x["A"], "e4m3"), gpu(x["B"], "e4m3")
    sa, sb = gpu(x["scale_a"], "u8"), gpu(x["scale_b"], "u8")
    Cx = torch.empty((x["M"], x["N"]), dtype=torch.bfloat16, device="cuda")
    f3 = 2.0 * x["M"] * x["N"] * x["K"]
    for kw in (dict(tile=(256, 256), offset=4, direction="zn", xcd_remap=0),
               dict(tile=(256, 256), offset=4, direction="zn", xcd_remap=1)):
        run("C3 MX-fp8 1024x2048x4096", f3, "e4m3", kw,
            lambda s: bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=s))
    run("C3 MX-fp8 1024x2048x4096", f3, "e4m3", dict(tile=(64, 128), offset=8, direction="zn",
                                                     xcd_remap=1),
        lambda s: bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=s))
    run("C3 MX-fp8 1024x2048x4096", f3, "e4m3", dict(tile=(64, 128), offset=8, direction="zn",
                                                     xcd_remap=1, shuffle_k=1),
        lambda s: bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=s), clock=True)
    oracle_time(orc, "C3 MX-fp8 1024x2048x4096", 2.0 * x["N"] * x["K"], x["M"],
                lambda rows: orc.gemm(orc.MXE4M3, x["A"], x["B"], scale_a=x["scale_a"],
                                      scale_b=x["scale_b"], tile=(256, 256), off=4, rows=rows))

    b = I.workload("bf16_batch")
    Ab, Bb = gpu(b["A"], "bf16"), gpu(b["B"], "bf16")
    Cb = torch.empty((b["batch"], b["M"], b["N"]), dtype=torch.bfloat16, device="cuda")
    f4 = 2.0 * b["batch"] * b["M"] * b["N"] * b["K"]
    for kw in (dict(tile=(128, 192), offset=1, direction="zn"),
               dict(tile=(128, 192), offset=1, direction="zn", xcd_remap=1),
               dict(tile=(256, 128), offset=2, direction="zn", xcd_remap=1),
               dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=2)):
        run("C4 bf16 16x512x768x1024", f4, "bf16", kw, lambda s: bst.batched_gemm(Ab, Bb, Cb, sched=s))
    # two resident workgroups per CU (the automatic choice at 128x128: 384 tiles)
    run("C4 bf16 16x512x768x1024", f4, "bf16", dict(tile=(128, 128), offset=4, direction="zn",
                                                    xcd_remap=1, path=3),
        lambda s: bst.batched_gemm(Ab, Bb, Cb, sched=s), cold=True, clock=True)
    oracle_time(orc, "C4 bf16 16x512x768x1024", 2.0 * b["N"] * b["K"], b["batch"] * b["M"],
                lambda rows: orc.gemm(orc.BF16, b["A"], b["B"], batch=b["batch"], M=b["M"],
                                      N=b["N"], K=b["K"], strideA=b["M"] * b["K"],
                                      strideB=b["K"] * b["N"], tile=(128, 192), rows=rows))

    g = I.workload("int8_groups")
    Ag, Bg = gpu(g["A"], "i8"), gpu(g["B"], "i8")
    gm = gpu(g["group_m"], "i32")
    rs, cs = gpu(g["row_scale"], "f32"), gpu(g["col_scale"], "f32")
    Cg = torch.empty((g["total_m"], g["N"]), dtype=torch.bfloat16, device="cuda")
    f5 = 2.0 * g["total_m"] * g["N"] * g["K"]
    c5 = lambda s: bst.grouped_gemm_slice_m(Ag, Bg, gm, Cg, row_scale=rs, col_scale=cs, sched=s)
    for kw in (dict(tile=(256, 256), offset=1, direction="zn"),
               dict(tile=(256, 256), offset=1, direction="zn", xcd_remap=1),
               dict(tile=(256, 128), offset=2, direction="zn", xcd_remap=1),
               dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=2),
               dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=2, preload=1),
               dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=2, dynamic=1),
               dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=3)):
        run("C5 int8 grouped 8192x4096x2048 dequant", f5, "i8", kw, c5)
    # two resident workgroups per CU (the automatic choice at 128x128) with dynamic allocation
    run("C5 int8 grouped 8192x4096x2048 dequant", f5, "i8",
        dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=3, dynamic=1), c5,
        cold=True, clock=True)
    oracle_time(orc, "C5 int8 grouped 8192x4096x2048 dequant", 2.0 * g["N"] * g["K"],
                int(g["group_m"].sum()),
                lambda rows: orc.grouped_gemm(g["group_m"], g["A"], g["B"], g["N"], g["K"],
                                              row_scale=g["row_scale"], col_scale=g["col_scale"],
                                              tile=(128, 128), off=4, rows=rows))

    k = I.workload("int8_slice_k")
    Ak, Bk, gk = gpu(k["A"], "i8"), gpu(k["B"], "i8"), gpu(k["group_k"], "i32")
    rk, ck = gpu(k["row_scale"], "f32"), gpu(k["col_scale"], "f32")
    Ck = torch.empty((k["G"], k["M"], k["N"]), dtype=torch.bfloat16, device="cuda")
    fk = 2.0 * k["M"] * k["N"] * k["total_k"]
    for kw in (dict(tile=(256, 256), offset=1, direction="zn", xcd_remap=1),
               dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, split_k=2),
               dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1)):
        run("int8 grouped slice-K 8 x (1024x2048), K 8192, dequant", fk, "i8", kw,
            lambda s: bst.grouped_gemm_slice_k(Ak, Bk, gk, Ck, row_scale=rk, col_scale=ck, sched=s),
            clock=kw["tile"] == (128, 128))
    oracle_time(orc, "int8 grouped slice-K 8 x (1024x2048), K 8192, dequant",
                2.0 * k["N"] * k["total_k"] / k["G"], k["G"] * k["M"],
                lambda rows: orc.grouped_gemm_slice_k(orc.I8, k["group_k"], k["A"], k["B"],
                                                      k["M"], k["N"], row_scale=k["row_scale"],
                                                      col_scale=k["col_scale"], tile=(128, 128),
                                                      rows=rows))
    return out


LARGE_SHAPES = [("f16", 4096, 4096, 4096), ("f16", 8192, 8192, 4096),
                ("mx", 4096, 4096, 4096), ("mx", 8192, 8192, 4096)]


def large_operands(torch, wl, M, N, K, seed):
    """Seeded synthetic operands of a large shape, made on the device: fp16
    uniform[-1, 1]; MX-fp8 e4m3 from N(0, 1) with e8m0 block scales drawn
    from 2^-4 .. 2^4 (the recipes of the 1024-size workloads, scaled up)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    if wl == "f16":
        A = (torch.rand((M, K), device="cuda", generator=g) * 2 - 1).half()
        B = (torch.rand((K, N), device="cuda", generator=g) * 2 - 1).half()
        return A, B, torch.empty((M, N), dtype=torch.float16, device="cuda"), {}
    A = torch.randn((M, K), device="cuda", generator=g).to(torch.float8_e4m3fn)
    B = torch.randn((K, N), device="cuda", generator=g).to(torch.float8_e4m3fn)
    sa = torch.randint(123, 132, (M, K // 32), device="cuda", generator=g, dtype=torch.int32)
    sb = torch.randint(123, 132, (K // 32, N), device="cuda", generator=g, dtype=torch.int32)
    kw = dict(scale_a=sa.to(torch.uint8), scale_b=sb.to(torch.uint8))
    return A, B, torch.empty((M, N), dtype=torch.bfloat16, device="cuda"), kw


def event_time(torch, fn, n):
    """ms per call of fn() over n eager calls between two events (after 5
    untimed calls and at least 0.1 s of warm-up work)."""
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.1:
        fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def large(args, bst, torch):
    """Large shapes at the 256x256 tile (Zn, offset 4, XCD remap), beside the
    library GEMMs torch calls on the same device (hipBLASLt: fp16 with B
    row-major as here, and with B stored transposed; MX-fp8 through
    torch._scaled_mm with e8m0 block scales, B stored transposed)."""
    for i, (wl, M, N, K) in enumerate(LARGE_SHAPES):
        A, B, C, kw = large_operands(torch, wl, M, N, K, 1000 + i)
        flop = 2.0 * M * N * K
        peak = PEAK["f16" if wl == "f16" else "e4m3"]
        s = bst.make_sched(tile=(256, 256), offset=4, direction="zn", xcd_remap=1)
        runs = [("bst 256x256", lambda: bst.gemm(A, B, C, sched=s, **kw))]
        if wl == "f16":
            Bt = B.t().contiguous().t()
            runs += [("torch.matmul (B row-major)", lambda: torch.matmul(A, B)),
                     ("torch.matmul (B transposed)", lambda: torch.matmul(A, Bt))]
        else:
            Bt = B.t().contiguous().t()
            e8 = torch.float8_e8m0fnu
            sa = kw["scale_a"].view(e8)
            sbt = kw["scale_b"].t().contiguous().view(e8)
            runs += [("torch._scaled_mm (B transposed)",
                      lambda: torch._scaled_mm(A, Bt, scale_a=sa, scale_b=sbt,
                                               out_dtype=torch.bfloat16))]
        for name, fn in runs:
            try:
                ms = event_time(torch, fn, 20)
            except Exception as ex:  # a library path this torch build lacks
                print(json.dumps({"shape": [M, N, K], "dtype": wl, "impl": name,
                                  "error": repr(ex)[:200]}), flush=True)
                continue
            tf = flop / (ms * 1e-3) / 1e12
            rec = {"shape": [M, N, K], "dtype": wl, "impl": name,
                   "us_per_launch": round(ms * 1e3, 2), "tflops": round(tf, 1),
                   "pct_of_peak": round(100.0 * tf / peak, 1)}
            if name.startswith("bst"):
                # the production kernel's own clock record (bst_set_clock_record)
                clk = shader_clock(bst, fn)
                rec["sclk_mhz"] = clk["sclk_mhz_median"]
                rec["pct_at_measured_clock"] = round(
                    100.0 * tf / (peak * clk["sclk_mhz_median"] / 2400.0), 1)
            print(json.dumps(rec), flush=True)
        del A, B, C, kw


def clock(args, torch, np, I, gpu):
    """Shader clock during each workload, from the cycle-accounting build:
    every workgroup records the 100 MHz reference counter at its start and
    end and the shader cycles in between (30 untimed launches first, so the
    clock has settled)."""
    import ctypes
    from block_swizzle_tile_amd import _lib as L
    from block_swizzle_tile_amd import build as bld
    if not os.path.exists(bld.TRACE_LIB):
        sys.exit("bench.py --clock needs %s (python -m block_swizzle_tile_amd.build --trace)"
                 % bld.TRACE_LIB)
    L.LIB_PATH = bld.TRACE_LIB
    import block_swizzle_tile_amd as bst
    lib = L.lib()
    lib.bst_debug_set_trace.argtypes = [ctypes.c_void_p]
    lib.bst_debug_set_trace.restype = None
    tr = torch.zeros(128 + 4 * 256, dtype=torch.int64, device="cuda")

    def one(name, fn):
        lib.bst_debug_set_trace(None)
        for _ in range(30):
            fn()
        torch.cuda.synchronize()
        tr.zero_()
        lib.bst_debug_set_trace(ctypes.c_void_p(tr.data_ptr()))
        fn()
        torch.cuda.synchronize()
        lib.bst_debug_set_trace(None)
        t = tr.cpu()[128:].view(256, 4)
        t = t[t[:, 3] == 1].double()
        mhz = t[:, 2] / ((t[:, 1] - t[:, 0]) / 100.0)
        life = (t[:, 1] - t[:, 0]) / 100.0
        print(json.dumps({"workload": name, "workgroups": int(t.shape[0]),
                          "shader_mhz_median": round(float(mhz.median()), 0),
                          "shader_mhz_min": round(float(mhz.min()), 0),
                          "shader_mhz_max": round(float(mhz.max()), 0),
                          "workgroup_life_us_median": round(float(life.median()), 2)}),
              flush=True)

    w = I.workload("fp16_2k")
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    s = bst.make_sched(tile=(64, 64), offset=8, direction="zn", xcd_remap=1)
    one("fp16 1024x1024x2048 64x64", lambda: bst.gemm(A, B, C, sched=s))
    x = I.workload("mxfp8_4k")
    Ax, Bx = gpu(x["A"], "e4m3"), gpu(x["B"], "e4m3")
    sa, sb = gpu(x["scale_a"], "u8"), gpu(x["scale_b"], "u8")
    Cx = torch.empty((x["M"], x["N"]), dtype=torch.bfloat16, device="cuda")
    s = bst.make_sched(tile=(64, 128), offset=8, direction="zn", xcd_remap=1)
    one("MX-fp8 1024x2048x4096 64x128", lambda: bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=s))
    for i, (wl, M, N, K) in enumerate(LARGE_SHAPES):
        A, B, C, kw = large_operands(torch, wl, M, N, K, 1000 + i)
        s = bst.make_sched(tile=(256, 256), offset=4, direction="zn", xcd_remap=1)
        one("%s %dx%dx%d 256x256" % ("fp16" if wl == "f16" else "MX-fp8", M, N, K),
            lambda: bst.gemm(A, B, C, sched=s, **kw))
        del A, B, C, kw


def phases(args, torch, np, I, gpu):
    """Where a work unit's shader cycles go, from the cycle-accounting build (python -m
    block_swizzle_tile_amd.build --trace): workgroup 0's waves record, per unit, the set-up
    (decode, lane offsets; the first unit from the kernel's start), the K loop (its prologue,
    the waits at the stage barriers and the step bodies), the split-K fix-up and the
    epilogue (stores issued, then complete).  Averages over the waves and the units of 5
    launches (after 20 untimed ones), one JSON line per workload.  The build runs about 20%
    slower than the production one; the split between phases is what it is for."""
    import ctypes
    from block_swizzle_tile_amd import _lib as L
    from block_swizzle_tile_amd import build as bld
    if not os.path.exists(bld.TRACE_LIB):
        sys.exit("bench.py --phases needs %s (python -m block_swizzle_tile_amd.build --trace)"
                 % bld.TRACE_LIB)
    L.LIB_PATH = bld.TRACE_LIB
    import block_swizzle_tile_amd as bst
    lib = L.lib()
    lib.bst_debug_set_trace.argtypes = [ctypes.c_void_p]
    lib.bst_debug_set_trace.restype = None
    tr = torch.zeros(128 + 4 * 256, dtype=torch.int64, device="cuda")

    def one(name, fn, waves=4):
        lib.bst_debug_set_trace(None)
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        tr.zero_()
        lib.bst_debug_set_trace(ctypes.c_void_p(tr.data_ptr()))
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        lib.bst_debug_set_trace(None)
        t = tr.cpu().numpy().astype(np.float64)
        loop = t[:32].reshape(8, 4)[:waves]       # wait, body, prologue, total
        task = t[32:64].reshape(8, 4)[:waves]     # set-up, K loop, fix-up + epilogue, units
        epi = t[64:96].reshape(8, 4)[:waves]      # fix-up, stores issued, stores complete
        units = task[:, 3].mean()
        per = lambda v: round(float(v.mean() / units), 0)
        print(json.dumps({"workload": name, "units_per_launch_wg0": round(units / 5, 2),
                          "setup": per(task[:, 0]), "k_loop": per(task[:, 1]),
                          "k_loop_prologue": per(loop[:, 2]), "k_loop_waits": per(loop[:, 0]),
                          "k_loop_bodies": per(loop[:, 1]), "fixup": per(epi[:, 0]),
                          "stores_issued": per(epi[:, 1]), "stores_complete": per(epi[:, 2]),
                          "unit": "shader cycles per work unit (workgroup 0, wave mean)"}),
              flush=True)

    w = I.workload("fp16_2k")
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    s = bst.make_sched(tile=(64, 64), offset=8, direction="zn", xcd_remap=1, shuffle_k=1)
    one("C2 fp16 1024x1024x2048 64x64", lambda: bst.gemm(A, B, C, sched=s))
    # larger tiles cut each unit's operand bytes; split-K brings the unit count back to the
    # CU count, at the price of the partial tiles' fix-up
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    for tile, split in [((128, 128), 4), ((128, 128), 1), ((64, 64), 2), ((256, 128), 8)]:
        ss = bst.make_sched(tile=tile, offset=4, direction="zn", xcd_remap=1, split_k=split)
        one("C2 fp16 1024x1024x2048 %dx%d split %d" % (tile + (split,)),
            lambda: bst.gemm(A, B, C, sched=ss, workspace=ws))
    x = I.workload("mxfp8_4k")
    Ax, Bx = gpu(x["A"], "e4m3"), gpu(x["B"], "e4m3")
    sa, sb = gpu(x["scale_a"], "u8"), gpu(x["scale_b"], "u8")
    Cx = torch.empty((x["M"], x["N"]), dtype=torch.bfloat16, device="cuda")
    sx = bst.make_sched(tile=(64, 128), offset=8, direction="zn", xcd_remap=1)
    one("C3 MX-fp8 1024x2048x4096 64x128", lambda: bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb,
                                                            sched=sx))
    b = I.workload("bf16_batch")
    Ab, Bb = gpu(b["A"], "bf16"), gpu(b["B"], "bf16")
    Cb = torch.empty((b["batch"], b["M"], b["N"]), dtype=torch.bfloat16, device="cuda")
    sbt = bst.make_sched(tile=(128, 192), offset=1, direction="zn", xcd_remap=1)
    one("C4 bf16 16x512x768x1024 128x192", lambda: bst.batched_gemm(Ab, Bb, Cb, sched=sbt))
    sb3 = bst.make_sched(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=3)
    one("C4 bf16 16x512x768x1024 128x128 two workgroups per CU",
        lambda: bst.batched_gemm(Ab, Bb, Cb, sched=sb3))
    g = I.workload("int8_groups")
    Ag, Bg, gm = gpu(g["A"], "i8"), gpu(g["B"], "i8"), gpu(g["group_m"], "i32")
    rs, cs = gpu(g["row_scale"], "f32"), gpu(g["col_scale"], "f32")
    Cg = torch.empty((g["total_m"], g["N"]), dtype=torch.bfloat16, device="cuda")
    for extra in ({}, {"preload": 1}, {"dynamic": 1}):
        sg = bst.make_sched(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=2,
                            **extra)
        one("C5 int8 grouped 128x128 %s" % (" ".join(extra) or "static"),
            lambda: bst.grouped_gemm_slice_m(Ag, Bg, gm, Cg, row_scale=rs, col_scale=cs, sched=sg))
    sg = bst.make_sched(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=3)
    one("C5 int8 grouped 128x128 two workgroups per CU",
        lambda: bst.grouped_gemm_slice_m(Ag, Bg, gm, Cg, row_scale=rs, col_scale=cs, sched=sg))
    sg = bst.make_sched(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=2)
    Craw = torch.empty((g["total_m"], g["N"]), dtype=torch.int32, device="cuda")
    one("C5 int8 grouped 128x128 raw int32 (no dequant)",
        lambda: bst.grouped_gemm_slice_m(Ag, Bg, gm, Craw, sched=sg))
    for wl, M, N, K in LARGE_SHAPES[1::2]:
        Al, Bl, Cl, kw = large_operands(torch, wl, M, N, K, 1001)
        sl = bst.make_sched(tile=(256, 256), offset=4, direction="zn", xcd_remap=1)
        one("%s %dx%dx%d 256x256" % ("fp16" if wl == "f16" else "MX-fp8", M, N, K),
            lambda: bst.gemm(Al, Bl, Cl, sched=sl, **kw), waves=8)


def wg_times(args, torch, np, I, gpu):
    """Per-workgroup life of one launch (after 0.1 s of warm-up launches), from the production
    kernels' clock record (bst_set_clock_record: the 100 MHz reference counter at each
    workgroup's start and end): the spread of the end times, their maximum per XCD (workgroup w
    runs on XCD w mod 8), and the time by which all but the last 1% / 10% had ended.  One JSON
    line per (workload, schedule).  It shows how evenly a schedule spreads the units."""
    import block_swizzle_tile_amd as bst

    def one(name, kind, ab, count, M, N, K, sk, fn):
        s = bst.make_sched(**sk)
        eff = bst.effective_sched(kind, ab, count, M, N, K, s)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.1:
            fn(s)
            torch.cuda.synchronize()
        nwg = 1024
        buf = torch.zeros(4 * nwg, dtype=torch.int64, device="cuda")
        bst.clock_record(buf, nwg)
        try:
            fn(s)
            torch.cuda.synchronize()
        finally:
            bst.clock_record()
        t = buf.cpu().view(nwg, 4).numpy()
        idx = np.nonzero(t[:, 3] == 1)[0]
        st, en = t[idx, 0].astype(np.float64), t[idx, 1].astype(np.float64)
        base = st.min()
        st, en = (st - base) / 100.0, (en - base) / 100.0   # microseconds
        rec = {"workload": name, "sched": {k: list(v) if isinstance(v, tuple) else v
                                           for k, v in sk.items()},
               "path": eff.path, "workgroups": int(len(idx)),
               "last_start_us": round(float(st.max()), 2),
               "end_us": {"min": round(float(en.min()), 2), "median": round(float(np.median(en)), 2),
                          "p90": round(float(np.percentile(en, 90)), 2),
                          "p99": round(float(np.percentile(en, 99)), 2),
                          "max": round(float(en.max()), 2)},
               "end_max_by_xcd_us": [round(float(en[idx % 8 == x].max()), 1) for x in range(8)]}
        print(json.dumps(rec), flush=True)

    g = I.workload("int8_groups")
    Ag, Bg, gm = gpu(g["A"], "i8"), gpu(g["B"], "i8"), gpu(g["group_m"], "i32")
    rs, cs = gpu(g["row_scale"], "f32"), gpu(g["col_scale"], "f32")
    Cg = torch.empty((g["total_m"], g["N"]), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    c5 = lambda s: bst.grouped_gemm_slice_m(Ag, Bg, gm, Cg, row_scale=rs, col_scale=cs, sched=s,
                                            workspace=ws)
    base = dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1)
    for extra in (dict(path=2), dict(path=2, dynamic=1), dict(path=3), dict(path=3, dynamic=1)):
        one("C5 int8 grouped 8192x4096x2048 dequant", 1, bst.I8, g["G"], g["total_m"], g["N"],
            g["K"], dict(base, **extra), c5)
    k = I.workload("int8_slice_k")
    Ak, Bk, gk = gpu(k["A"], "i8"), gpu(k["B"], "i8"), gpu(k["group_k"], "i32")
    rk, ck = gpu(k["row_scale"], "f32"), gpu(k["col_scale"], "f32")
    Ck = torch.empty((k["G"], k["M"], k["N"]), dtype=torch.bfloat16, device="cuda")
    sk = lambda s: bst.grouped_gemm_slice_k(Ak, Bk, gk, Ck, row_scale=rk, col_scale=ck, sched=s,
                                            workspace=ws)
    for extra in ({}, dict(dynamic=1), dict(xcd_remap=0)):
        one("int8 grouped slice-K 8 x (1024x2048), K 8192, dequant", 3, bst.I8, k["G"], k["M"],
            k["N"], k["total_k"], dict(base, **extra), sk)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the GEMM would shard by tiles / batches / groups with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        traffic_summary(args.traffic_from, CALIB_BYTES)
        return
    if args.summarize:
        summarize(args.summarize)
        return
    import numpy as np
    import torch

    if args.calib_copy:
        n = CALIB_BYTES
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 5}), flush=True)
        return

    from block_swizzle_tile_amd import inputs as I

    def gpu(arr, kind):
        a = np.ascontiguousarray(arr)
        if kind == "f16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
        if kind == "e4m3":
            return torch.from_numpy(a.view(np.uint8)).cuda().view(torch.float8_e4m3fn)
        if kind == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    if args.clock:
        clock(args, torch, np, I, gpu)
        return
    if args.wg_times:
        wg_times(args, torch, np, I, gpu)
        return
    if args.phases:
        phases(args, torch, np, I, gpu)
        return
    import block_swizzle_tile_amd as bst
    if args.large:
        large(args, bst, torch)
        return
    if args.all_configs:
        all_configs(args, bst, I, gpu, torch)
        return
    if args.l2_sweep:
        l2_sweep(args, bst, I, gpu, torch)
        return
    if args.sweep_configs:
        sweep_configs(args, bst, I, gpu, torch)
        return

    # ---------------------------------------------------------- fp16 2k --
    w = I.workload("fp16_2k")
    M, N, K = w["M"], w["N"], w["K"]
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    tm, tn = map(int, args.tile.split("x"))
    sched = bst.make_sched(tile=(tm, tn), offset=args.offset, direction=args.direction,
                           split_k=args.split, xcd_remap=args.remap, grid=args.grid,
                           shuffle_k=args.shuffle_k)
    eff = bst.effective_sched(0, bst.F16, 1, M, N, K, sched)
    nb = bst.workspace_bytes(0, bst.F16, 1, M, N, K, sched)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")

    def step():
        bst.gemm(A, B, C, sched=sched, workspace=ws)

    total_ms, mean_ms = time_launches(step, args.steps, args.warmup)
    flop = 2.0 * M * N * K
    ms_per_step = total_ms / args.steps
    value = flop * args.steps / (total_ms * 1e-3) / 1e12
    achieved = flop / (mean_ms * 1e-3) / 1e12

    # the same launch timed alone (median of 50), the shader clock it runs at, and the tile
    # the workload's definition names (256 x 128, SwizzleOffset 4, Zn)
    med_ms = median_launch(bst, step)
    clk = shader_clock(bst, step)
    named = bst.make_sched(tile=(256, 128), offset=4, direction="zn")
    named_per = time_launches(lambda: bst.gemm(A, B, C, sched=named), args.steps, args.warmup)[1]
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
            "xcd_remap": eff.xcd_remap, "grid": eff.grid, "shuffle_k": eff.shuffle_k,
        },
        "pct_of_peak": round(100.0 * value / PEAK["f16"], 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK["f16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK["f16"], 4),
                     "traffic": traffic, "kernel_ms_mean": round(mean_ms, 5),
                     "flop_per_launch": flop,
                     "timing": "one HIP-graph replay of the timed launches between two events",
                     "sclk_mhz": clk["sclk_mhz_median"],
                     "frac_at_measured_clock": round(
                         achieved / (PEAK["f16"] * clk["sclk_mhz_median"] / 2400.0), 4)},
        "median_of_50": {"us": round(med_ms * 1e3, 3),
                         "tflops": round(flop / (med_ms * 1e-3) / 1e12, 2),
                         "timing": "median over 50 launches of the span from the first "
                                   "workgroup's start to the last one's end (device clock record)"},
        "clock": clk,
        "named_tile": {"tile": [256, 128], "swizzle": {"offset": 4, "direction": "zn"},
                       "us": round(named_per * 1e3, 3),
                       "tflops": round(flop / (named_per * 1e-3) / 1e12, 2),
                       "pct_of_peak": round(100.0 * flop / (named_per * 1e-3) / 1e12 / PEAK["f16"], 2),
                       "note": "32 tiles for 256 CUs: at most 12.5% of the chip busy"},
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
                            split_k=args.mx_split, xcd_remap=args.remap,
                            shuffle_k=args.mx_shuffle_k)
        effx = bst.effective_sched(0, bst.MXE4M3, 1, Mx, Nx, Kx, sx)
        nbx = bst.workspace_bytes(0, bst.MXE4M3, 1, Mx, Nx, Kx, sx)
        wsx = torch.zeros(max(nbx, 16), dtype=torch.uint8, device="cuda")

        def stepx():
            bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=sx, workspace=wsx)

        tot, mean_x = time_launches(stepx, args.steps, args.warmup)
        fx = 2.0 * Mx * Nx * Kx
        vx = fx * args.steps / (tot * 1e-3) / 1e12
        medx = median_launch(bst, stepx)
        clkx = shader_clock(bst, stepx)
        namedx = bst.make_sched(tile=(256, 256), offset=4, direction="zn")
        named_x = time_launches(lambda: bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=namedx),
                                args.steps, args.warmup)[1]
        out["mxfp8"] = {
            "workload": "MX-fp8 GEMM M=1024 N=2048 K=4096, e4m3 + e8m0 per-32 scales, bf16 out",
            "value": round(vx, 2), "unit": "TFLOP/s",
            "pct_of_peak": round(100.0 * vx / PEAK["e4m3"], 2),
            "ms_per_step": round(tot / args.steps, 5),
            "kernel_ms_mean": round(mean_x, 5),
            "achieved": round(fx / (mean_x * 1e-3) / 1e12, 2), "peak": PEAK["e4m3"],
            "frac": round(fx / (mean_x * 1e-3) / 1e12 / PEAK["e4m3"], 4),
            "frac_at_measured_clock": round(fx / (mean_x * 1e-3) / 1e12 /
                                            (PEAK["e4m3"] * clkx["sclk_mhz_median"] / 2400.0), 4),
            "tile": [effx.tile_m, effx.tile_n, effx.tile_k], "split_k": effx.split_k, "shuffle_k": effx.shuffle_k,
            "median_of_50": {"us": round(medx * 1e3, 3),
                             "tflops": round(fx / (medx * 1e-3) / 1e12, 2)},
            "clock": clkx,
            "named_tile": {"tile": [256, 256], "swizzle": {"offset": 4, "direction": "zn"},
                           "us": round(named_x * 1e3, 3),
                           "tflops": round(fx / (named_x * 1e-3) / 1e12, 2),
                           "pct_of_peak": round(100.0 * fx / (named_x * 1e-3) / 1e12 / PEAK["e4m3"], 2)},
        }

    # ---------------------------------------------------- CPU baseline --
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        nrows = args.cpu_rows or M
        rows = None if nrows >= M else np.linspace(0, M - 1, nrows).astype(np.int64)
        # repeat the sample until it is about 10 s of CPU work (bounded at 15 repeats)
        reps, t = 0, time.perf_counter()
        while True:
            ref, den = oracle.gemm(oracle.F16, w["A"], w["B"], tile=(tm, tn), rows=rows)
            reps += 1
            dt = time.perf_counter() - t
            if dt >= 10.0 or reps >= 15:
                break
        omp = oracle.threads()
        # the oracle's result also checks the last timed launch's output
        got = C.cpu().view(torch.int16).numpy().view(np.uint16)
        got = oracle.decode("f16", got if rows is None else got[rows])
        err, _ = oracle.compare(got, ref, den)
        if not err <= 2.0 ** -9:
            print("parity check failed: %g" % err, file=sys.stderr)
            sys.exit(1)
        out["cpu_baseline"] = {
            "value": round(2.0 * nrows * N * K * reps / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": min(omp, cores), "host_cores_visible": cores, "kind": "oracle",
            "sample": "%d x %d of %d output rows of the fp16 1024x1024x2048 workload (fp64 "
                      "oracle, %.2f s)" % (reps, nrows, M, dt),
            "parity_max_norm_err": err,
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
