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
    p.add_argument("--mx-shuffle-k", type=int, default=0,
                   help="MX-fp8 workload: ShuffleK (about 3%% slower there, so off)")
    p.add_argument("--mx-tile", default="64x128")
    p.add_argument("--mx-split", type=int, default=1)
    p.add_argument("--no-mx", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = auto)")
    p.add_argument("--l2-sweep", action="store_true",
                   help="only run the fp16 workload under every swizzle setting (Zn / Nz offsets "
                        "1, 2, 4, 8 and RASTER, XCD remap off / on) at the 256x128 and the 64x64 "
                        "tile, --steps launches each, for per-setting rocprofv3 counters")
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


def l2_sweep(args, bst, I, gpu, torch):
    """Every swizzle setting on the fp16 1024x1024x2048 workload, in a fixed
    order printed first as JSON (one kernel launch per step, no graph), so a
    rocprofv3 run can attribute its per-dispatch counters to settings."""
    w = I.workload("fp16_2k")
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    cfgs = []
    for tile in ((256, 128), (64, 64)):
        for remap in (0, 1):
            for d in ("zn", "nz"):
                for off in (1, 2, 4, 8):
                    cfgs.append({"tile": tile, "direction": d, "offset": off, "xcd_remap": remap})
            cfgs.append({"tile": tile, "direction": "raster", "offset": 1, "xcd_remap": remap})
    print(json.dumps({"l2_sweep": cfgs, "launches_each": args.steps}), flush=True)
    for c in cfgs:
        s = bst.make_sched(tile=c["tile"], offset=c["offset"], direction=c["direction"],
                           split_k=1, xcd_remap=c["xcd_remap"])
        for _ in range(args.steps):
            bst.gemm(A, B, C, sched=s)
        torch.cuda.synchronize()


def all_configs(args, bst, I, gpu, torch):
    """Every configuration of the workload set, at its stated tile and at the
    faster schedules, timed like the headline (warm, graph replay of
    args.steps launches); one JSON line per (config, schedule)."""
    out = []

    def run(name, flop, dtype, sched_kw, fn):
        s = bst.make_sched(**sched_kw)
        tot, per = time_launches(lambda: fn(s), args.steps, args.warmup)
        tf = flop / (per * 1e-3) / 1e12
        rec = {"config": name, "sched": {k: list(v) if isinstance(v, tuple) else v
                                         for k, v in sched_kw.items()},
               "us_per_launch": round(per * 1e3, 3), "tflops": round(tf, 2),
               "pct_of_peak": round(100.0 * tf / PEAK[dtype], 2)}
        out.append(rec)
        print(json.dumps(rec), flush=True)

    w = I.workload("tails")
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    f1 = 2.0 * w["M"] * w["N"] * w["K"]
    run("C1 fp16 200x136x256", f1, "f16", dict(tile=(64, 64), offset=3, direction="zn"),
        lambda s: bst.gemm(A, B, C, sched=s))

    w = I.workload("fp16_2k")
    A, B = gpu(w["A"], "f16"), gpu(w["B"], "f16")
    C = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    f2 = 2.0 * w["M"] * w["N"] * w["K"]
    for kw in (dict(tile=(256, 128), offset=1, direction="zn", xcd_remap=1),
               dict(tile=(256, 128), offset=4, direction="zn", xcd_remap=0),
               dict(tile=(64, 64), offset=8, direction="zn", xcd_remap=1),
               dict(tile=(64, 64), offset=8, direction="zn", xcd_remap=1, shuffle_k=1)):
        run("C2 fp16 1024x1024x2048", f2, "f16", kw, lambda s: bst.gemm(A, B, C, sched=s))

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
               dict(tile=(256, 256), offset=4, direction="zn", xcd_remap=1),
               dict(tile=(64, 128), offset=8, direction="zn", xcd_remap=1)):
        run("C3 MX-fp8 1024x2048x4096", f3, "e4m3", kw,
            lambda s: bst.gemm(Ax, Bx, Cx, scale_a=sa, scale_b=sb, sched=s))

    b = I.workload("bf16_batch")
    Ab, Bb = gpu(b["A"], "bf16"), gpu(b["B"], "bf16")
    Cb = torch.empty((b["batch"], b["M"], b["N"]), dtype=torch.bfloat16, device="cuda")
    f4 = 2.0 * b["batch"] * b["M"] * b["N"] * b["K"]
    for kw in (dict(tile=(128, 192), offset=1, direction="zn"),
               dict(tile=(128, 192), offset=1, direction="zn", xcd_remap=1),
               dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1),
               dict(tile=(256, 128), offset=2, direction="zn", xcd_remap=1)):
        run("C4 bf16 16x512x768x1024", f4, "bf16", kw, lambda s: bst.batched_gemm(Ab, Bb, Cb, sched=s))

    g = I.workload("int8_groups")
    Ag, Bg = gpu(g["A"], "i8"), gpu(g["B"], "i8")
    gm = gpu(g["group_m"], "i32")
    rs, cs = gpu(g["row_scale"], "f32"), gpu(g["col_scale"], "f32")
    Cg = torch.empty((g["total_m"], g["N"]), dtype=torch.bfloat16, device="cuda")
    f5 = 2.0 * g["total_m"] * g["N"] * g["K"]
    for kw in (dict(tile=(256, 256), offset=1, direction="zn"),
               dict(tile=(256, 256), offset=1, direction="zn", xcd_remap=1),
               dict(tile=(256, 128), offset=2, direction="zn", xcd_remap=1),
               dict(tile=(128, 128), offset=4, direction="zn", xcd_remap=1)):
        run("C5 int8 grouped 8192x4096x2048 dequant", f5, "i8", kw,
            lambda s: bst.grouped_gemm_slice_m(Ag, Bg, gm, Cg, row_scale=rs, col_scale=cs,
                                                sched=s))
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
            print(json.dumps({"shape": [M, N, K], "dtype": wl, "impl": name,
                              "us_per_launch": round(ms * 1e3, 2), "tflops": round(tf, 1),
                              "pct_of_peak": round(100.0 * tf / peak, 1)}), flush=True)
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


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the GEMM would shard by tiles / batches / groups with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        traffic_summary(args.traffic_from, CALIB_BYTES)
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
                     "timing": "one HIP-graph replay of the timed launches between two events"},
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
        out["mxfp8"] = {
            "workload": "MX-fp8 GEMM M=1024 N=2048 K=4096, e4m3 + e8m0 per-32 scales, bf16 out",
            "value": round(vx, 2), "unit": "TFLOP/s",
            "pct_of_peak": round(100.0 * vx / PEAK["e4m3"], 2),
            "ms_per_step": round(tot / args.steps, 5),
            "kernel_ms_mean": round(mean_x, 5),
            "achieved": round(fx / (mean_x * 1e-3) / 1e12, 2), "peak": PEAK["e4m3"],
            "tile": [effx.tile_m, effx.tile_n, effx.tile_k], "split_k": effx.split_k, "shuffle_k": effx.shuffle_k,
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
        omp = int(os.environ.get("OMP_NUM_THREADS", cores))
        # the oracle's result also checks the last timed launch's output
        got = C.cpu().view(torch.int16).numpy().view(np.uint16)
        got = oracle.decode("f16", got if rows is None else got[rows])
        err, _ = oracle.compare(got, ref, den)
        if not err <= 2.0 ** -9:
            print("parity check failed: %g" % err, file=sys.stderr)
            sys.exit(1)
        out["cpu_baseline"] = {
            "value": round(2.0 * nrows * N * K * reps / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": min(omp, cores), "kind": "oracle",
            "sample": "%d x %d of %d output rows of the fp16 1024x1024x2048 workload (fp64 "
                      "oracle, %.2f s)" % (reps, nrows, M, dt),
            "parity_max_norm_err": err,
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
