"""Build the gfx950 HIP library libbst.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["bst.hip", "inst_f16.hip", "inst_bf16.hip", "inst_i8.hip", "inst_fp8.hip",
           "inst_mxfp8.hip", "inst_slicek.hip"]
HEADERS = ["bst_device.hpp", "bst_kernel_dma.hpp", "bst_instances.hpp"]
DEPS = ([os.path.join(CSRC, f) for f in SOURCES + HEADERS] +
        [os.path.join(ROOT, "include", "bst.h")])
LIB = os.path.join(PKG, "libbst.so")
# The same kernels with cycle accounting (-DBST_TRACE): per-wave K-loop and
# task phase cycles of workgroup 0 and a per-workgroup shader-clock record,
# written to a device buffer set with bst_debug_set_trace.  For measurement
# only; bench.py --clock loads it.
TRACE_LIB = os.path.join(PKG, "libbst_trace.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-pass-failed",
]


def build(force: bool = True, verbose: bool = False, trace: bool = False) -> str:
    """Compile libbst.so (always when force, else only when a source is newer);
    trace=True builds libbst_trace.so instead."""
    lib = TRACE_LIB if trace else LIB
    if not force and os.path.exists(lib) and all(
            os.path.getmtime(lib) >= os.path.getmtime(d) for d in DEPS):
        return lib
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build_trace" if trace else "_build")
    flags = HIPCC_FLAGS + (["-DBST_TRACE"] if trace else [])
    os.makedirs(objdir, exist_ok=True)
    procs = []
    for src in SOURCES:     # one process per translation unit, in parallel
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = ([hipcc] + flags + ["-I", os.path.join(ROOT, "include"), "-c",
                                  os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    objs, failed = [], False
    for obj, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out)
            failed = True
        objs.append(obj)
    if failed:
        raise RuntimeError("hipcc failed building " + os.path.basename(lib))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking %s failed" % os.path.basename(lib))
    os.replace(tmp, lib)
    return lib

if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv[1:]))
