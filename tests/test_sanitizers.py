"""CPU runs of the native code under AddressSanitizer + UndefinedBehaviorSanitizer.

Three builds, each with -fsanitize=address,undefined and no recovery (the
first report aborts the run):
  * oracle.c (gcc), driven by the oracle's own pin tests;
  * the library's host code (bst.hip: argument validation, planning,
    workspace layout; the host sanitizer flags are passed with -Xarch_host, so
    the gfx950 code is built as usual), linked with the instance objects of
    the normal build and driven by the C-ABI tests, which need no GPU;
  * the LDS-DMA addressing checker (tests/native/check_dma_bounds.hip, host
    only), which runs the kernels' scheduler and addressing code on the CPU.
The sanitizer runtime is preloaded into the child process; a report fails the
test with its text."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CSRC = os.path.join(ROOT, "block_swizzle_tile_amd", "csrc")
OBJ = os.path.join(ROOT, "block_swizzle_tile_amd", "_build")
SAN_OPTS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]


def _env(tmp, preload, **extra):
    env = dict(os.environ)
    env.update(LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:log_path=%s/asan" % tmp,
               UBSAN_OPTIONS="print_stacktrace=1:log_path=%s/ubsan" % tmp, **extra)
    return env


def _reports(tmp):
    text = ""
    for f in sorted(glob.glob(os.path.join(tmp, "asan*")) + glob.glob(os.path.join(tmp, "ubsan*"))):
        text += open(f).read()[:4000]
    return text


def _clang_asan_runtime():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no clang ASan runtime under /opt/rocm/llvm")
    return rt[-1]


def test_oracle_under_sanitizers(tmp_path):
    tmp = str(tmp_path)
    lib = os.path.join(tmp, "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-fopenmp", "-shared", "-fPIC",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
                           "-o", lib, "-lm"])
    libasan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + tests,
                       cwd=ROOT, env=_env(tmp, libasan, ORACLE_LIB=lib), capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and " passed" in r.stdout, (r.stdout[-2000:], _reports(tmp))
    assert not _reports(tmp), _reports(tmp)


def test_host_abi_under_sanitizers(tmp_path):
    objs = [os.path.join(OBJ, f) for f in ("inst_f16.o", "inst_bf16.o", "inst_i8.o", "inst_fp8.o",
                                           "inst_mxfp8.o", "inst_slicek.o")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the instance objects of the normal build are missing "
                    "(python -m block_swizzle_tile_amd.build)")
    tmp = str(tmp_path)
    obj, lib = os.path.join(tmp, "bst_san.o"), os.path.join(tmp, "libbst_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-Wno-pass-failed"] + SAN_OPTS +
                          ["-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, "bst.hip"),
                           "-o", obj], stderr=subprocess.DEVNULL)
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", obj] + objs +
                          ["-o", lib])
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT,
                       env=_env(tmp, _clang_asan_runtime(), BST_LIB=lib), capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and " passed" in r.stdout, (r.stdout[-2000:], _reports(tmp))
    assert not _reports(tmp), _reports(tmp)


def test_dma_addressing_under_sanitizers(tmp_path):
    tmp = str(tmp_path)
    exe = os.path.join(tmp, "check_dma_bounds_san")
    subprocess.check_call([HIPCC, "--cuda-host-only", "-std=c++17", "-O1", "-g"] + SAN_OPTS +
                          ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           os.path.join(ROOT, "tests", "native", "check_dma_bounds.hip"),
                           "-o", exe], stderr=subprocess.DEVNULL)
    env = _env(tmp, "")
    env.pop("LD_PRELOAD")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "ALL OK" in r.stdout, (r.stdout[-2000:], _reports(tmp))
    assert not _reports(tmp), _reports(tmp)
