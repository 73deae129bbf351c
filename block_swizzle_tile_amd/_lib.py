"""ctypes loader for libbst.so (the C ABI of include/bst.h).

There is no fallback: if the library is missing or fails to load, every call
raises.  Build it with ``python -m block_swizzle_tile_amd.build`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# BST_LIB selects another build of the same library (the sanitizer build of the
# CPU tests); there is no other library and no fallback
LIB_PATH = os.environ.get("BST_LIB") or os.path.join(PKG, "libbst.so")

# bst_status
OK, E_INVAL, E_UNSUPPORTED, E_ALIGN, E_WORKSPACE, E_HIP = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "BST_OK", -1: "BST_E_INVAL", -2: "BST_E_UNSUPPORTED", -3: "BST_E_ALIGN",
                -4: "BST_E_WORKSPACE", -5: "BST_E_HIP"}
# bst_dtype
F16, BF16, E4M3, MXE4M3, I8, I32, F32 = 1, 2, 3, 4, 5, 6, 7

EXPORTS = ["bst_gemm", "bst_gemm_noalloc", "bst_gemm_add", "bst_gemm_padded", "bst_batched_gemm",
           "bst_grouped_gemm_slice_m", "bst_grouped_gemm_slice_k", "bst_quant_gemm_per_token",
           "bst_tile_map", "bst_grouped_tile_map", "bst_workspace_bytes", "bst_effective_sched",
           "bst_task_count", "bst_set_clock_record", "bst_last_error", "bst_version"]


class Sched(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in
                ("tile_m", "tile_n", "tile_k", "swizzle_offset", "swizzle_direction", "split_k",
                 "xcd_remap", "grid", "path", "shuffle_k", "dynamic", "preload")]


_lock = threading.Lock()
_lib = None


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libbst.so is not built (%s); run "
                                   "`python -m block_swizzle_tile_amd.build`" % LIB_PATH)
            # torch carries its own HIP runtime under the soname libamdhip64.so.7, the same
            # as the system one libbst.so links: whichever loads first serves the process.
            # torch is loaded first so that it keeps its own (loading libbst.so first binds
            # the system runtime, and torch then finds no GPU).
            import torch  # noqa: F401
            L = ctypes.CDLL(LIB_PATH)
            i64, i32, p, st = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
            sz, sp = ctypes.c_size_t, ctypes.POINTER(Sched)
            L.bst_gemm.argtypes = [st, st, i64, i64, i64, p, i64, p, i64, p, i64, p, p, sp, p, sz, p]
            L.bst_gemm_noalloc.argtypes = [st, st, i64, i64, i64, p, i64, p, i64, p, i64, p, p,
                                           sp, p]
            L.bst_gemm_add.argtypes = [st, st, i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, p,
                                       sp, p, sz, p]
            L.bst_gemm_padded.argtypes = [st, st, i64, i64, i64, p, i64, p, i64, p, i64, p, p, sp,
                                          p, sz, p]
            L.bst_batched_gemm.argtypes = [st, st, i64, i64, i64, i64, p, i64, i64, p, i64, i64, p,
                                           i64, i64, sp, p, sz, p]
            L.bst_grouped_gemm_slice_m.argtypes = [st, st, i32, p, i64, i64, i64, p, i64, p, i64,
                                                   i64, p, i64, p, p, sp, p, sz, p]
            L.bst_grouped_gemm_slice_k.argtypes = [st, st, i32, p, i64, i64, i64, p, i64, p, i64,
                                                   p, i64, i64, p, p, sp, p, sz, p]
            L.bst_quant_gemm_per_token.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, p, i64, st,
                                                   sp, p, sz, p]
            L.bst_tile_map.argtypes = [st, i64, i64, i64, sp, p, i64, p]
            L.bst_grouped_tile_map.argtypes = [st, i32, p, i64, i64, sp, p, i64, p]
            L.bst_workspace_bytes.argtypes = [ctypes.c_int, st, i64, i64, i64, i64, sp]
            L.bst_workspace_bytes.restype = sz
            L.bst_effective_sched.argtypes = [ctypes.c_int, st, i64, i64, i64, i64, sp, sp]
            L.bst_task_count.argtypes = [ctypes.c_int, st, i64, i64, i64, sp,
                                         ctypes.POINTER(i64)]
            for fn in ("bst_gemm", "bst_gemm_noalloc", "bst_gemm_add", "bst_gemm_padded", "bst_batched_gemm",
                       "bst_grouped_gemm_slice_m", "bst_grouped_gemm_slice_k",
                       "bst_quant_gemm_per_token", "bst_tile_map", "bst_grouped_tile_map",
                       "bst_effective_sched", "bst_task_count"):
                getattr(L, fn).restype = st
            L.bst_set_clock_record.argtypes = [p, i64]
            L.bst_set_clock_record.restype = st
            L.bst_last_error.restype = ctypes.c_char_p
            L.bst_version.restype = ctypes.c_char_p
            _lib = L
    return _lib


class BstError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


def check(status):
    if status != OK:
        raise BstError(status, lib().bst_last_error().decode(errors="replace"))
