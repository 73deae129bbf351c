"""CPU oracle for the swizzled tiled GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``block_swizzle_tile_amd``) never imports it and shares no code with it.

This module is argument marshalling around ``oracle.c`` (plain C, fp64 /
int64, OpenMP over tasks); every computation lives there and is documented
there with the passage of the pages it follows ("Block Scheduler Code
Explained": s4.1-s4.6 for the map, s6 for runtime offset/direction).

Parity status: the map (Zn, RASTER), the tail shapes, the batch / group
decomposition, the decoders, the GEMM, the dequant and the compare are pinned
by the CPU tests in ``tests/test_oracle_*.py``.  The Nz order is the mirror
reading of an elided passage: its self-consistency is pinned, its choice
among mirror readings is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB selects a prebuilt copy (the sanitizer build of the CPU tests), used as is
_LIB_ENV = os.environ.get("ORACLE_LIB")
_LIB = _LIB_ENV or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

# dtype codes of the oracle (its own numbering, see oracle.c)
F16, BF16, E4M3, MXE4M3, I8 = 1, 2, 3, 4, 5
DIR = {"zn": 0, "nz": 1, "raster": 2}
_DECODE_KIND = {"f16": 1, "bf16": 2, "e4m3": 3, "i8": 5, "i32": 6, "f32": 7, "e8m0": 8}


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP)."""
    if _LIB_ENV:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-shared",
                               "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            i64, i32, p, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
            L.orc_tile_map.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int, p, i64]
            L.orc_tile_map.restype = i64
            L.orc_grouped_tile_map.argtypes = [i32, p, i64, i64, i64, i64, ctypes.c_int, p, i64]
            L.orc_grouped_tile_map.restype = i64
            L.orc_decode.argtypes = [ctypes.c_int, p, i64, p]
            L.orc_decode.restype = ctypes.c_int
            L.orc_gemm.argtypes = [ctypes.c_int, i64, i64, i64, i64, p, i64, i64, p, i64, i64,
                                   p, i64, p, i64, i64, i64, i64, ctypes.c_int, p, i64, p, p, p]
            L.orc_gemm.restype = ctypes.c_int
            L.orc_grouped_gemm.argtypes = [i32, p, i64, i64, i64, p, i64, p, i64, i64, p, p,
                                           i64, i64, i64, ctypes.c_int, p, i64, p, p, p]
            L.orc_grouped_gemm.restype = ctypes.c_int
            L.orc_grouped_gemm_slice_k.argtypes = [ctypes.c_int, i32, p, i64, i64, i64, p, i64,
                                                   p, i64, p, p, i64, i64, i64, ctypes.c_int, p,
                                                   i64, p, p, p]
            L.orc_grouped_gemm_slice_k.restype = ctypes.c_int
            L.orc_add_addend.argtypes = [i64, p, p, p]
            L.orc_add_addend.restype = ctypes.c_int
            L.orc_threads.argtypes = [ctypes.c_int]
            L.orc_threads.restype = ctypes.c_int
            L.orc_compare.argtypes = [i64, p, p, p, p]
            L.orc_compare.restype = dbl
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dir(direction):
    return DIR[direction] if isinstance(direction, str) else int(direction)


def tile_map(batch, M, N, tm, tn, off, direction):
    """[T, 5] uint32 rows {batch, m, n, mActual, nActual} in task order."""
    T = batch * (-(-M // tm)) * (-(-N // tn))
    out = np.zeros((max(T, 1), 5), np.uint32)
    r = lib().orc_tile_map(batch, M, N, tm, tn, off, _dir(direction), _ptr(out), T)
    if r < 0:
        raise ValueError("orc_tile_map failed (%d)" % r)
    return out[:r]


def grouped_tile_map(group_m, N, tm, tn, off, direction):
    """[T, 6] uint32 rows {g, m, n, mActual, nActual, first stacked row}."""
    gm = np.ascontiguousarray(group_m, dtype=np.int32)
    T = int(sum((-(-int(x) // tm)) * (-(-N // tn)) for x in gm))
    out = np.zeros((max(T, 1), 6), np.uint32)
    r = lib().orc_grouped_tile_map(len(gm), _ptr(gm), N, tm, tn, off, _dir(direction),
                                   _ptr(out), T)
    if r < 0:
        raise ValueError("orc_grouped_tile_map failed (%d)" % r)
    return out[:r]


def decode(kind, bits):
    """Exact value of each raw code as float64 (kind: f16 bf16 e4m3 e8m0 i8 i32 f32)."""
    src = np.ascontiguousarray(bits)
    dst = np.zeros(src.size, np.float64)
    if lib().orc_decode(_DECODE_KIND[kind], _ptr(src), src.size, _ptr(dst)) != 0:
        raise ValueError(kind)
    return dst.reshape(src.shape)


def gemm(ab, A, B, *, batch=1, M=None, N=None, K=None, lda=None, ldb=None, strideA=0,
         strideB=0, scale_a=None, scale_b=None, tile=(64, 64), off=1, direction="zn",
         rows=None, want_acc=False):
    """fp64 (int64 for int8) oracle of C_b = A_b . B_b; returns (ref, den[, acc]).

    A, B hold raw codes (uint16 for f16/bf16, uint8 for e4m3, int8 for i8)
    flattened or 2-D; rows selects stacked rows b*M+i (None = all) and the
    outputs are [len(rows), N].
    """
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if M is None:
        M, K = A.shape[-2], A.shape[-1]
    if N is None:
        N = B.shape[-1]
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    nrows = batch * M if rows is None else len(rows)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    ref = np.zeros((nrows, N), np.float64)
    den = np.zeros((nrows, N), np.float64)
    acc = np.zeros((nrows, N), np.int64) if want_acc else None
    sa = None if scale_a is None else np.ascontiguousarray(scale_a, dtype=np.uint8)
    sb = None if scale_b is None else np.ascontiguousarray(scale_b, dtype=np.uint8)
    ldsa = K // 32 if sa is not None else 0
    ldsb = N if sb is not None else 0
    rc = lib().orc_gemm(ab, batch, M, N, K, _ptr(A), lda, strideA, _ptr(B), ldb, strideB,
                        _ptr(sa), ldsa, _ptr(sb), ldsb, tile[0], tile[1], off, _dir(direction),
                        _ptr(rows_a), nrows, _ptr(ref), _ptr(den), _ptr(acc))
    if rc != 0:
        raise ValueError("orc_gemm failed (%d)" % rc)
    return (ref, den, acc) if want_acc else (ref, den)


def grouped_gemm(group_m, A, B, N, K, *, row_scale=None, col_scale=None, tile=(128, 128),
                 off=1, direction="zn", rows=None, lda=None, ldb=None, strideB=None):
    """int8 grouped slice-M oracle; returns (ref, den, acc) for the selected stacked rows."""
    gm = np.ascontiguousarray(group_m, dtype=np.int32)
    A = np.ascontiguousarray(A, dtype=np.int8)
    B = np.ascontiguousarray(B, dtype=np.int8)
    lda = K if lda is None else lda
    total_m = A.size // lda if lda else int(gm.sum())
    ldb = N if ldb is None else ldb
    strideB = K * ldb if strideB is None else strideB
    sumM = int(gm.sum())
    nrows = sumM if rows is None else len(rows)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    ref = np.zeros((nrows, N), np.float64)
    den = np.zeros((nrows, N), np.float64)
    acc = np.zeros((nrows, N), np.int64)
    rs = None if row_scale is None else np.ascontiguousarray(row_scale, dtype=np.float32)
    cs = None if col_scale is None else np.ascontiguousarray(col_scale, dtype=np.float32)
    rc = lib().orc_grouped_gemm(len(gm), _ptr(gm), max(total_m, sumM), N, K, _ptr(A), lda,
                                _ptr(B), ldb, strideB, _ptr(rs), _ptr(cs), tile[0], tile[1],
                                off, _dir(direction), _ptr(rows_a), nrows, _ptr(ref),
                                _ptr(den), _ptr(acc))
    if rc != 0:
        raise ValueError("orc_grouped_gemm failed (%d)" % rc)
    return ref, den, acc


def grouped_gemm_slice_k(ab, group_k, A, B, M, N, *, total_k=None, lda=None, ldb=None,
                         row_scale=None, col_scale=None, tile=(128, 128), off=1,
                         direction="zn", rows=None):
    """Grouped slice-K oracle (orc_grouped_gemm_slice_k in oracle.c): group g multiplies
    A[:, Q_g:Q_g+k_g] by B[Q_g:Q_g+k_g, :]; outputs stacked as rows g*M + i.  A, B: raw
    codes (uint16 f16/bf16, int8); row_scale [G][M], col_scale [G][N] (int8 only).
    Returns (ref, den, acc) for the selected stacked rows (acc: int64, int8 only)."""
    gk = np.ascontiguousarray(group_k, dtype=np.int32)
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    total_k = int(gk.sum()) if total_k is None else total_k
    lda = total_k if lda is None else lda
    ldb = N if ldb is None else ldb
    G = len(gk)
    nrows = G * M if rows is None else len(rows)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    ref = np.zeros((nrows, N), np.float64)
    den = np.zeros((nrows, N), np.float64)
    acc = np.zeros((nrows, N), np.int64)
    rs = None if row_scale is None else np.ascontiguousarray(row_scale, dtype=np.float32)
    cs = None if col_scale is None else np.ascontiguousarray(col_scale, dtype=np.float32)
    rc = lib().orc_grouped_gemm_slice_k(ab, G, _ptr(gk), total_k, M, N, _ptr(A), lda, _ptr(B),
                                        ldb, _ptr(rs), _ptr(cs), tile[0], tile[1], off,
                                        _dir(direction), _ptr(rows_a), nrows, _ptr(ref),
                                        _ptr(den), _ptr(acc))
    if rc != 0:
        raise ValueError("orc_grouped_gemm_slice_k failed (%d)" % rc)
    return ref, den, acc


def gemm_add(ab, A, B, X, x_kind, **kw):
    """matmul-add oracle C = A . B + X: (ref, den) of gemm() with the addend's exact values
    (X: raw codes of kind x_kind, the output's shape, or the selected rows when rows= is
    given) added to ref and their magnitudes to den (orc_add_addend in oracle.c)."""
    ref, den = gemm(ab, A, B, **kw)
    x = np.ascontiguousarray(decode(x_kind, X), dtype=np.float64).reshape(ref.shape)
    if lib().orc_add_addend(ref.size, _ptr(x), _ptr(ref), _ptr(den)) != 0:
        raise ValueError("orc_add_addend failed")
    return ref, den


def threads(n=0):
    """OpenMP thread count of the oracle's loops: n > 0 sets it; returns the count in use."""
    return lib().orc_threads(int(n))


def compare(got, ref, den):
    """(max normalised error, flat argmax) -- see orc_compare in oracle.c."""
    g = np.ascontiguousarray(got, dtype=np.float64).ravel()
    r = np.ascontiguousarray(ref, dtype=np.float64).ravel()
    d = np.ascontiguousarray(den, dtype=np.float64).ravel()
    assert g.size == r.size == d.size
    am = ctypes.c_int64(-1)
    e = lib().orc_compare(g.size, _ptr(g), _ptr(r), _ptr(d), ctypes.byref(am))
    return e, am.value
