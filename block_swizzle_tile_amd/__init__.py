"""Swizzled tiled GEMM for AMD MI355X (gfx950): Python binding of libbst.so.

Every function here is argument marshalling around the C ABI of
``include/bst.h``: it checks that operands are CUDA (HIP) tensors, passes
their data pointers, leading dimensions and the current stream, allocates
the output and the split-K workspace with torch when the caller gives none,
and raises :class:`BstError` on a non-OK status.  All computation runs in the
HIP kernels of libbst.so; there is no CPU path.

Names follow the C ABI without the ``bst_`` prefix: :func:`gemm`,
:func:`batched_gemm`, :func:`grouped_gemm_slice_m`, :func:`grouped_gemm_slice_k`,
:func:`quant_gemm_per_token`, :func:`tile_map`, :func:`grouped_tile_map`,
:func:`workspace_bytes`, :func:`effective_sched`.
"""
from __future__ import annotations

import ctypes

from ._lib import (BF16, E4M3, F16, F32, I8, I32, MXE4M3, BstError, Sched, check, lib,  # noqa: F401
                   LIB_PATH)

ZN, NZ, RASTER = 0, 1, 2
_DIRS = {"zn": ZN, "nz": NZ, "raster": RASTER}

__all__ = ["Sched", "BstError", "make_sched", "gemm", "gemm_padded", "batched_gemm",
           "grouped_gemm_slice_m", "grouped_gemm_slice_k",
           "quant_gemm_per_token", "tile_map", "grouped_tile_map", "workspace_bytes",
           "effective_sched", "task_count", "clock_record", "version", "LIB_PATH"]


def make_sched(tile=(0, 0), tile_k=0, offset=1, direction="zn", split_k=1, xcd_remap=0, grid=0,
               path=0, shuffle_k=0, dynamic=0, preload=0):
    """A :class:`Sched` from Python values (direction: 'zn', 'nz', 'raster' or 0/1/2;
    path: 0 automatic, 1 register-staged kernels, 2 LDS-DMA kernels, 3 LDS-DMA kernels with
    two resident workgroups per CU; shuffle_k: 1 rotates
    each task's K-loop start; dynamic: 1 per-XCD work queues; preload: 1 issues the next
    task's first stages before the current epilogue)."""
    d = _DIRS[direction] if isinstance(direction, str) else int(direction)
    return Sched(tile[0], tile[1], tile_k, offset, d, split_k, xcd_remap, grid, path,
                 int(shuffle_k), int(dynamic), int(preload))


def gemm_padded(A, B, C=None, *, out_dtype=None, scale_a=None, scale_b=None, sched=None,
                workspace=None):
    """C = A @ B for operands with any row stride and element-aligned base (e.g. column
    slices): they are repacked into an aligned workspace first (bst_gemm_padded)."""
    torch = _torch()
    _dev(A, B, C, scale_a, scale_b)
    scaled = scale_a is not None
    ab = _code(A.dtype, scaled)
    if _code(B.dtype, scaled) != ab:
        raise TypeError("A and B dtypes differ")
    M, K = A.shape
    N = B.shape[1]
    if C is None:
        if out_dtype is None:
            out_dtype = {F16: torch.float16, BF16: torch.bfloat16, E4M3: torch.bfloat16,
                         MXE4M3: torch.bfloat16, I8: torch.int32}[ab]
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    c = _code(C.dtype)
    nb = workspace_bytes(2, ab, 1, M, N, K, sched)
    ws, wsb = (workspace, workspace.numel()) if workspace is not None else _workspace(nb, A.device)
    check(lib().bst_gemm_padded(ab, c, M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(C),
                                _ld(C), _ptr(scale_a), _ptr(scale_b), _sched(sched), _ptr(ws),
                                wsb, _stream(A.device)))
    return C


def version():
    return lib().bst_version().decode()


def clock_record(buf=None, n=0):
    """Measurement hook: while set, GEMMs on the LDS-DMA kernels record each of their first n
    workgroups' clock in buf (an int64 GPU tensor of at least 4 n elements: reference counter
    at start and end, shader cycles, 1); clock_record() turns it off."""
    check(lib().bst_set_clock_record(_ptr(buf), n))


def _torch():
    import torch
    return torch


def _code(t, scaled=False):
    torch = _torch()
    m = {torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8, torch.int32: I32,
         torch.float32: F32, torch.float8_e4m3fn: MXE4M3 if scaled else E4M3}
    if t not in m:
        raise TypeError("unsupported dtype %s" % t)
    return m[t]


def _out_dtype(code):
    torch = _torch()
    return {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32, I32: torch.int32}[code]


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("operands must be GPU tensors")


def _ld(t):
    """Leading dimension of a row-major 2-D (or batched 3-D) tensor."""
    if t.stride(-1) != 1:
        raise ValueError("innermost dimension must be contiguous")
    return t.stride(-2) if t.dim() >= 2 else t.shape[-1]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_ws_cache = {}


def _workspace(nbytes, device):
    """Zero-initialised workspace, cached per (device, stream); grown on demand.
    The kernels leave its counters zero again after every call."""
    if nbytes == 0:
        return None, 0
    torch = _torch()
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws, ws.numel()


def _sched(s):
    if s is None:
        return None
    return ctypes.byref(s)


def workspace_bytes(kind, ab, count, M, N, K, sched=None):
    """Workspace bytes (kind 0: plain/batched with count = batch, 1: grouped slice-M with
    count = G, 2: padding GEMM, 3: grouped slice-K with count = G and K = total_k)."""
    return lib().bst_workspace_bytes(kind, ab, count, M, N, K, _sched(sched))


def effective_sched(kind, ab, count, M, N, K, sched=None):
    out = Sched()
    check(lib().bst_effective_sched(kind, ab, count, M, N, K, _sched(sched), ctypes.byref(out)))
    return out


def gemm(A, B, C=None, *, out_dtype=None, scale_a=None, scale_b=None, sched=None, workspace=None,
         add=None):
    """C = A @ B for row-major A[M][K], B[K][N] (fp16, bf16, e4m3fn (+ MX scales) or int8);
    with add=X (C's shape and dtype, may be C itself): C = A @ B + X."""
    torch = _torch()
    _dev(A, B, C, scale_a, scale_b, add)
    scaled = scale_a is not None
    ab = _code(A.dtype, scaled)
    if _code(B.dtype, scaled) != ab:
        raise TypeError("A and B dtypes differ")
    M, K = A.shape
    N = B.shape[1]
    if C is None:
        if out_dtype is None:
            out_dtype = {F16: torch.float16, BF16: torch.bfloat16, E4M3: torch.bfloat16,
                         MXE4M3: torch.bfloat16, I8: torch.int32}[ab]
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    c = _code(C.dtype)
    nb = workspace_bytes(0, ab, 1, M, N, K, sched)
    ws, wsb = (workspace, workspace.numel()) if workspace is not None else _workspace(nb, A.device)
    if add is not None:
        if add.dtype != C.dtype or tuple(add.shape) != (M, N):
            raise TypeError("the addend must have C's dtype and shape")
        check(lib().bst_gemm_add(ab, c, M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(add),
                                 _ld(add), _ptr(C), _ld(C), _ptr(scale_a), _ptr(scale_b),
                                 _sched(sched), _ptr(ws), wsb, _stream(A.device)))
        return C
    check(lib().bst_gemm(ab, c, M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(C), _ld(C),
                         _ptr(scale_a), _ptr(scale_b), _sched(sched), _ptr(ws), wsb,
                         _stream(A.device)))
    return C


def batched_gemm(A, B, C=None, *, out_dtype=None, sched=None, workspace=None):
    """C[b] = A[b] @ B[b] for 3-D row-major A[batch][M][K], B[batch][K][N]."""
    torch = _torch()
    _dev(A, B, C)
    ab = _code(A.dtype)
    batch, M, K = A.shape
    N = B.shape[2]
    if C is None:
        if out_dtype is None:
            out_dtype = {F16: torch.float16, BF16: torch.bfloat16, E4M3: torch.bfloat16,
                         I8: torch.int32}[ab]
        C = torch.empty((batch, M, N), dtype=out_dtype, device=A.device)
    c = _code(C.dtype)
    nb = workspace_bytes(0, ab, batch, M, N, K, sched)
    ws, wsb = (workspace, workspace.numel()) if workspace is not None else _workspace(nb, A.device)
    check(lib().bst_batched_gemm(ab, c, batch, M, N, K, _ptr(A), _ld(A), A.stride(0), _ptr(B),
                                 _ld(B), B.stride(0), _ptr(C), _ld(C), C.stride(0), _sched(sched),
                                 _ptr(ws), wsb, _stream(A.device)))
    return C


def grouped_gemm_slice_m(A, B, group_m, C=None, *, row_scale=None, col_scale=None,
                         out_dtype=None, sched=None, workspace=None):
    """Groups stacked along M: rows of group g of A / C use B[g]; group_m is a
    device int32 tensor of G row counts (never read on the host)."""
    torch = _torch()
    _dev(A, B, C, group_m, row_scale, col_scale)
    if group_m.dtype != torch.int32:
        raise TypeError("group_m must be int32")
    ab = _code(A.dtype)
    total_m, K = A.shape
    G, _, N = B.shape
    if C is None:
        if out_dtype is None:
            out_dtype = torch.bfloat16 if row_scale is not None else (
                torch.int32 if ab == I8 else A.dtype)
        C = torch.empty((total_m, N), dtype=out_dtype, device=A.device)
    c = _code(C.dtype)
    nb = workspace_bytes(1, ab, G, total_m, N, K, sched)
    ws, wsb = (workspace, workspace.numel()) if workspace is not None else _workspace(nb, A.device)
    check(lib().bst_grouped_gemm_slice_m(ab, c, G, _ptr(group_m), total_m, N, K, _ptr(A), _ld(A),
                                         _ptr(B), _ld(B), B.stride(0), _ptr(C), _ld(C),
                                         _ptr(row_scale), _ptr(col_scale), _sched(sched),
                                         _ptr(ws), wsb, _stream(A.device)))
    return C


def grouped_gemm_slice_k(A, B, group_k, C=None, *, row_scale=None, col_scale=None,
                         out_dtype=None, sched=None, workspace=None):
    """K cut into groups: group g multiplies A[:, Q_g:Q_g+k_g] by B[Q_g:Q_g+k_g, :] into
    C[g] (A [M][total_k], B [total_k][N], C [G][M][N]); group_k is a device int32 tensor of
    G sizes (never read on the host); row_scale [G][M] / col_scale [G][N] for int8 dequant."""
    torch = _torch()
    _dev(A, B, C, group_k, row_scale, col_scale)
    if group_k.dtype != torch.int32:
        raise TypeError("group_k must be int32")
    ab = _code(A.dtype)
    M, total_k = A.shape
    N = B.shape[1]
    G = group_k.numel()
    if C is None:
        if out_dtype is None:
            out_dtype = torch.bfloat16 if row_scale is not None else (
                torch.int32 if ab == I8 else A.dtype)
        C = torch.empty((G, M, N), dtype=out_dtype, device=A.device)
    c = _code(C.dtype)
    nb = workspace_bytes(3, ab, G, M, N, total_k, sched)
    ws, wsb = (workspace, workspace.numel()) if workspace is not None else _workspace(nb, A.device)
    check(lib().bst_grouped_gemm_slice_k(ab, c, G, _ptr(group_k), total_k, M, N, _ptr(A), _ld(A),
                                         _ptr(B), _ld(B), _ptr(C), _ld(C),
                                         C.stride(0) if C.dim() == 3 else 0, _ptr(row_scale),
                                         _ptr(col_scale), _sched(sched), _ptr(ws), wsb,
                                         _stream(A.device)))
    return C


def quant_gemm_per_token(A, B, row_scale, col_scale, C=None, *, out_dtype=None, sched=None,
                         workspace=None):
    """int8 A[M][K] @ int8 B[K][N], int32 accumulate, out = acc * row_scale[i] * col_scale[j]
    (out_dtype int32 writes the raw accumulators)."""
    torch = _torch()
    _dev(A, B, C, row_scale, col_scale)
    M, K = A.shape
    N = B.shape[1]
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=A.device)
    c = _code(C.dtype)
    nb = workspace_bytes(0, I8, 1, M, N, K, sched)
    ws, wsb = (workspace, workspace.numel()) if workspace is not None else _workspace(nb, A.device)
    check(lib().bst_quant_gemm_per_token(M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B),
                                         _ptr(row_scale), _ptr(col_scale), _ptr(C), _ld(C), c,
                                         _sched(sched), _ptr(ws), wsb, _stream(A.device)))
    return C


def task_count(kind, ab, count, M, N, sched=None):
    """Task count of the scheduler (kind 0: exact, count = batch; kind 1: the bound for a
    grouped problem, count = G, M = total_m)."""
    n = ctypes.c_int64(0)
    check(lib().bst_task_count(kind, ab, count, M, N, _sched(sched), ctypes.byref(n)))
    return n.value


def tile_map(batch, M, N, sched=None, *, ab=F16, device="cuda"):
    """[T, 8] int32 tensor of {batch, m, n, mActual, nActual, 0, xcc, workgroup} per task,
    computed on the GPU by the kernels' scheduler."""
    torch = _torch()
    T = task_count(0, ab, batch, M, N, sched)
    out = torch.full((max(T, 1), 8), -1, dtype=torch.int32, device=device)
    check(lib().bst_tile_map(ab, batch, M, N, _sched(sched), _ptr(out), out.shape[0],
                             _stream(out.device)))
    return out[:T]


def grouped_tile_map(group_m, total_m, N, sched=None, *, ab=I8):
    """[T_bound, 8] int32 tensor {g, m, n, mActual, nActual, row0, xcc, workgroup}; rows past
    the device-side task count stay -1."""
    torch = _torch()
    _dev(group_m)
    G = group_m.numel()
    bound = task_count(1, ab, G, total_m, N, sched)
    out = torch.full((max(bound, 1), 8), -1, dtype=torch.int32, device=group_m.device)
    check(lib().bst_grouped_tile_map(ab, G, _ptr(group_m), total_m, N, _sched(sched), _ptr(out),
                                     out.shape[0], _stream(group_m.device)))
    return out
