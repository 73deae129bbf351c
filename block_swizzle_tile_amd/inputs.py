"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method (no tile map, no GEMM): it
only draws random operands and returns them as raw codes on the host
(``numpy`` arrays of uint16 fp16/bf16 bits, uint8 e4m3fn / e8m0 codes, int8,
float32 scales), so that the CPU oracle and the GPU path consume exactly the
same bytes.  Every draw uses
``numpy.random.Generator(PCG64(SeedSequence([workload_id, tensor_id])))``.

Recipes (one per workload of the method's measurement set):

* tails       -- fp16 A[200][256], B[256][136] = RNE(U[-1, 1]).
* fp16_2k     -- fp16 A[1024][2048], B[2048][1024] = RNE(U[-1, 1]).
* mxfp8_4k    -- e4m3fn A[1024][4096], B[4096][2048] with e8m0 block scales
                 (one per row and 32-wide K block for A, per K block and
                 column for B): scale code 127 + U{-2..2}; element =
                 e4m3fn_RNE(clamp(x / 2^(scale-127), +-448)), x ~ N(0, 1).
* bf16_batch  -- 16 x { A[512][1024], B[1024][768] } bf16 = RNE(N(0, 0.02)).
* int8_groups -- 8 groups, sizes ~ Multinomial(8192, Dirichlet(0.5 * 1_8))
                 (first draw with no empty group and at least one group of
                 1..127 rows), A int8[8192][2048], B int8[8][2048][4096]
                 = U{-127..127}, row scales f32[8192] and column scales
                 f32[8][4096] = LogNormal(0, 0.5).
* int8_slice_k -- grouped slice-K: 8 groups cutting K = 8192, sizes
                 16 * Multinomial(512, Dirichlet(0.5 * 1_8)) (whole 16-byte
                 units; first draw with no empty group and one group under
                 128), A int8[1024][8192], B int8[8192][2048] = U{-127..127},
                 row scales f32[8][1024] and column scales f32[8][2048] =
                 LogNormal(0, 0.5); one bf16 [1024][2048] output per group.
"""
from __future__ import annotations

import numpy as np

WORKLOAD_IDS = {"tails": 1, "fp16_2k": 2, "mxfp8_4k": 3, "bf16_batch": 4, "int8_groups": 5,
                "int8_slice_k": 6}


def rng(workload_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, tensor_id])))


def f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to fp16 (numpy RNE) and return the uint16 codes."""
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (torch RNE cast) and return the uint16 codes."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Clamp to +-448, round to OCP e4m3fn (torch RNE cast), return uint8 codes."""
    import torch
    c = np.clip(np.asarray(x, np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(c)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def uniform_f16(shape, workload_id, tensor_id, lo=-1.0, hi=1.0):
    return f16_bits(rng(workload_id, tensor_id).uniform(lo, hi, size=shape))


def uniform_bf16(shape, workload_id, tensor_id, lo=-1.0, hi=1.0):
    return bf16_bits(rng(workload_id, tensor_id).uniform(lo, hi, size=shape))


def normal_bf16(shape, workload_id, tensor_id, std=0.02):
    return bf16_bits(rng(workload_id, tensor_id).normal(0.0, std, size=shape))


def int8_uniform(shape, workload_id, tensor_id, lo=-127, hi=127):
    return rng(workload_id, tensor_id).integers(lo, hi + 1, size=shape).astype(np.int8)


def lognormal_f32(shape, workload_id, tensor_id, sigma=0.5):
    return rng(workload_id, tensor_id).lognormal(0.0, sigma, size=shape).astype(np.float32)


def mx_a(M, K, workload_id, tensor_id):
    """e4m3fn A[M][K] and e8m0 scales sa[M][K/32] (one per row and K block)."""
    g = rng(workload_id, tensor_id)
    sa = (127 + g.integers(-2, 3, size=(M, K // 32))).astype(np.uint8)
    x = g.normal(0.0, 1.0, size=(M, K))
    scale = np.repeat(np.exp2(sa.astype(np.float64) - 127.0), 32, axis=1)
    return e4m3_bits(x / scale), sa


def mx_b(K, N, workload_id, tensor_id):
    """e4m3fn B[K][N] and e8m0 scales sb[K/32][N] (one per K block and column)."""
    g = rng(workload_id, tensor_id)
    sb = (127 + g.integers(-2, 3, size=(K // 32, N))).astype(np.uint8)
    x = g.normal(0.0, 1.0, size=(K, N))
    scale = np.repeat(np.exp2(sb.astype(np.float64) - 127.0), 32, axis=0)
    return e4m3_bits(x / scale), sb


def group_sizes(G=8, total=8192, workload_id=5, small=128, max_attempts=1000):
    """Group row counts: first draw with no empty group and one group < `small` rows."""
    for attempt in range(max_attempts):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, 100 + attempt])))
        p = g.dirichlet(np.full(G, 0.5))
        m = g.multinomial(total, p)
        if m.min() >= 1 and ((m >= 1) & (m < small)).any():
            return m.astype(np.int32)
    raise RuntimeError("no acceptable group-size draw")


def group_k_sizes(G=8, total=8192, workload_id=6, unit=16, small=128, max_attempts=1000):
    """Slice-K group sizes in whole `unit`s: first draw with no empty group and one
    group under `small`."""
    for attempt in range(max_attempts):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, 100 + attempt])))
        p = g.dirichlet(np.full(G, 0.5))
        k = g.multinomial(total // unit, p) * unit
        if k.min() >= unit and (k < small).any():
            return k.astype(np.int32)
    raise RuntimeError("no acceptable group-size draw")


def workload(name: str, *, small: bool = False) -> dict:
    """Host arrays of one named workload.  small=True shrinks the big ones
    (same recipe, fewer rows/cols) for quick checks."""
    wid = WORKLOAD_IDS[name]
    if name == "tails":
        M, N, K = 200, 136, 256
        return dict(dtype="f16", M=M, N=N, K=K, A=uniform_f16((M, K), wid, 0),
                    B=uniform_f16((K, N), wid, 1), tile=(64, 64), off=3, direction="zn")
    if name == "fp16_2k":
        M, N, K = (256, 256, 512) if small else (1024, 1024, 2048)
        return dict(dtype="f16", M=M, N=N, K=K, A=uniform_f16((M, K), wid, 0),
                    B=uniform_f16((K, N), wid, 1), tile=(256, 128), off=1, direction="zn")
    if name == "mxfp8_4k":
        M, N, K = (256, 512, 1024) if small else (1024, 2048, 4096)
        A, sa = mx_a(M, K, wid, 0)
        B, sb = mx_b(K, N, wid, 1)
        return dict(dtype="mxe4m3", M=M, N=N, K=K, A=A, B=B, scale_a=sa, scale_b=sb,
                    tile=(256, 256), off=4, direction="zn")
    if name == "bf16_batch":
        batch, M, N, K = (2, 128, 192, 256) if small else (16, 512, 768, 1024)
        return dict(dtype="bf16", batch=batch, M=M, N=N, K=K,
                    A=normal_bf16((batch, M, K), wid, 0), B=normal_bf16((batch, K, N), wid, 1),
                    tile=(128, 192), off=1, direction="zn")
    if name == "int8_groups":
        G, total, N, K = (4, 1024, 512, 256) if small else (8, 8192, 4096, 2048)
        gm = group_sizes(G, total, wid)
        return dict(dtype="i8", G=G, group_m=gm, total_m=total, N=N, K=K,
                    A=int8_uniform((total, K), wid, 0), B=int8_uniform((G, K, N), wid, 1),
                    row_scale=lognormal_f32((total,), wid, 2),
                    col_scale=lognormal_f32((G, N), wid, 3), tile=(256, 256), off=1,
                    direction="zn")
    if name == "int8_slice_k":
        G, M, N, total = (4, 128, 256, 1024) if small else (8, 1024, 2048, 8192)
        gk = group_k_sizes(G, total, wid)
        return dict(dtype="i8", G=G, group_k=gk, total_k=total, M=M, N=N,
                    A=int8_uniform((M, total), wid, 0), B=int8_uniform((total, N), wid, 1),
                    row_scale=lognormal_f32((G, M), wid, 2),
                    col_scale=lognormal_f32((G, N), wid, 3), tile=(256, 256), off=1,
                    direction="zn")
    raise KeyError(name)
