"""GPU parity of the tail paths that whole-tile workloads never reach.

Tail tiles are part of the map itself ("Block Scheduler Code Explained",
s4.6 GetActualBlockShape and s5.3): the last tile-row and tile-column of a
problem are shorter than the tile.  These tests run the 8-bit paths (MX-fp8
on the LDS-DMA kernels, whose block-scale DMAs mask the rows and columns
past the problem; MX-fp8 on the register-staged kernels with K not a
multiple of the 128-deep stage; plain e4m3), batched problems with ragged M
and N, and the MX matmul-add, all at shapes whose M and N are not multiples
of the tile.  Every output sits inside a NaN guard band (rows above and
below, columns to the right, and between batches), so a store outside the
M x N result is caught as well as a wrong value.
"""
import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I
from gpu_util import TOL_16, TOL_8, check_close, codes, say, to_gpu

pytestmark = pytest.mark.gpu


def bst():
    import block_swizzle_tile_amd as m
    return m


def guarded(M, N, dtype, lead=()):
    """NaN-filled buffer [*lead][M + 2][ldc] and the [*lead][M][N] view at row 1,
    ldc = N rounded up to 8 elements, plus 8 more (16-byte rows either way)."""
    import torch
    ldc = -(-N // 8) * 8 + 8
    full = torch.full(tuple(lead) + (M + 2, ldc), float("nan"), dtype=dtype, device="cuda")
    return full, full[..., 1:M + 1, :N]


def assert_guard(orc, full, M, N, kind):
    """Nothing outside the [M][N] result (per batch) was written."""
    c = orc.decode(kind, codes(full))
    c = c.reshape((-1,) + c.shape[-2:])
    for b in range(c.shape[0]):
        assert np.all(np.isnan(c[b, 0])), "row above the result written (batch %d)" % b
        assert np.all(np.isnan(c[b, M + 1])), "row below the result written (batch %d)" % b
        assert np.all(np.isnan(c[b, 1:M + 1, N:])), "columns right of the result written (batch %d)" % b


def pad_cols(x, fill, align=16):
    """x with its last dimension padded to a whole number of 16-byte units plus
    one more, the padding holding `fill` (a huge value's code, so that a read of
    the padding shows up in the result); returns (padded array, leading dim)."""
    es = x.dtype.itemsize
    cols = x.shape[-1]
    ld = -(-cols * es // align) * align // es + align // es
    out = np.full(x.shape[:-1] + (ld,), fill, dtype=x.dtype)
    out[..., :cols] = x
    return out, ld


E4M3_BIG = 0x7E     # 448, the largest e4m3fn value
F16_BIG = 0x7BFF    # 65504
BF16_BIG = 0x7F7F   # about 3.4e38


def mx_operands(M, N, K, seed):
    A, sa = I.mx_a(M, K, 90 + seed, 0)
    B, sb = I.mx_b(K, N, 90 + seed, 1)
    return A, sa, B, sb


# ------------------------------------------------------------- MX-fp8 ------
@pytest.mark.parametrize("M,N,K", [(200, 144, 384), (130, 96, 1024)])
def test_mxfp8_dma_ragged(orc, M, N, K):
    """MX-fp8 on the LDS-DMA kernels (path 2) with M and N tails: the A-row and
    B-column scale DMAs of the last tile-row / tile-column have lanes past the
    problem, which must write zeros (scale 2^-127 would do no harm, but a
    read of the next row's scales or a write past the tile would)."""
    import torch
    A, sa, B, sb = mx_operands(M, N, K, M)
    ref, den = orc.gemm(orc.MXE4M3, A, B, scale_a=sa, scale_b=sb, tile=(64, 64))
    At, Bt = to_gpu(A, "e4m3"), to_gpu(B, "e4m3")
    sat, sbt = to_gpu(sa, "u8"), to_gpu(sb, "u8")
    for tile in [(64, 128), (128, 128), (256, 256), (64, 64), (128, 64), (256, 128)]:
        for split in [1, 3]:
            sched = dict(tile=tile, offset=2, split_k=split, path=2)
            say("mx dma ragged", M, N, K, sched)
            eff = bst().effective_sched(0, bst().MXE4M3, 1, M, N, K, bst().make_sched(**sched))
            assert eff.path == 2
            full, C = guarded(M, N, torch.bfloat16)
            bst().gemm(At, Bt, C, scale_a=sat, scale_b=sbt, sched=bst().make_sched(**sched))
            check_close(orc, C, ref, den, TOL_8, str(sched))
            assert_guard(orc, full, M, N, "bf16")


@pytest.mark.parametrize("M,N,K", [(70, 50, 96), (130, 40, 160), (257, 129, 224)])
def test_mxfp8_register_path_k_tail(orc, M, N, K):
    """MX-fp8 with K a multiple of 32 but not of the 128-deep stage: the
    register-staged kernels (the automatic choice here) load a partial last
    stage and its scales; M and N are ragged too, and B's rows are padded to
    whole 16-byte units with huge values that must never be read."""
    import torch
    A, sa, B, sb = mx_operands(M, N, K, K)
    Ap, lda = pad_cols(A, E4M3_BIG)
    Bp, ldb = pad_cols(B, E4M3_BIG)
    ref, den = orc.gemm(orc.MXE4M3, Ap, Bp, M=M, N=N, K=K, lda=lda, ldb=ldb, scale_a=sa,
                        scale_b=sb, tile=(64, 64))
    At, Bt = to_gpu(Ap, "e4m3")[:, :K], to_gpu(Bp, "e4m3")[:, :N]
    sat, sbt = to_gpu(sa, "u8"), to_gpu(sb, "u8")
    for sched in [dict(tile=(64, 64)), dict(tile=(128, 128), offset=2, direction="nz"),
                  dict(tile=(256, 256), offset=1), dict(tile=(64, 128), split_k=2),
                  dict(tile=(128, 64), xcd_remap=1, path=1), dict(tile=(256, 128), path=1)]:
        say("mx register ragged", M, N, K, sched)
        eff = bst().effective_sched(0, bst().MXE4M3, 1, M, N, K, bst().make_sched(**sched))
        assert eff.path == 1
        full, C = guarded(M, N, torch.bfloat16)
        bst().gemm(At, Bt, C, scale_a=sat, scale_b=sbt, sched=bst().make_sched(**sched))
        check_close(orc, C, ref, den, TOL_8, str(sched))
        assert_guard(orc, full, M, N, "bf16")


def test_mxfp8_add_ragged(orc):
    """MX matmul-add C = A.B + X at a ragged shape (both MX matmul-add tiles)."""
    import torch
    M, N, K = 200, 144, 384
    A, sa, B, sb = mx_operands(M, N, K, 7)
    X = I.bf16_bits(I.rng(97, 2).uniform(-8.0, 8.0, size=(M, N)))
    ref, den = orc.gemm_add(orc.MXE4M3, A, B, X, "bf16", scale_a=sa, scale_b=sb, tile=(64, 64))
    At, Bt = to_gpu(A, "e4m3"), to_gpu(B, "e4m3")
    sat, sbt = to_gpu(sa, "u8"), to_gpu(sb, "u8")
    Xt = to_gpu(X, "bf16")
    for tile in [(64, 128), (128, 128)]:
        for split in [1, 2]:
            say("mx add ragged", tile, split)
            full, C = guarded(M, N, torch.bfloat16)
            bst().gemm(At, Bt, C, scale_a=sat, scale_b=sbt, add=Xt,
                       sched=bst().make_sched(tile=tile, offset=3, split_k=split))
            check_close(orc, C, ref, den, TOL_8, "%s %s" % (tile, split))
            assert_guard(orc, full, M, N, "bf16")


# ------------------------------------------------------------ plain e4m3 ---
@pytest.mark.parametrize("M,N,K,path", [(200, 144, 384, 2), (77, 160, 256, 2),
                                        (200, 136, 200, 1), (130, 96, 1000, 1)])
def test_plain_e4m3_ragged(orc, M, N, K, path):
    """Unscaled e4m3 with ragged M, N and K; the first two shapes run the
    LDS-DMA kernels, the last two (N or K not whole 16-byte chunks) the
    register-staged ones.  Operand rows are padded with huge values."""
    import torch
    g = I.rng(98, M + K)
    A, lda = pad_cols(I.e4m3_bits(g.normal(0.0, 1.0, size=(M, K))), E4M3_BIG)
    B, ldb = pad_cols(I.e4m3_bits(g.normal(0.0, 1.0, size=(K, N))), E4M3_BIG)
    ref, den = orc.gemm(orc.E4M3, A, B, M=M, N=N, K=K, lda=lda, ldb=ldb, tile=(64, 64))
    At, Bt = to_gpu(A, "e4m3")[:, :K], to_gpu(B, "e4m3")[:, :N]
    for tile in [(64, 64), (128, 128), (256, 256), (128, 64)]:
        for split in [1, 3]:
            sched = dict(tile=tile, offset=2, split_k=split, direction="nz" if split == 3 else "zn")
            say("e4m3 ragged", M, N, K, sched)
            eff = bst().effective_sched(0, bst().E4M3, 1, M, N, K, bst().make_sched(**sched))
            assert eff.path == path
            full, C = guarded(M, N, torch.bfloat16)
            bst().gemm(At, Bt, C, sched=bst().make_sched(**sched))
            check_close(orc, C, ref, den, TOL_8, str(sched))
            assert_guard(orc, full, M, N, "bf16")


# --------------------------------------------------------------- batched ---
@pytest.mark.parametrize("batch,M,N,K,path", [(3, 100, 200, 136, 2), (3, 70, 100, 72, 1),
                                              (2, 129, 264, 256, 2)])
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_batched_ragged(orc, batch, M, N, K, path, kind):
    """Batched GEMM whose M and N are not multiples of the tile: every batch
    has its own tail tile-row and tile-column, and the batch index of task t
    is t / (tiles per batch) (s4.4 GetBatchIdx).  Batches of C sit inside
    guard rows, so a store into a neighbouring batch is caught; operand rows
    are padded with huge values."""
    import torch
    g = I.rng(99, batch * M + N)
    x = g.uniform(-1.0, 1.0, size=(batch, M, K))
    y = g.uniform(-1.0, 1.0, size=(batch, K, N))
    A = I.f16_bits(x) if kind == "f16" else I.bf16_bits(x)
    B = I.f16_bits(y) if kind == "f16" else I.bf16_bits(y)
    big = F16_BIG if kind == "f16" else BF16_BIG
    A, lda = pad_cols(A, big)
    B, ldb = pad_cols(B, big)
    code = orc.F16 if kind == "f16" else orc.BF16
    ab = bst().F16 if kind == "f16" else bst().BF16
    ref, den = orc.gemm(code, A, B, batch=batch, M=M, N=N, K=K, lda=lda, ldb=ldb,
                        strideA=M * lda, strideB=K * ldb, tile=(64, 64))
    At, Bt = to_gpu(A, kind)[:, :, :K], to_gpu(B, kind)[:, :, :N]
    # bf16 operands write fp32 (bf16 rounding alone can reach 2^-8 of a result
    # whose terms share a sign); fp16 operands write fp16
    out_dt = torch.float16 if kind == "f16" else torch.float32
    okind = "f16" if kind == "f16" else "f32"
    for sched in [dict(tile=(64, 64), offset=3), dict(tile=(128, 128), offset=1, direction="nz"),
                  dict(tile=(128, 192), split_k=2, xcd_remap=1), dict(tile=(256, 128), offset=2),
                  dict(tile=(64, 64), split_k=3, direction="raster", grid=7)]:
        say("batched ragged", kind, batch, M, N, K, sched)
        eff = bst().effective_sched(0, ab, batch, M, N, K, bst().make_sched(**sched))
        assert eff.path == path
        full, C = guarded(M, N, out_dt, lead=(batch,))
        bst().batched_gemm(At, Bt, C, sched=bst().make_sched(**sched))
        check_close(orc, C.contiguous().reshape(batch * M, N), ref, den, TOL_16, str(sched))
        assert_guard(orc, full, M, N, okind)
