"""GPU parity of the MX-fp8 kernels' A-scale groups.

Whole MX tasks of the four-stage LDS-DMA kernels load A's e8m0 block scales
four stages at a time (16 bytes per row into one of two group slots) instead
of four bytes per row and stage.  These cases run that scheme with block
scales that differ from row to row and block to block (so a stage that read
another group's or another row's scales would be off by a power of two),
over ragged M, split-K slices that start on and off a group boundary,
ShuffleK, dynamic allocation and preloading, and compare with the oracle
(2^-7 of sum |a*b|); where the two-workgroup kernel (which loads the scales
per stage) runs the same products in the same order, the two outputs must be
bit-identical.
"""
import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I
from gpu_util import TOL_8, check_close, codes, say, to_gpu

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    g = np.random.default_rng(seed)
    A = I.e4m3_bits(g.standard_normal((M, K)))
    B = I.e4m3_bits(g.standard_normal((K, N)))
    sa = (120 + g.integers(0, 15, size=(M, K // 32))).astype(np.uint8)
    sb = (120 + g.integers(0, 15, size=(K // 32, N))).astype(np.uint8)
    return A, B, sa, sb


@pytest.mark.parametrize("tile", [(64, 128), (64, 64), (128, 64), (128, 128)])
def test_scale_groups_against_oracle(orc, tile):
    import torch
    import block_swizzle_tile_amd as bst
    M, N, K = 200, 256, 2048
    A, B, sa, sb = _operands(M, N, K, 700 + tile[0] + tile[1])
    ref, den = orc.gemm(orc.MXE4M3, A, B, scale_a=sa, scale_b=sb, tile=tile)
    At, Bt = to_gpu(A, "e4m3"), to_gpu(B, "e4m3")
    sat, sbt = to_gpu(sa, "u8"), to_gpu(sb, "u8")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    for kw in (dict(), dict(shuffle_k=1), dict(split_k=2), dict(split_k=3), dict(split_k=4),
               dict(split_k=3, shuffle_k=1), dict(dynamic=1), dict(preload=1),
               dict(grid=7, shuffle_k=1)):
        s = bst.make_sched(tile=tile, offset=3, direction="zn", xcd_remap=1, path=2, **kw)
        say("mx groups", tile, kw)
        C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        bst.gemm(At, Bt, C, scale_a=sat, scale_b=sbt, sched=s, workspace=ws)
        torch.cuda.synchronize()
        check_close(orc, C, ref, den, TOL_8, "%s %s" % (tile, kw))


def test_scale_groups_match_per_stage_scales():
    """128x128: the four-stage kernel (scale groups) and the two-workgroup kernel
    (per-stage scales) add the same products in the same order."""
    import torch
    import block_swizzle_tile_amd as bst
    M, N, K = 328, 512, 4096
    A, B, sa, sb = _operands(M, N, K, 711)
    At, Bt = to_gpu(A, "e4m3"), to_gpu(B, "e4m3")
    sat, sbt = to_gpu(sa, "u8"), to_gpu(sb, "u8")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    for kw in (dict(), dict(split_k=2), dict(split_k=3), dict(dynamic=1)):
        out = []
        for path in (2, 3):
            s = bst.make_sched(tile=(128, 128), offset=4, direction="zn", xcd_remap=1, path=path,
                               **kw)
            say("mx groups vs per-stage", path, kw)
            C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
            bst.gemm(At, Bt, C, scale_a=sat, scale_b=sbt, sched=s, workspace=ws)
            torch.cuda.synchronize()
            out.append(codes(C))
        assert np.array_equal(out[0], out[1]), kw
