"""Seeded random parity sweep over shapes, operand types and schedules.

Each case draws a problem (M, N, K up to a few hundred, K tails and ragged
M / N included), an operand type (fp16, bf16, e4m3, MX-fp8, int8), a tile
the library builds, and every schedule knob (swizzle offset and direction,
split-K, XCD remap, grid, kernel family, ShuffleK, dynamic allocation,
preload), runs the GEMM once and compares it with the oracle: int8 raw
accumulators bit-exact, 16-bit outputs within 2^-9 and 8-bit within 2^-7 of
sum |a*b| (bf16 outputs of short K sums also get their own rounding, up to
2^-8 of the result, as the slice-K tests do).  The tiles and kernel families are drawn among those the library
builds for the drawn problem, so every case runs.  The cases are fixed by
the seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I
from gpu_util import TOL_8, TOL_16, check_close, check_close_rounded, codes, say, to_gpu

pytestmark = pytest.mark.gpu

# the tiles the library builds per operand type (both kernel families), and the 128x128 ones that
# also come with two workgroups per CU
TILES = {"f16": [(64, 64), (128, 128), (256, 128), (128, 256), (128, 192), (128, 64), (64, 128),
                 (256, 256)],
         "i8": [(64, 64), (128, 128), (256, 128), (256, 256)],
         "e4m3": [(64, 64), (128, 128), (256, 128), (256, 256), (128, 64), (64, 128)],
         "mx": [(64, 64), (128, 128), (256, 128), (256, 256), (128, 64), (64, 128)]}
TILES["bf16"] = TILES["f16"]
KINDS = ["f16", "bf16", "e4m3", "mx", "i8"]


def _case(g):
    kind = KINDS[int(g.integers(len(KINDS)))]
    # rows of whole 16-byte chunks (the layout bst_gemm takes; the tiles' M / N / K tails are
    # still ragged); MX K in blocks of 32
    q = 16 if kind in ("e4m3", "mx", "i8") else 8
    M = int(g.integers(1, 320))
    N = int(g.integers(1, 320 // q + 1)) * q
    K = int(g.integers(1, 20)) * (32 if kind == "mx" else q)
    tile = TILES[kind][int(g.integers(len(TILES[kind])))]
    paths = [0, 0, 1]
    if kind != "mx" or K % 128 == 0:          # the LDS-DMA family takes MX K in blocks of 128
        paths += [2] + ([3] if tile == (128, 128) and kind != "e4m3" else [])
    sched = dict(tile=tile,
                 offset=int(g.integers(1, 9)),
                 direction=["zn", "nz", "raster"][int(g.integers(3))],
                 split_k=int(g.choice([1, 1, 2, 3, 0])),
                 xcd_remap=int(g.integers(2)),
                 grid=int(g.choice([0, 0, 1, 3, 7])),
                 path=int(g.choice(paths)),
                 shuffle_k=int(g.integers(2)),
                 dynamic=int(g.integers(2)),
                 preload=int(g.integers(2)))
    return kind, M, N, K, sched


def _operands(kind, M, N, K, g):
    if kind == "i8":
        return (g.integers(-127, 128, size=(M, K)).astype(np.int8),
                g.integers(-127, 128, size=(K, N)).astype(np.int8), None, None)
    if kind in ("e4m3", "mx"):
        A = I.e4m3_bits(g.standard_normal((M, K)) * 8.0)
        B = I.e4m3_bits(g.standard_normal((K, N)) * 8.0)
        if kind == "e4m3":
            return A, B, None, None
        sa = (127 + g.integers(-2, 3, size=(M, K // 32))).astype(np.uint8)
        sb = (127 + g.integers(-2, 3, size=(K // 32, N))).astype(np.uint8)
        return A, B, sa, sb
    x, y = g.uniform(-1, 1, size=(M, K)), g.uniform(-1, 1, size=(K, N))
    if kind == "f16":
        return I.f16_bits(x), I.f16_bits(y), None, None
    return I.bf16_bits(x), I.bf16_bits(y), None, None


def test_random_schedules(orc):
    import torch
    import block_swizzle_tile_amd as bst
    g = np.random.default_rng(20261202)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    ran = 0
    for case in range(200):
        kind, M, N, K, sched = _case(g)
        A, B, sa, sb = _operands(kind, M, N, K, g)
        code = {"f16": orc.F16, "bf16": orc.BF16, "e4m3": orc.E4M3, "mx": orc.MXE4M3,
                "i8": orc.I8}[kind]
        gk = {"mx": "e4m3", "e4m3": "e4m3"}.get(kind, kind)
        At, Bt = to_gpu(A, gk), to_gpu(B, gk)
        kw = {}
        if kind == "mx":
            kw = dict(scale_a=to_gpu(sa, "u8"), scale_b=to_gpu(sb, "u8"))
        say("case", case, kind, (M, N, K), sched)
        C = bst.gemm(At, Bt, sched=bst.make_sched(**sched), workspace=ws, **kw)
        ran += 1
        if kind == "i8":
            _, _, acc = orc.gemm(code, A, B, tile=sched["tile"], want_acc=True)
            assert np.array_equal(codes(C), acc.astype(np.int32)), (case, kind, M, N, K, sched)
        else:
            ref, den = orc.gemm(code, A, B, scale_a=sa, scale_b=sb, tile=sched["tile"])
            what = str((case, kind, M, N, K, sched))
            if kind == "bf16":
                # short K sums can come close to sum |a*b|, and then bf16's own rounding of
                # the result (up to 2^-8 of it) exceeds 2^-9 of that sum: allowed on top
                check_close_rounded(orc, C, ref, den, TOL_16, 2.0 ** -8, what)
            else:
                check_close(orc, C, ref, den, TOL_16 if kind == "f16" else TOL_8, what)
    say("random schedules: ran", ran)
    assert ran == 200
    torch.cuda.synchronize()
