"""GPU tests of dynamic task allocation and block preloading (LDS-DMA kernels).

Dynamic allocation ("Block Scheduler Code Explained", s1) hands units to
workgroups from per-XCD queues instead of a static stride; preloading (the
Preload dispatch policies of "Block Dispatch Policies") issues a task's first
stages before the previous task's epilogue.  Neither changes what a unit
computes, so every result must be bit-identical to the static, non-preloaded
schedule (fp outputs included), and match the oracle.  The launches run
several units per workgroup (small grids), split-K fix-ups, all problem forms,
repeated calls on one workspace (the queue counters must be back at zero after
each call) and grouped launches in which some workgroups find no unit.
"""
import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I
from gpu_util import TOL_16, TOL_8, check_close, codes, say, to_gpu

pytestmark = pytest.mark.gpu

MODES = [dict(dynamic=1), dict(preload=1), dict(dynamic=1, preload=1)]


def bst():
    import block_swizzle_tile_amd as m
    return m


def test_flags_reported_and_need_counters(orc):
    s = bst().make_sched(tile=(64, 64), dynamic=1)
    eff = bst().effective_sched(0, bst().F16, 1, 1024, 1024, 2048, s)
    assert eff.dynamic == 1 and eff.preload == 0 and eff.path == 2
    assert bst().workspace_bytes(0, bst().F16, 1, 1024, 1024, 2048, s) == 73728
    eff = bst().effective_sched(0, bst().F16, 1, 1024, 1024, 2048,
                                bst().make_sched(tile=(64, 64), preload=1))
    assert eff.dynamic == 0 and eff.preload == 1
    # preload applies with the static stride only: with dynamic allocation the next task is
    # known only after the epilogue
    eff = bst().effective_sched(0, bst().F16, 1, 1024, 1024, 2048,
                                bst().make_sched(tile=(64, 64), dynamic=1, preload=1))
    assert eff.dynamic == 1 and eff.preload == 0
    # the register-staged family runs a static stride without preload
    s = bst().make_sched(tile=(64, 64), dynamic=1, preload=1, path=1)
    eff = bst().effective_sched(0, bst().F16, 1, 1024, 1024, 2048, s)
    assert eff.dynamic == 0 and eff.preload == 0 and eff.path == 1


@pytest.mark.parametrize("grid", [1, 7, 64, 0])
def test_fp16_identical_to_static(orc, grid):
    """fp16 1024x1024x2048 at 64x64 (256 tiles) with few workgroups: bit-identical outputs."""
    import torch
    w = I.workload("fp16_2k")
    A, B = to_gpu(w["A"], "f16"), to_gpu(w["B"], "f16")
    ref, den = orc.gemm(orc.F16, w["A"], w["B"], tile=(64, 64))
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    for tile, split, shk in [((64, 64), 1, 1), ((128, 128), 2, 0), ((256, 256), 1, 0),
                             ((128, 64), 3, 1)]:
        base = dict(tile=tile, offset=4, split_k=split, xcd_remap=1, grid=grid, shuffle_k=shk)
        C0 = bst().gemm(A, B, sched=bst().make_sched(**base), workspace=ws)
        check_close(orc, C0, ref, den, TOL_16, str(base))
        c0 = codes(C0)
        for m in MODES:
            for rep in range(2):     # twice on one workspace: counters back at zero
                say("fp16 2k", base, m, rep)
                C = bst().gemm(A, B, sched=bst().make_sched(**base, **m), workspace=ws)
                assert np.array_equal(codes(C), c0), (base, m, rep)


def test_mxfp8_identical_to_static(orc):
    w = I.workload("mxfp8_4k", small=True)
    ref, den = orc.gemm(orc.MXE4M3, w["A"], w["B"], scale_a=w["scale_a"], scale_b=w["scale_b"],
                        tile=(64, 64))
    A, B = to_gpu(w["A"], "e4m3"), to_gpu(w["B"], "e4m3")
    sa, sb = to_gpu(w["scale_a"], "u8"), to_gpu(w["scale_b"], "u8")
    for tile, split, grid in [((64, 128), 1, 5), ((128, 128), 2, 3), ((256, 256), 1, 2),
                              ((64, 64), 1, 0)]:
        base = dict(tile=tile, offset=2, split_k=split, xcd_remap=1, grid=grid)
        c0 = codes(bst().gemm(A, B, scale_a=sa, scale_b=sb, sched=bst().make_sched(**base)))
        for m in MODES:
            say("mx", base, m)
            C = bst().gemm(A, B, scale_a=sa, scale_b=sb, sched=bst().make_sched(**base, **m))
            check_close(orc, C, ref, den, TOL_8, str((base, m)))
            assert np.array_equal(codes(C), c0), (base, m)


def test_int8_grouped_slice_m(orc):
    """The int8 grouped slice-M workload (uneven groups, per-token dequant) and a grouped
    problem whose bound exceeds its task count (some workgroups find no unit)."""
    w = I.workload("int8_groups", small=True)
    gm, N, K = w["group_m"], w["N"], w["K"]
    ref, den, acc = orc.grouped_gemm(gm, w["A"], w["B"], N, K, row_scale=w["row_scale"],
                                     col_scale=w["col_scale"], tile=(64, 64))
    A, B = to_gpu(w["A"], "i8"), to_gpu(w["B"], "i8")
    gmt = to_gpu(gm, "i32")
    rs, cs = to_gpu(w["row_scale"], "f32"), to_gpu(w["col_scale"], "f32")
    for tile, split, grid in [((64, 64), 1, 9), ((128, 128), 2, 0), ((256, 256), 1, 3),
                              ((128, 128), 1, 0)]:
        base = dict(tile=tile, offset=4, split_k=split, xcd_remap=1, grid=grid)
        for m in [{}] + MODES:
            say("int8 groups", base, m)
            s = bst().make_sched(**base, **m)
            raw = bst().grouped_gemm_slice_m(A, B, gmt, sched=s)
            assert np.array_equal(codes(raw)[:acc.shape[0]], acc.astype(np.int32)), (base, m)
            out = bst().grouped_gemm_slice_m(A, B, gmt, row_scale=rs, col_scale=cs, sched=s)
            check_close(orc, out[:acc.shape[0]], ref, den, TOL_16, str((base, m)))
    # tiny groups: the host's task bound (ceil(total/tile) + G tile-rows) is far above the
    # device task count, so most of the launched workgroups have no unit at all
    gm2 = np.array([1, 0, 3, 0, 2], np.int32)
    total, N2, K2 = 16, 64, 128
    A2 = I.int8_uniform((total, K2), 71, 0)
    B2 = I.int8_uniform((len(gm2), K2, N2), 71, 1)
    _, _, acc2 = orc.grouped_gemm(gm2, A2, B2, N2, K2, tile=(64, 64))
    for m in MODES:
        for rep in range(3):
            s = bst().make_sched(tile=(64, 64), xcd_remap=1, **m)
            raw = bst().grouped_gemm_slice_m(to_gpu(A2, "i8"), to_gpu(B2, "i8"),
                                             to_gpu(gm2, "i32"), sched=s)
            assert np.array_equal(codes(raw)[:acc2.shape[0]], acc2.astype(np.int32)), (m, rep)


def test_bf16_batched_and_slice_k(orc):
    w = I.workload("bf16_batch", small=True)
    b, M, N, K = w["batch"], w["M"], w["N"], w["K"]
    A, B = to_gpu(w["A"], "bf16"), to_gpu(w["B"], "bf16")
    base = dict(tile=(64, 64), offset=3, xcd_remap=1, grid=5)
    c0 = codes(bst().batched_gemm(A, B, sched=bst().make_sched(**base)))
    for m in MODES:
        say("bf16 batch", m)
        assert np.array_equal(codes(bst().batched_gemm(A, B, sched=bst().make_sched(**base, **m))), c0)
    k = I.workload("int8_slice_k", small=True)
    _, _, acc = orc.grouped_gemm_slice_k(orc.I8, k["group_k"], k["A"], k["B"], k["M"], k["N"],
                                         tile=(64, 64))
    Ak, Bk, gk = to_gpu(k["A"], "i8"), to_gpu(k["B"], "i8"), to_gpu(k["group_k"], "i32")
    for m in MODES:
        for split in [1, 3]:
            say("slice-K", m, split)
            s = bst().make_sched(tile=(64, 64), split_k=split, xcd_remap=1, grid=6, **m)
            C = bst().grouped_gemm_slice_k(Ak, Bk, gk, sched=s)
            assert np.array_equal(codes(C).reshape(-1, k["N"]), acc.astype(np.int32)), (m, split)


def test_ragged_fp16_with_preload(orc):
    """Tails and partial stages in the preloaded prologue (the non-whole-stage DMA path)."""
    import torch
    M, N, K = 333, 200, 1000
    g = I.rng(72, 0)
    A = I.f16_bits(g.uniform(-1, 1, size=(M, K)))
    B = I.f16_bits(g.uniform(-1, 1, size=(K, N)))
    ref, den = orc.gemm(orc.F16, A, B, tile=(64, 64))
    At, Bt = to_gpu(A, "f16"), to_gpu(B, "f16")
    for tile, split in [((64, 64), 1), ((128, 128), 3), ((256, 128), 2)]:
        base = dict(tile=tile, split_k=split, grid=4, xcd_remap=1)
        c0 = codes(bst().gemm(At, Bt, sched=bst().make_sched(**base)))
        for m in MODES:
            say("ragged", base, m)
            C = bst().gemm(At, Bt, sched=bst().make_sched(**base, **m))
            check_close(orc, C, ref, den, TOL_16, str((base, m)))
            assert np.array_equal(codes(C), c0)
    torch.cuda.synchronize()
