"""GPU parity of the two-workgroups-per-CU LDS-DMA kernels (bst_sched.path = 3).

These instances (fp16 / bf16 / int8 at 128x128, plain, batched and grouped
slice-M) run two pipeline stages and two resident workgroups per CU; they
add the same products in the same order as the one-workgroup kernels
(path 2), so for random operands their results are bit-identical to path 2,
and both match the oracle.  The cases cover tails (ragged M, N, K), several
units per workgroup (small grids), split-K fix-ups, dynamic allocation and
preloading, repeated calls on one workspace, empty and short groups, and
the automatic choice of the family.
"""
import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I
from gpu_util import TOL_16, check_close, codes, say, to_gpu

pytestmark = pytest.mark.gpu


def bst():
    import block_swizzle_tile_amd as m
    return m


def _pair_and_single(call, base, what):
    """Runs call(sched) with the schedule base at path 3, then at path 2; returns both
    results."""
    s3 = bst().make_sched(**base, path=3)
    s2 = bst().make_sched(**base, path=2)
    say(what, base)
    return call(s3), call(s2)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_16bit_ragged_and_multi_unit(orc, kind):
    import torch
    M, N, K = 333, 264, 1000
    g = I.rng(81, 0 if kind == "f16" else 1)
    x, y = g.uniform(-1, 1, size=(M, K)), g.uniform(-1, 1, size=(K, N))
    A = I.f16_bits(x) if kind == "f16" else I.bf16_bits(x)
    B = I.f16_bits(y) if kind == "f16" else I.bf16_bits(y)
    ref, den = orc.gemm(orc.F16 if kind == "f16" else orc.BF16, A, B, tile=(128, 128))
    At, Bt = to_gpu(A, kind), to_gpu(B, kind)
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    for base in [dict(tile=(128, 128)), dict(tile=(128, 128), grid=2, offset=2),
                 dict(tile=(128, 128), split_k=3, xcd_remap=1),
                 dict(tile=(128, 128), grid=3, dynamic=1, xcd_remap=1),
                 dict(tile=(128, 128), grid=2, preload=1, shuffle_k=1)]:
        C3, C2 = _pair_and_single(lambda s: bst().gemm(At, Bt, sched=s, workspace=ws), base, kind)
        check_close(orc, C3, ref, den, TOL_16, str(base))
        assert np.array_equal(codes(C3), codes(C2)), base
    eff = bst().effective_sched(0, bst().F16 if kind == "f16" else bst().BF16, 1, M, N, K,
                                bst().make_sched(tile=(128, 128), path=3))
    assert eff.path == 3


def test_fp16_many_tiles_auto(orc):
    """2048x1024x512 at 128x128 (128 tiles, split 4 = 512 units): the automatic choice is path 3;
    sampled rows against the oracle, all rows against path 2."""
    import torch
    M, N, K = 2048, 1024, 512
    g = I.rng(82, 0)
    A = I.f16_bits(g.uniform(-1, 1, size=(M, K)))
    B = I.f16_bits(g.uniform(-1, 1, size=(K, N)))
    rows = np.array(sorted({0, 1, 127, 128, 1000, 1023, 1024, 2047} |
                           set(g.integers(0, M, size=24).tolist())), np.int64)
    ref, den = orc.gemm(orc.F16, A, B, tile=(128, 128), rows=rows)
    At, Bt = to_gpu(A, "f16"), to_gpu(B, "f16")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    s = bst().make_sched(tile=(128, 128), split_k=4, offset=4, xcd_remap=1)
    assert bst().effective_sched(0, bst().F16, 1, M, N, K, s).path == 3
    C = bst().gemm(At, Bt, sched=s, workspace=ws)
    check_close(orc, C[torch.as_tensor(rows, device="cuda")], ref, den, TOL_16, "auto")
    C2 = bst().gemm(At, Bt, sched=bst().make_sched(tile=(128, 128), split_k=4, offset=4,
                                                  xcd_remap=1, path=2), workspace=ws)
    assert np.array_equal(codes(C), codes(C2))


def test_int8_plain_and_quant(orc):
    """int8 raw accumulators bit-exact at path 3 (ragged, several units per workgroup, split);
    per-token dequant within 2^-9."""
    import torch
    M, N, K = 300, 272, 1040
    A = I.int8_uniform((M, K), 83, 0)
    B = I.int8_uniform((K, N), 83, 1)
    rs = I.lognormal_f32((M,), 83, 2)
    cs = I.lognormal_f32((1, N), 83, 3)
    # the oracle's dequant of a one-group problem is the per-token quant GEMM
    ref, den, acc = orc.grouped_gemm(np.array([M], np.int32), A, B, N, K, row_scale=rs,
                                     col_scale=cs, tile=(128, 128))
    At, Bt = to_gpu(A, "i8"), to_gpu(B, "i8")
    rst, cst = to_gpu(rs, "f32"), to_gpu(cs.ravel(), "f32")
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    for base in [dict(tile=(128, 128), grid=2), dict(tile=(128, 128), split_k=2, xcd_remap=1),
                 dict(tile=(128, 128), grid=1, dynamic=1)]:
        C3, C2 = _pair_and_single(
            lambda s: bst().gemm(At, Bt, out_dtype=torch.int32, sched=s, workspace=ws), base, "i8")
        assert np.array_equal(codes(C3), acc.astype(np.int32)), base
        assert np.array_equal(codes(C2), acc.astype(np.int32)), base
        Q3, Q2 = _pair_and_single(
            lambda s: bst().quant_gemm_per_token(At, Bt, rst, cst, sched=s, workspace=ws),
            base, "quant")
        assert np.array_equal(codes(Q3), codes(Q2)), base
    check_close(orc, Q3, ref, den, TOL_16, "quant per token")


def test_int8_grouped_slice_m(orc):
    """The int8 grouped workload (small: uneven groups, per-token dequant) and tiny groups, at
    path 3 with the static stride, dynamic allocation and preload; repeated calls on one
    workspace."""
    import torch
    w = I.workload("int8_groups", small=True)
    gm, N, K = w["group_m"], w["N"], w["K"]
    ref, den, acc = orc.grouped_gemm(gm, w["A"], w["B"], N, K, row_scale=w["row_scale"],
                                     col_scale=w["col_scale"], tile=(128, 128))
    A, B = to_gpu(w["A"], "i8"), to_gpu(w["B"], "i8")
    gmt = to_gpu(gm, "i32")
    rs, cs = to_gpu(w["row_scale"], "f32"), to_gpu(w["col_scale"], "f32")
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    for base in [dict(tile=(128, 128), offset=4, xcd_remap=1), dict(tile=(128, 128), grid=5),
                 dict(tile=(128, 128), grid=7, dynamic=1, xcd_remap=1),
                 dict(tile=(128, 128), grid=3, preload=1), dict(tile=(128, 128), split_k=2)]:
        for rep in range(2):
            R3, R2 = _pair_and_single(
                lambda s: bst().grouped_gemm_slice_m(A, B, gmt, sched=s, workspace=ws),
                base, "int8 groups raw")
            assert np.array_equal(codes(R3)[:acc.shape[0]], acc.astype(np.int32)), (base, rep)
            assert np.array_equal(codes(R2)[:acc.shape[0]], acc.astype(np.int32)), (base, rep)
        D3, D2 = _pair_and_single(
            lambda s: bst().grouped_gemm_slice_m(A, B, gmt, row_scale=rs, col_scale=cs, sched=s,
                                                 workspace=ws), base, "int8 groups dequant")
        check_close(orc, D3[:acc.shape[0]], ref, den, TOL_16, str(base))
        assert np.array_equal(codes(D3), codes(D2)), base
    # empty and one-row groups: most workgroups find no unit
    gm2 = np.array([1, 0, 3, 0, 2], np.int32)
    A2 = I.int8_uniform((16, 128), 84, 0)
    B2 = I.int8_uniform((len(gm2), 128, 64), 84, 1)
    _, _, acc2 = orc.grouped_gemm(gm2, A2, B2, 64, 128, tile=(128, 128))
    for m in [{}, dict(dynamic=1), dict(preload=1)]:
        raw = bst().grouped_gemm_slice_m(to_gpu(A2, "i8"), to_gpu(B2, "i8"), to_gpu(gm2, "i32"),
                                         sched=bst().make_sched(tile=(128, 128), path=3, **m),
                                         workspace=ws)
        assert np.array_equal(codes(raw)[:acc2.shape[0]], acc2.astype(np.int32)), m


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_16bit_batched_and_grouped(orc, kind):
    import torch
    w = I.workload("bf16_batch", small=True)
    b, M, N, K = w["batch"], w["M"], w["N"], w["K"]
    A = w["A"] if kind == "bf16" else I.f16_bits(I.rng(85, 0).uniform(-1, 1, size=(b, M, K)))
    B = w["B"] if kind == "bf16" else I.f16_bits(I.rng(85, 1).uniform(-1, 1, size=(b, K, N)))
    code = orc.BF16 if kind == "bf16" else orc.F16
    ref, den = orc.gemm(code, A, B, batch=b, M=M, N=N, K=K, strideA=M * K, strideB=K * N,
                        tile=(128, 128))
    At, Bt = to_gpu(A, kind), to_gpu(B, kind)
    for base in [dict(tile=(128, 128), offset=3, xcd_remap=1), dict(tile=(128, 128), grid=1),
                 dict(tile=(128, 128), grid=3, dynamic=1)]:
        C3, C2 = _pair_and_single(lambda s: bst().batched_gemm(At, Bt, sched=s), base, kind)
        check_close(orc, C3.reshape(b * M, N), ref, den, TOL_16, str(base))
        assert np.array_equal(codes(C3), codes(C2)), base
    # grouped slice-M with 16-bit operands: an empty group and a group under one tile
    gm = np.array([100, 0, 37, 260], np.int32)
    Kg, Ng = 264, 136
    g = I.rng(86, 0)
    Ag = I.f16_bits(g.uniform(-1, 1, size=(int(gm.sum()), Kg))) if kind == "f16" else \
        I.bf16_bits(g.uniform(-1, 1, size=(int(gm.sum()), Kg)))
    Bg = I.f16_bits(g.uniform(-1, 1, size=(len(gm), Kg, Ng))) if kind == "f16" else \
        I.bf16_bits(g.uniform(-1, 1, size=(len(gm), Kg, Ng)))
    # the groups are independent products stacked along M (each its own plain GEMM)
    parts, q = [], 0
    for gi, m in enumerate(gm):
        if m:
            parts.append(orc.gemm(code, Ag[q:q + m], Bg[gi], tile=(128, 128)))
        q += m
    refg = np.concatenate([r for r, _ in parts])
    deng = np.concatenate([d for _, d in parts])
    Agt, Bgt, gmt = to_gpu(Ag, kind), to_gpu(Bg, kind), to_gpu(gm, "i32")
    out_dt = torch.float32
    G3, G2 = _pair_and_single(
        lambda s: bst().grouped_gemm_slice_m(Agt, Bgt, gmt, out_dtype=out_dt, sched=s),
        dict(tile=(128, 128), grid=2), kind + " groups")
    assert np.array_equal(codes(G3), codes(G2))
    check_close(orc, G3, refg, deng, TOL_16, "16-bit groups")
    torch.cuda.synchronize()


def test_mxfp8_pair(orc):
    """MX-fp8 at 128x128 with two workgroups per CU: ragged M / N with K tails of whole 128-wide
    blocks, several units per workgroup, a split; bit-identical to path 2, within 2^-7."""
    import torch
    from gpu_util import TOL_8
    M, N, K = 300, 272, 640
    g = I.rng(87, 0)
    sa = (127 + g.integers(-2, 3, size=(M, K // 32))).astype(np.uint8)
    sb = (127 + g.integers(-2, 3, size=(K // 32, N))).astype(np.uint8)
    A = I.e4m3_bits(g.standard_normal((M, K)) * 4.0)
    B = I.e4m3_bits(g.standard_normal((K, N)) * 4.0)
    ref, den = orc.gemm(orc.MXE4M3, A, B, scale_a=sa, scale_b=sb, tile=(128, 128))
    At, Bt = to_gpu(A, "e4m3"), to_gpu(B, "e4m3")
    sat, sbt = to_gpu(sa, "u8"), to_gpu(sb, "u8")
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    for base in [dict(tile=(128, 128)), dict(tile=(128, 128), grid=2, xcd_remap=1),
                 dict(tile=(128, 128), split_k=2), dict(tile=(128, 128), grid=3, dynamic=1)]:
        C3, C2 = _pair_and_single(lambda s: bst().gemm(At, Bt, scale_a=sat, scale_b=sbt, sched=s,
                                                       workspace=ws), base, "mx")
        check_close(orc, C3, ref, den, TOL_8, str(base))
        assert np.array_equal(codes(C3), codes(C2)), base
