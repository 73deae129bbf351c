"""GPU parity of the grouped slice-K GEMM (bst_grouped_gemm_slice_k).

K is cut into consecutive groups; group g multiplies A[:, Q_g:Q_g+k_g] by
B[Q_g:Q_g+k_g, :] into its own output ("Block Dispatch Policies", grouped
slice-K examples, read so).  int8 raw int32 accumulators are bit-exact
against the oracle; dequantised and 16-bit outputs meet 2^-9 of
sum |a*b| (times the scales).  Outputs sit in NaN guard bands.
"""
import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I
from gpu_util import TOL_16, check_close, check_close_rounded, codes, say, to_gpu

pytestmark = pytest.mark.gpu


def bst():
    import block_swizzle_tile_amd as m
    return m


def take(t, rows):
    import torch
    return t[torch.as_tensor(rows, device=t.device)]


def guarded(G, M, N, dtype):
    """[G][M + 2][ldc] buffer filled with a guard value; the [G][M][N] view at row 1."""
    import torch
    ldc = -(-N // 8) * 8 + 8
    fill = float("nan") if dtype.is_floating_point else -7
    full = torch.full((G, M + 2, ldc), fill, dtype=dtype, device="cuda")
    return full, full[:, 1:M + 1, :N]


def assert_guard(full, M, N):
    import torch
    c = full.float().cpu()
    guard = torch.isnan(c) if full.dtype.is_floating_point else (c == -7)
    assert bool(guard[:, 0].all()) and bool(guard[:, M + 1].all()), "guard rows written"
    assert bool(guard[:, 1:M + 1, N:].all()), "guard columns written"


def test_int8_slice_k_small_full(orc):
    """The small int8 workload (4 groups of K, 128 x 256 outputs) in full: raw int32 bit-exact,
    dequant within 2^-9, over tiles, splits, both kernel families and orders."""
    import torch
    w = I.workload("int8_slice_k", small=True)
    gk, M, N = w["group_k"], w["M"], w["N"]
    ref, den, acc = orc.grouped_gemm_slice_k(orc.I8, gk, w["A"], w["B"], M, N,
                                             row_scale=w["row_scale"], col_scale=w["col_scale"],
                                             tile=(64, 64))
    A, B = to_gpu(w["A"], "i8"), to_gpu(w["B"], "i8")
    gkt = to_gpu(gk, "i32")
    rs, cs = to_gpu(w["row_scale"], "f32"), to_gpu(w["col_scale"], "f32")
    G = len(gk)
    for sched in [dict(tile=(64, 64)), dict(tile=(128, 128), offset=2, direction="nz"),
                  dict(tile=(256, 128), split_k=2, xcd_remap=1), dict(tile=(256, 256), split_k=3),
                  dict(tile=(128, 128), path=1), dict(tile=(256, 256), path=1, split_k=2),
                  dict(tile=(64, 64), path=2, split_k=4, shuffle_k=1),
                  dict(tile=(128, 128), split_k=0, grid=7)]:
        say("slice-K small", sched)
        s = bst().make_sched(**sched)
        full, C = guarded(G, M, N, torch.int32)
        bst().grouped_gemm_slice_k(A, B, gkt, C, sched=s)
        assert np.array_equal(codes(C.contiguous()).reshape(G * M, N), acc.astype(np.int32)), sched
        assert_guard(full, M, N)
        full, C = guarded(G, M, N, torch.float32)
        bst().grouped_gemm_slice_k(A, B, gkt, C, row_scale=rs, col_scale=cs, sched=s)
        check_close(orc, C.contiguous().reshape(G * M, N), ref, den, TOL_16, str(sched))
        assert_guard(full, M, N)
        full, C = guarded(G, M, N, torch.bfloat16)
        bst().grouped_gemm_slice_k(A, B, gkt, C, row_scale=rs, col_scale=cs, sched=s)
        check_close_rounded(orc, C.contiguous().reshape(G * M, N), ref, den, TOL_16, 2.0 ** -8,
                            str(sched))
        assert_guard(full, M, N)


def test_int8_slice_k_workload(orc):
    """The int8 slice-K workload (8 groups cutting K = 8192, one of them under 128, 1024 x 2048
    outputs, per-token dequant), sampled rows of every group."""
    w = I.workload("int8_slice_k")
    gk, M, N = w["group_k"], w["M"], w["N"]
    G = len(gk)
    g = np.random.default_rng(8)
    rows = sorted({int(x) for x in g.integers(0, G * M, size=40)} |
                  {gi * M + r for gi in range(G) for r in (0, M - 1)})
    rows = np.array(rows, np.int64)
    say("oracle slice-K on", len(rows), "rows")
    ref, den, acc = orc.grouped_gemm_slice_k(orc.I8, gk, w["A"], w["B"], M, N,
                                             row_scale=w["row_scale"], col_scale=w["col_scale"],
                                             tile=(256, 256), rows=rows)
    A, B = to_gpu(w["A"], "i8"), to_gpu(w["B"], "i8")
    gkt = to_gpu(gk, "i32")
    rs, cs = to_gpu(w["row_scale"], "f32"), to_gpu(w["col_scale"], "f32")
    import torch
    for sched in [dict(tile=(256, 256), offset=1), dict(tile=(128, 128), offset=4, xcd_remap=1),
                  dict(tile=(256, 128), offset=2, xcd_remap=1, split_k=2)]:
        say("slice-K workload", sched)
        s = bst().make_sched(**sched)
        raw = bst().grouped_gemm_slice_k(A, B, gkt, sched=s)
        assert np.array_equal(codes(take(raw.reshape(G * M, N), rows)), acc.astype(np.int32)), sched
        # the dequant arithmetic at fp32 output: 2^-9 of sum |a*b| * scales
        out = bst().grouped_gemm_slice_k(A, B, gkt, row_scale=rs, col_scale=cs,
                                         out_dtype=torch.float32, sched=s)
        check_close(orc, take(out.reshape(G * M, N), rows), ref, den, TOL_16, str(sched))
        # bf16 output: groups of 16 and 32 K values give short sums whose |ref| nears den, where
        # bf16's own rounding (2^-8 |ref|) is more than 2^-9 den; it is allowed on top
        out = bst().grouped_gemm_slice_k(A, B, gkt, row_scale=rs, col_scale=cs, sched=s)
        check_close_rounded(orc, take(out.reshape(G * M, N), rows), ref, den, TOL_16, 2.0 ** -8,
                            str(sched))


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_16bit_slice_k_ragged(orc, kind):
    """fp16 / bf16 slice-K with ragged M and N, an empty group and spare K columns."""
    import torch
    gk = np.array([64, 0, 200, 8, 136], np.int32)
    M, N, K = 129, 264, int(gk.sum()) + 24
    g = I.rng(61, 0)
    x, y = g.uniform(-1, 1, size=(M, K)), g.uniform(-1, 1, size=(K, N))
    A = I.f16_bits(x) if kind == "f16" else I.bf16_bits(x)
    B = I.f16_bits(y) if kind == "f16" else I.bf16_bits(y)
    code = orc.F16 if kind == "f16" else orc.BF16
    ref, den, _ = orc.grouped_gemm_slice_k(code, gk, A, B, M, N, total_k=K, tile=(64, 64))
    At, Bt, gkt = to_gpu(A, kind), to_gpu(B, kind), to_gpu(gk, "i32")
    G = len(gk)
    # bf16 operands write fp32 (bf16 rounding alone can reach 2^-8 of a short sum)
    out_dt = torch.float16 if kind == "f16" else torch.float32
    for sched in [dict(tile=(64, 64), offset=3), dict(tile=(128, 128), split_k=3, xcd_remap=1),
                  dict(tile=(256, 128), direction="nz", offset=2), dict(tile=(128, 128), path=1),
                  dict(tile=(64, 64), path=1, split_k=2)]:
        say("slice-K", kind, sched)
        full, C = guarded(G, M, N, out_dt)
        bst().grouped_gemm_slice_k(At, Bt, gkt, C, sched=bst().make_sched(**sched))
        check_close(orc, C.contiguous().reshape(G * M, N), ref, den, TOL_16, str(sched))
        assert_guard(full, M, N)
        # the empty group's output is zeros
        assert bool((C[1] == 0).all())


def test_group_sizes_cut_to_total_k(orc):
    """Sizes past the allocation are cut (the last group ends at total_k, later groups are
    empty) and negative sizes count as 0: the result equals the oracle's on the cut sizes."""
    import torch
    K, M, N = 256, 64, 96
    gk = np.array([64, -5, 160, 128, 32], np.int32)       # 64 + 160 = 224; 128 is cut to 32
    cut = np.array([64, 0, 160, 32, 0], np.int32)
    A = I.int8_uniform((M, K), 62, 0)
    B = I.int8_uniform((K, N), 62, 1)
    _, _, acc = orc.grouped_gemm_slice_k(orc.I8, cut, A, B, M, N, total_k=K, tile=(64, 64))
    for sched in [dict(tile=(64, 64)), dict(tile=(128, 128), path=1, split_k=2)]:
        C = bst().grouped_gemm_slice_k(to_gpu(A, "i8"), to_gpu(B, "i8"), to_gpu(gk, "i32"),
                                       sched=bst().make_sched(**sched))
        assert np.array_equal(codes(C).reshape(-1, N), acc.astype(np.int32)), sched
    torch.cuda.synchronize()


def test_unaligned_groups(orc):
    """Group sizes that break A's 16-byte chunks: the register-staged kernels compute every
    group; the LDS-DMA kernels compute the groups that start and end on a chunk and write NaN
    (INT32_MIN raw) for the others, as the header documents."""
    import torch
    gk = np.array([48, 24, 64, 16], np.int32)   # int8 chunks: 16; group 1 ends off a chunk,
    M, N = 96, 80                               # so groups 1, 2 and 3 start off one
    K = int(gk.sum())                           # 152: A's rows padded to 160 bytes
    A = I.int8_uniform((M, 160), 63, 0)
    B = I.int8_uniform((K, N), 63, 1)
    rs = I.lognormal_f32((len(gk), M), 63, 2)
    cs = I.lognormal_f32((len(gk), N), 63, 3)
    ref, den, acc = orc.grouped_gemm_slice_k(orc.I8, gk, A, B, M, N, total_k=K, lda=160,
                                             row_scale=rs, col_scale=cs, tile=(64, 64))
    At, Bt, gkt = to_gpu(A, "i8")[:, :K], to_gpu(B, "i8"), to_gpu(gk, "i32")
    rst, cst = to_gpu(rs, "f32"), to_gpu(cs, "f32")
    for sched in [dict(tile=(64, 64), path=1), dict(tile=(128, 128), path=1, split_k=2)]:
        say("unaligned slice-K register", sched)
        s = bst().make_sched(**sched)
        C = bst().grouped_gemm_slice_k(At, Bt, gkt, sched=s)
        assert np.array_equal(codes(C).reshape(-1, N), acc.astype(np.int32)), sched
        C = bst().grouped_gemm_slice_k(At, Bt, gkt, row_scale=rst, col_scale=cst,
                                       out_dtype=torch.float32, sched=s)
        check_close(orc, C.reshape(-1, N), ref, den, TOL_16, str(sched))
    say("unaligned slice-K dma")
    s = bst().make_sched(tile=(64, 64), path=2)
    C = codes(bst().grouped_gemm_slice_k(At, Bt, gkt, sched=s))
    assert np.array_equal(C[0], acc[:M].astype(np.int32))
    assert np.all(C[1:] == np.int32(-2 ** 31))
    Cd = bst().grouped_gemm_slice_k(At, Bt, gkt, row_scale=rst, col_scale=cst,
                                    out_dtype=torch.float32, sched=s)
    check_close(orc, Cd[0], ref[:M], den[:M], TOL_16, "aligned group on the DMA kernels")
    assert bool(torch.isnan(Cd[1:].float()).all())
