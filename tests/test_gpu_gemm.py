"""GPU parity of every GEMM form against the CPU oracle.

Floating outputs: max |gpu - oracle| / sum_k |a_ik b_kj| <= 2^-9 (fp16 /
bf16 outputs) or 2^-7 (fp8 / MX-fp8); int8 raw int32 accumulators and the
map are bit-exact.  Inputs come from block_swizzle_tile_amd.inputs (seeded);
the oracle computes from the same host bytes.  Large workloads are checked
on a sample of whole rows that covers every tile-row and the tails.
"""
import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I
from gpu_util import TOL_16, TOL_8, check_close, codes, say, to_gpu

pytestmark = pytest.mark.gpu


def bst():
    import block_swizzle_tile_amd as m
    return m


def take(t, rows):
    import torch
    return t[torch.as_tensor(rows, device=t.device)]


@pytest.fixture(scope="module")
def fp16_2k(orc):
    w = I.workload("fp16_2k")
    say("oracle fp16 2k ...")
    ref, den = orc.gemm(orc.F16, w["A"], w["B"], tile=(256, 128))
    return w, ref, den


def sample_rows(total, tile_m, n=48, seed=0):
    """Rows covering every tile-row start / end, the last row, plus random ones."""
    g = np.random.default_rng(seed)
    s = set()
    for r0 in range(0, total, tile_m):
        s.update({r0, min(r0 + tile_m, total) - 1})
    s.update(g.integers(0, total, size=n).tolist())
    s.add(total - 1)
    return np.array(sorted(x for x in s if 0 <= x < total), np.int64)


# ------------------------------------------------------------------ fp16 ---
def test_tails_workload_fp16(orc):
    """200x136x256 fp16, tile 64x64, Zn, offset 3 (non-multiple tails)."""
    w = I.workload("tails")
    A, B = to_gpu(w["A"], "f16"), to_gpu(w["B"], "f16")
    ref, den = orc.gemm(orc.F16, w["A"], w["B"], tile=w["tile"], off=3, direction="zn")
    for sched in [dict(tile=(64, 64), offset=3, direction="zn"),
                  dict(tile=(64, 64), offset=1, direction="nz", xcd_remap=1),
                  dict(tile=(128, 128), offset=2, direction="raster"),
                  dict(tile=(64, 64), offset=3, direction="zn", split_k=2),
                  dict(tile=(128, 192), offset=1, direction="zn", split_k=4, grid=5),
                  dict(tile=(256, 128), offset=3, direction="nz", grid=1),
                  dict(tile=(64, 64), offset=3, direction="zn", path=1),
                  dict(tile=(64, 64), offset=3, direction="zn", path=2),
                  dict(tile=(128, 128), offset=2, split_k=3, path=2, xcd_remap=1)]:
        say("tails", sched)
        C = bst().gemm(A, B, sched=bst().make_sched(**sched))
        check_close(orc, C, ref, den, TOL_16, str(sched))


def _padded(g, rows, cols, ld, kind):
    """Row-major matrix with ld > cols whose padding holds huge values (a read
    of the padding would show up in the result)."""
    x = np.full((rows, ld), 60000.0 if kind == "f16" else 1e30)
    x[:, :cols] = g.uniform(-1, 1, size=(rows, cols))
    return I.f16_bits(x) if kind == "f16" else I.bf16_bits(x)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 9, 13), (65, 130, 200), (300, 17, 72),
                                   (129, 257, 1000), (64, 64, 64), (33, 8, 520),
                                   (256, 256, 200), (512, 384, 136)])
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_ragged_shapes(orc, M, N, K, kind):
    g = np.random.default_rng(M * 1000 + N * 10 + K)
    lda, ldb, ldc = -(-K // 8) * 8 + 8, -(-N // 8) * 8 + 8, -(-N // 8) * 8 + 8
    A = _padded(g, M, K, lda, kind)
    B = _padded(g, K, N, ldb, kind)
    code = orc.F16 if kind == "f16" else orc.BF16
    ref, den = orc.gemm(code, A, B, M=M, N=N, K=K, lda=lda, ldb=ldb, tile=(64, 64))
    import torch
    At, Bt = to_gpu(A, kind)[:, :K], to_gpu(B, kind)[:, :N]
    # bf16 inputs write fp32 here: with K this small |ref| can equal den, and
    # bf16 rounding alone is then up to 2^-8 of the result (fp16: 2^-11).
    out_dt = torch.float16 if kind == "f16" else torch.float32
    okind = "f16" if kind == "f16" else "f32"
    for tile in [(64, 64), (128, 128), (256, 128), (128, 64), (64, 128), (256, 256)]:
        for split in [1, 3]:
            say("ragged", kind, M, N, K, tile, split)
            Cfull = torch.full((M + 2, ldc), float("nan"), dtype=out_dt, device="cuda")
            C = Cfull[1:M + 1, :N]
            bst().gemm(At, Bt, C, sched=bst().make_sched(tile=tile, offset=2, split_k=split))
            check_close(orc, C, ref, den, TOL_16, "%s %s" % (tile, split))
            # guard band: nothing outside the M x N result was written
            cf = codes(Cfull)
            assert np.all(np.isnan(orc.decode(okind, cf[0]))) and np.all(np.isnan(orc.decode(okind, cf[M + 1])))
            assert np.all(np.isnan(orc.decode(okind, cf[1:M + 1, N:])))


def test_k_zero_and_empty(orc):
    import torch
    A = torch.zeros((5, 0), dtype=torch.float16, device="cuda")
    B = torch.zeros((0, 7), dtype=torch.float16, device="cuda")
    C = torch.full((5, 8), 3.0, dtype=torch.float16, device="cuda")[:, :7]
    bst().gemm(A, B, C)
    assert torch.all(C == 0)
    Z = torch.zeros((0, 16), dtype=torch.float16, device="cuda")
    out = bst().gemm(Z, torch.zeros((16, 8), dtype=torch.float16, device="cuda"))
    assert out.shape == (0, 8)


@pytest.mark.parametrize("sched", [
    dict(tile=(256, 128), offset=o, direction=d) for o in (1, 2, 4, 8) for d in ("zn", "nz")
] + [dict(tile=(128, 128), offset=2, split_k=4), dict(tile=(256, 128), offset=1, split_k=8,
                                                       xcd_remap=1),
     dict(tile=(128, 128), offset=1, split_k=0, xcd_remap=1),
     dict(tile=(128, 128), offset=2, split_k=4, path=1),
     dict(tile=(256, 128), offset=4, direction="nz", path=1),
     dict(tile=(128, 256), offset=2, split_k=2, path=2),
     dict(tile=(64, 64), offset=8, path=2, xcd_remap=1),
     dict(tile=(256, 256), offset=2, xcd_remap=1),
     dict(tile=(128, 192), offset=1, path=2),
     dict(tile=(64, 64), offset=8, xcd_remap=1, shuffle_k=1),
     dict(tile=(128, 128), offset=2, split_k=2, shuffle_k=1),
     dict(tile=(256, 256), offset=4, shuffle_k=1)])
def test_fp16_2k_workload(orc, fp16_2k, sched):
    """1024x1024x2048 fp16, every swizzle setting at 256x128 plus split-K forms and
    the tiles whose epilogue stages a whole tile in several passes."""
    w, ref, den = fp16_2k
    say("fp16 2k", sched)
    C = bst().gemm(to_gpu(w["A"], "f16"), to_gpu(w["B"], "f16"),
                   sched=bst().make_sched(**sched))
    check_close(orc, C, ref, den, TOL_16, str(sched))


# ----------------------------------------------------------------- bf16 ---
def test_bf16_batch_workload(orc):
    """16 x 512x768x1024 bf16, contiguous batches, sampled rows of every batch."""
    w = I.workload("bf16_batch")
    b, M, N, K = w["batch"], w["M"], w["N"], w["K"]
    rows = sample_rows(b * M, 128, n=64, seed=4)
    ref, den = orc.gemm(orc.BF16, w["A"], w["B"], batch=b, M=M, N=N, K=K, strideA=M * K,
                        strideB=K * N, tile=w["tile"], rows=rows)
    A, B = to_gpu(w["A"], "bf16"), to_gpu(w["B"], "bf16")
    for sched in [dict(tile=(128, 192), offset=1), dict(tile=(256, 128), offset=2, direction="nz"),
                  dict(tile=(128, 128), offset=4, xcd_remap=1), dict(tile=(128, 192), path=1)]:
        say("bf16 batch", sched)
        C = bst().batched_gemm(A, B, sched=bst().make_sched(**sched))
        check_close(orc, take(C.reshape(b * M, N), rows), ref, den, TOL_16, str(sched))


def test_bf16_batch_small_full(orc):
    w = I.workload("bf16_batch", small=True)
    b, M, N, K = w["batch"], w["M"], w["N"], w["K"]
    ref, den = orc.gemm(orc.BF16, w["A"], w["B"], batch=b, M=M, N=N, K=K, strideA=M * K,
                        strideB=K * N, tile=(64, 64))
    C = bst().batched_gemm(to_gpu(w["A"], "bf16"), to_gpu(w["B"], "bf16"),
                           sched=bst().make_sched(tile=(64, 64), offset=3, split_k=2))
    check_close(orc, C.reshape(b * M, N), ref, den, TOL_16)


# ----------------------------------------------------------------- fp8 -----
def test_mxfp8_small_full(orc):
    w = I.workload("mxfp8_4k", small=True)
    ref, den = orc.gemm(orc.MXE4M3, w["A"], w["B"], scale_a=w["scale_a"], scale_b=w["scale_b"],
                        tile=(128, 128))
    A, B = to_gpu(w["A"], "e4m3"), to_gpu(w["B"], "e4m3")
    sa, sb = to_gpu(w["scale_a"], "u8"), to_gpu(w["scale_b"], "u8")
    for sched in [dict(tile=(128, 128)), dict(tile=(256, 256), offset=4),
                  dict(tile=(64, 64), offset=2, direction="nz", split_k=2),
                  dict(tile=(128, 128), path=1), dict(tile=(256, 128), path=1, split_k=2),
                  dict(tile=(256, 128), path=2, offset=3), dict(tile=(64, 64), path=2),
                  dict(tile=(128, 64), offset=2), dict(tile=(64, 128), split_k=2, xcd_remap=1),
                  dict(tile=(64, 128), offset=2, xcd_remap=1, shuffle_k=1),
                  dict(tile=(256, 256), offset=4, shuffle_k=1)]:
        say("mxfp8 small", sched)
        C = bst().gemm(A, B, scale_a=sa, scale_b=sb, sched=bst().make_sched(**sched))
        check_close(orc, C, ref, den, TOL_8, str(sched))


def test_plain_e4m3_small(orc):
    w = I.workload("mxfp8_4k", small=True)
    ref, den = orc.gemm(orc.E4M3, w["A"], w["B"], tile=(128, 128))
    C = bst().gemm(to_gpu(w["A"], "e4m3"), to_gpu(w["B"], "e4m3"),
                   sched=bst().make_sched(tile=(128, 128)))
    check_close(orc, C, ref, den, TOL_8)


def test_mxfp8_workload(orc):
    """1024x2048x4096 MX-fp8, tile 256x256, Zn offset 4, sampled rows."""
    w = I.workload("mxfp8_4k")
    rows = sample_rows(w["M"], 128, n=40, seed=3)
    ref, den = orc.gemm(orc.MXE4M3, w["A"], w["B"], scale_a=w["scale_a"], scale_b=w["scale_b"],
                        tile=(256, 256), off=4, rows=rows)
    A, B = to_gpu(w["A"], "e4m3"), to_gpu(w["B"], "e4m3")
    sa, sb = to_gpu(w["scale_a"], "u8"), to_gpu(w["scale_b"], "u8")
    for sched in [dict(tile=(256, 256), offset=4), dict(tile=(128, 128), offset=2, split_k=2),
                  dict(tile=(256, 128), offset=1, split_k=0, xcd_remap=1),
                  dict(tile=(128, 64), offset=8, xcd_remap=1),
                  dict(tile=(64, 128), offset=8, xcd_remap=1)]:
        say("mxfp8", sched)
        C = bst().gemm(A, B, scale_a=sa, scale_b=sb, sched=bst().make_sched(**sched))
        check_close(orc, take(C, rows), ref, den, TOL_8, str(sched))


# ----------------------------------------------------------------- int8 ----
def test_int8_groups_small_full(orc):
    w = I.workload("int8_groups", small=True)
    gm, N, K = w["group_m"], w["N"], w["K"]
    ref, den, acc = orc.grouped_gemm(gm, w["A"], w["B"], N, K, row_scale=w["row_scale"],
                                     col_scale=w["col_scale"], tile=(64, 64))
    A, B = to_gpu(w["A"], "i8"), to_gpu(w["B"], "i8")
    gmt = to_gpu(gm, "i32")
    rs, cs = to_gpu(w["row_scale"], "f32"), to_gpu(w["col_scale"], "f32")
    for sched in [dict(tile=(64, 64)), dict(tile=(128, 128), offset=2, direction="nz"),
                  dict(tile=(256, 256), offset=1, split_k=2), dict(tile=(256, 128), xcd_remap=1),
                  dict(tile=(128, 128), path=1), dict(tile=(256, 256), path=1, offset=2),
                  dict(tile=(64, 64), path=2, split_k=2), dict(tile=(256, 256), path=2),
                  dict(tile=(256, 256), offset=1, shuffle_k=1)]:
        say("int8 groups small", sched)
        s = bst().make_sched(**sched)
        raw = bst().grouped_gemm_slice_m(A, B, gmt, sched=s)
        assert np.array_equal(codes(raw)[:acc.shape[0]], acc.astype(np.int32)), sched
        out = bst().grouped_gemm_slice_m(A, B, gmt, row_scale=rs, col_scale=cs, sched=s)
        check_close(orc, out[:acc.shape[0]], ref, den, TOL_16, str(sched))


def test_int8_groups_workload(orc):
    """8 groups (some < 128 rows), K 2048, N 4096, per-token dequant, sampled rows."""
    w = I.workload("int8_groups")
    gm, N, K = w["group_m"], w["N"], w["K"]
    rows = sample_rows(int(gm.sum()), 256, n=24, seed=5)
    starts = np.concatenate([[0], np.cumsum(gm)])
    rows = np.array(sorted(set(rows.tolist()) | set(int(x) for x in starts[:-1]) |
                           set(int(x) - 1 for x in starts[1:])), np.int64)
    say("oracle int8 groups on", len(rows), "rows")
    ref, den, acc = orc.grouped_gemm(gm, w["A"], w["B"], N, K, row_scale=w["row_scale"],
                                     col_scale=w["col_scale"], tile=(256, 256), rows=rows)
    A, B = to_gpu(w["A"], "i8"), to_gpu(w["B"], "i8")
    gmt = to_gpu(gm, "i32")
    rs, cs = to_gpu(w["row_scale"], "f32"), to_gpu(w["col_scale"], "f32")
    for sched in [dict(tile=(256, 256), offset=1), dict(tile=(256, 128), offset=2, xcd_remap=1)]:
        say("int8 groups", sched)
        s = bst().make_sched(**sched)
        raw = bst().grouped_gemm_slice_m(A, B, gmt, sched=s)
        assert np.array_equal(codes(raw)[rows], acc.astype(np.int32)), sched
        out = bst().grouped_gemm_slice_m(A, B, gmt, row_scale=rs, col_scale=cs, sched=s)
        check_close(orc, take(out, rows), ref, den, TOL_16, str(sched))


def test_grouped_edge_cases(orc):
    """Empty groups, groups smaller than a tile, one-row groups, spare rows."""
    g = np.random.default_rng(11)
    gm = np.array([0, 1, 300, 0, 0, 127, 129, 5, 0], np.int32)
    total, N, K = int(gm.sum()) + 9, 144, 96
    A = I.int8_uniform((total, K), 77, 0); B = I.int8_uniform((len(gm), K, N), 77, 1)
    _, _, acc = orc.grouped_gemm(gm, A, B, N, K, tile=(64, 64))
    import torch
    for tile in [(64, 64), (128, 128), (256, 256)]:
        say("grouped edges", tile)
        C = torch.full((total, N), -7, dtype=torch.int32, device="cuda")
        bst().grouped_gemm_slice_m(to_gpu(A, "i8"), to_gpu(B, "i8"), to_gpu(gm, "i32"), C,
                                   sched=bst().make_sched(tile=tile, offset=2))
        c = codes(C)
        assert np.array_equal(c[:acc.shape[0]], acc.astype(np.int32))
        assert np.all(c[acc.shape[0]:] == -7)     # rows after the last group untouched
    # f16 grouped (no scales)
    Af = I.uniform_f16((total, K), 78, 0); Bf = I.uniform_f16((len(gm), K, N), 78, 1)
    gmo = gm.copy()
    ref = np.concatenate([orc.gemm(orc.F16, Af[r0:r0 + m], Bf[i], M=int(m), N=N, K=K,
                                   tile=(32, 32))[0]
                          for i, (r0, m) in enumerate(zip(np.concatenate([[0], np.cumsum(gmo)[:-1]]), gmo))])
    den = np.concatenate([orc.gemm(orc.F16, Af[r0:r0 + m], Bf[i], M=int(m), N=N, K=K,
                                   tile=(32, 32))[1]
                          for i, (r0, m) in enumerate(zip(np.concatenate([[0], np.cumsum(gmo)[:-1]]), gmo))])
    C = bst().grouped_gemm_slice_m(to_gpu(Af, "f16"), to_gpu(Bf, "f16"), to_gpu(gm, "i32"),
                                   sched=bst().make_sched(tile=(128, 128)))
    check_close(orc, C[:ref.shape[0]], ref, den, TOL_16, "f16 grouped")


def test_quant_gemm_per_token(orc):
    M, N, K = 333, 528, 384
    A = I.int8_uniform((M, K), 66, 0); B = I.int8_uniform((K, N), 66, 1)
    rs = I.lognormal_f32((M,), 66, 2); cs = I.lognormal_f32((1, N), 66, 3)
    ref, den, acc = orc.grouped_gemm(np.array([M], np.int32), A, B, N, K, row_scale=rs,
                                     col_scale=cs, tile=(128, 128))
    At, Bt = to_gpu(A, "i8"), to_gpu(B, "i8")
    rst, cst = to_gpu(rs, "f32"), to_gpu(cs.ravel(), "f32")
    import torch
    for sched in [dict(tile=(128, 128)), dict(tile=(256, 256), split_k=3, offset=2),
                  dict(tile=(128, 128), path=1), dict(tile=(256, 128), path=2, split_k=2)]:
        say("quant per token", sched)
        s = bst().make_sched(**sched)
        out = bst().quant_gemm_per_token(At, Bt, rst, cst, sched=s)
        check_close(orc, out, ref, den, TOL_16, str(sched))
        raw = bst().quant_gemm_per_token(At, Bt, rst, cst, out_dtype=torch.int32, sched=s)
        assert np.array_equal(codes(raw), acc.astype(np.int32))


def test_int8_extremes_exact(orc):
    """All -128 operands: |acc| = K * 16384, the largest int32 sums, exact."""
    M, N, K = 64, 64, 4096
    A = np.full((M, K), -128, np.int8); B = np.full((K, N), -128, np.int8)
    C = bst().gemm(to_gpu(A, "i8"), to_gpu(B, "i8"), sched=bst().make_sched(tile=(64, 64),
                                                                             split_k=4))
    assert np.all(codes(C) == K * 16384)


def test_determinism_and_split_invariance(orc):
    """Repeated calls are bit-identical; int8 results do not depend on split
    or order at all, and fp16 integer-valued products are exact."""
    g = np.random.default_rng(2)
    M, N, K = 256, 384, 1024
    A = I.int8_uniform((M, K), 55, 0); B = I.int8_uniform((K, N), 55, 1)
    At, Bt = to_gpu(A, "i8"), to_gpu(B, "i8")
    base = codes(bst().gemm(At, Bt, sched=bst().make_sched(tile=(128, 128))))
    for s in [dict(tile=(64, 64), split_k=8), dict(tile=(256, 256), direction="nz", offset=3),
              dict(tile=(256, 128), split_k=2, xcd_remap=1), dict(tile=(128, 128), path=1),
              dict(tile=(128, 128), path=2), dict(tile=(256, 256), path=1, split_k=3)]:
        assert np.array_equal(codes(bst().gemm(At, Bt, sched=bst().make_sched(**s))), base)
    Ai = I.f16_bits(g.integers(-4, 5, size=(M, K)).astype(np.float64))
    Bi = I.f16_bits(g.integers(-4, 5, size=(K, N)).astype(np.float64))
    want = (orc.decode("f16", Ai) @ orc.decode("f16", Bi))
    import torch
    for s in [dict(tile=(128, 128), split_k=4), dict(tile=(256, 128), offset=4)]:
        C = bst().gemm(to_gpu(Ai, "f16"), to_gpu(Bi, "f16"), out_dtype=torch.float32,
                       sched=bst().make_sched(**s))
        assert np.array_equal(codes(C).astype(np.float64), want)
    s = bst().make_sched(tile=(128, 128), split_k=4)
    C1 = codes(bst().gemm(to_gpu(Ai, "f16"), to_gpu(Bi, "f16"), sched=s))
    for _ in range(5):
        assert np.array_equal(codes(bst().gemm(to_gpu(Ai, "f16"), to_gpu(Bi, "f16"), sched=s)), C1)
