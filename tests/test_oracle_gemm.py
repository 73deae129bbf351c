"""Pins of the oracle's GEMM, dequant and compare against things other than
itself: exact integer brute force in pure Python on tiny shapes, closed forms
(identity, rank-1, all-ones), numpy fp64 / int64 matmul on medium shapes
(a library routine used here only), and planted errors for the compare.

Semantics pinned: C = A . B over (M, N, K) with row-major A[M][K] and
B[K][N]; batched C_b = A_b . B_b with the batch index of the task
("Block Scheduler Code Explained", s4.4); grouped slice-M (groups stacked
along M, s4.2 Update per group); MX block scales one per 32-wide K block;
dequant out = acc * s_row[i] * s_col[g][j].
"""
import itertools

import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I


def f16(x):
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def test_brute_force_tiny_exact(orc):
    """All M, N, K in 1..4 with several tiles/orders; small integer-valued
    fp16 inputs, so fp64 sums are exact; compared with Python int sums."""
    g = np.random.default_rng(7)
    for M, N, K in itertools.product(range(1, 5), repeat=3):
        a = g.integers(-8, 9, size=(M, K))
        b = g.integers(-8, 9, size=(K, N))
        want = [[sum(int(a[i, k]) * int(b[k, j]) for k in range(K)) for j in range(N)]
                for i in range(M)]
        want_den = [[sum(abs(int(a[i, k]) * int(b[k, j])) for k in range(K)) for j in range(N)]
                    for i in range(M)]
        for (tm, tn), off, d in [((1, 1), 1, "zn"), ((2, 3), 2, "nz"), ((4, 4), 1, "raster"),
                                 ((1, 2), 3, "zn")]:
            ref, den = orc.gemm(orc.F16, f16(a), f16(b), tile=(tm, tn), off=off, direction=d)
            assert ref.tolist() == want and den.tolist() == want_den


def test_closed_forms(orc):
    g = np.random.default_rng(1)
    M, K, N = 37, 37, 53
    B = f16(g.uniform(-1, 1, size=(K, N)))
    # A = I  ->  C = B exactly
    ref, _ = orc.gemm(orc.F16, f16(np.eye(M)), B, tile=(16, 16), off=2)
    assert np.array_equal(ref, orc.decode("f16", B))
    # B = [I | 0]  ->  C = A (first M columns), zeros elsewhere
    A = f16(g.uniform(-1, 1, size=(M, K)))
    Bi = np.zeros((K, N)); Bi[:, :K] = np.eye(K)
    ref, _ = orc.gemm(orc.F16, A, f16(Bi), tile=(8, 32), off=3, direction="nz")
    assert np.array_equal(ref[:, :K], orc.decode("f16", A)) and not ref[:, K:].any()
    # rank-1: A = u 1^T, B = 1 v^T  ->  C = K u v^T
    u = g.integers(-5, 6, size=M); v = g.integers(-5, 6, size=N); K2 = 64
    ref, _ = orc.gemm(orc.F16, f16(np.outer(u, np.ones(K2))), f16(np.outer(np.ones(K2), v)),
                      tile=(16, 8))
    assert np.array_equal(ref, K2 * np.outer(u, v).astype(np.float64))
    # all ones -> K
    ref, den = orc.gemm(orc.F16, f16(np.ones((5, 300))), f16(np.ones((300, 7))), tile=(4, 4))
    assert np.all(ref == 300) and np.all(den == 300)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_numpy_fp64_medium(orc, dtype):
    M, N, K = 67, 45, 129
    if dtype == "f16":
        A, B, code = I.uniform_f16((M, K), 99, 0), I.uniform_f16((K, N), 99, 1), orc.F16
    else:
        A, B, code = I.uniform_bf16((M, K), 99, 0), I.uniform_bf16((K, N), 99, 1), orc.BF16
    a, b = orc.decode(dtype, A), orc.decode(dtype, B)
    ref, den = orc.gemm(code, A, B, tile=(32, 16), off=2, direction="zn")
    assert np.allclose(ref, a @ b, rtol=0, atol=1e-12)
    assert np.allclose(den, np.abs(a) @ np.abs(b), rtol=1e-14, atol=0)


def test_strided_operands(orc):
    """lda > K and ldb > N: only the leading K / N columns take part."""
    M, N, K, lda, ldb = 20, 12, 24, 40, 16
    A = I.uniform_f16((M, lda), 98, 0); B = I.uniform_f16((K, ldb), 98, 1)
    a = orc.decode("f16", A)[:, :K]; b = orc.decode("f16", B)[:, :N]
    ref, _ = orc.gemm(orc.F16, A, B, M=M, N=N, K=K, lda=lda, ldb=ldb, tile=(8, 8))
    assert np.allclose(ref, a @ b, rtol=0, atol=1e-12)


def test_batched_vs_numpy(orc):
    batch, M, N, K = 3, 33, 20, 48
    A = I.normal_bf16((batch, M, K), 97, 0); B = I.normal_bf16((batch, K, N), 97, 1)
    ref, den = orc.gemm(orc.BF16, A, B, batch=batch, M=M, N=N, K=K, strideA=M * K,
                        strideB=K * N, tile=(16, 16), off=2)
    a = orc.decode("bf16", A); b = orc.decode("bf16", B)
    want = np.concatenate([a[i] @ b[i] for i in range(batch)])
    assert np.allclose(ref, want, rtol=0, atol=1e-15)
    # a row subset returns the same rows
    rows = [0, 40, 98, 5]
    r2, d2 = orc.gemm(orc.BF16, A, B, batch=batch, M=M, N=N, K=K, strideA=M * K,
                      strideB=K * N, tile=(16, 16), off=2, rows=rows)
    assert np.array_equal(r2, ref[rows]) and np.array_equal(d2, den[rows])


def test_int8_vs_numpy_int64(orc):
    M, N, K = 50, 70, 300
    A = I.int8_uniform((M, K), 96, 0); B = I.int8_uniform((K, N), 96, 1)
    ref, den, acc = orc.gemm(orc.I8, A, B, tile=(32, 32), off=2, direction="nz", want_acc=True)
    want = A.astype(np.int64) @ B.astype(np.int64)
    assert np.array_equal(acc, want) and np.array_equal(ref, want.astype(np.float64))
    assert np.array_equal(den, np.abs(A.astype(np.int64)) @ np.abs(B.astype(np.int64)))


def test_mx_e4m3_vs_expanded_scales(orc):
    """MX: sum over blocks of 2^(sa-127) 2^(sb-127) sum_block a b equals the
    plain product of the operands with their block scales expanded."""
    M, N, K = 24, 40, 256
    A, sa = I.mx_a(M, K, 95, 0)
    B, sb = I.mx_b(K, N, 95, 1)
    a = orc.decode("e4m3", A) * np.repeat(orc.decode("e8m0", sa), 32, axis=1)
    b = orc.decode("e4m3", B) * np.repeat(orc.decode("e8m0", sb), 32, axis=0)
    ref, den = orc.gemm(orc.MXE4M3, A, B, scale_a=sa, scale_b=sb, tile=(16, 16), off=2)
    assert np.allclose(ref, a @ b, rtol=1e-13, atol=1e-12)
    assert np.allclose(den, np.abs(a) @ np.abs(b), rtol=1e-13, atol=0)
    # with every scale 2^0 it is the plain e4m3 product
    ones_a = np.full_like(sa, 127); ones_b = np.full_like(sb, 127)
    r1, _ = orc.gemm(orc.MXE4M3, A, B, scale_a=ones_a, scale_b=ones_b, tile=(8, 8))
    r2, _ = orc.gemm(orc.E4M3, A, B, tile=(8, 8))
    assert np.allclose(r1, orc.decode("e4m3", A) @ orc.decode("e4m3", B), rtol=1e-13, atol=1e-12)
    assert np.array_equal(r1, r2)


def test_mx_rejects_unaligned_k(orc):
    A = np.zeros((4, 40), np.uint8); B = np.zeros((40, 4), np.uint8)
    with pytest.raises(ValueError):
        orc.gemm(orc.MXE4M3, A, B, scale_a=np.zeros((4, 1), np.uint8),
                 scale_b=np.zeros((1, 4), np.uint8))


def test_grouped_dequant_vs_numpy(orc):
    gm = np.array([70, 0, 129, 3, 64], np.int32)
    total, N, K = int(gm.sum()) + 11, 96, 160   # spare rows after the last group
    A = I.int8_uniform((total, K), 94, 0); B = I.int8_uniform((len(gm), K, N), 94, 1)
    rs = I.lognormal_f32((total,), 94, 2); cs = I.lognormal_f32((len(gm), N), 94, 3)
    ref, den, acc = orc.grouped_gemm(gm, A, B, N, K, row_scale=rs, col_scale=cs,
                                     tile=(64, 32), off=2, direction="zn")
    r0 = 0
    for g, Mg in enumerate(gm):
        a = A[r0:r0 + Mg].astype(np.int64); b = B[g].astype(np.int64)
        want = a @ b
        assert np.array_equal(acc[r0:r0 + Mg], want)
        scale = rs[r0:r0 + Mg, None].astype(np.float64) * cs[g][None, :].astype(np.float64)
        assert np.allclose(ref[r0:r0 + Mg], want * scale, rtol=1e-15, atol=0)
        assert np.allclose(den[r0:r0 + Mg], (np.abs(a) @ np.abs(b)) * np.abs(scale), rtol=1e-15)
        r0 += Mg
    assert acc.shape[0] == int(gm.sum())
    # raw mode (no scales): ref is the accumulator itself
    ref2, _, acc2 = orc.grouped_gemm(gm, A, B, N, K, tile=(32, 32), rows=[0, 75, 201])
    assert np.array_equal(acc2, acc[[0, 75, 201]]) and np.array_equal(ref2, acc2.astype(np.float64))


def test_k_zero_gives_zero(orc):
    ref, den = orc.gemm(orc.F16, np.zeros((5, 0), np.uint16), np.zeros((0, 6), np.uint16),
                        M=5, N=6, K=0, tile=(2, 2))
    assert not ref.any() and not den.any()


def test_compare_detects_planted_errors(orc):
    g = np.random.default_rng(3)
    ref = g.normal(size=1000); den = np.abs(ref) + 1.0
    e, am = orc.compare(ref.copy(), ref, den)
    assert e == 0.0 and am == -1
    got = ref.copy(); got[417] += 0.01 * den[417]
    e, am = orc.compare(got, ref, den)
    assert am == 417 and abs(e - 0.01) < 1e-12
    got = ref.copy(); got[3] = np.nan
    assert orc.compare(got, ref, den) == (np.inf, 3)
    den0 = den.copy(); den0[10] = 0.0
    z = ref.copy(); z[10] = 0.0
    assert orc.compare(z, ref, den0)[0] == 0.0
    z[10] = 1e-30
    assert orc.compare(z, ref, den0) == (np.inf, 10)
