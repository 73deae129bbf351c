"""Pins of the oracle's grouped slice-K product (orc_grouped_gemm_slice_k).

Reading ("Block Dispatch Policies" names the grouped-matmul-slice-K example
and its per-token-dequant variant): K is cut into G consecutive groups;
group g multiplies A[:, Q_g : Q_g + k_g] by B[Q_g : Q_g + k_g, :] into its own
M x N output (stacked as rows g*M + i); its tasks are numbered like the
batches of a batched problem (s4.4 GetBatchIdx).

The pins do not reuse the oracle's arithmetic: brute force in exact Python
integers on tiny shapes, numpy's int64 / float64 matmul per group, the
identity that the groups' outputs sum to the plain product over the whole K
range, closed forms (all-ones operands, one-element groups as outer
products, empty groups as zeros), dequant with power-of-two scales (exact
in fp64), and the argument checks.  A wrong group offset, a dropped or
extra K index, a transposed operand or a wrong scale index fails at least
one of them.
"""
import itertools

import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I


def brute(gk, A, B, M, N):
    """Per-group products in exact Python integers."""
    out, q = [], 0
    for k in gk:
        C = [[0] * N for _ in range(M)]
        for i in range(M):
            for j in range(N):
                C[i][j] = sum(int(A[i][q + kk]) * int(B[q + kk][j]) for kk in range(k))
        out.extend(C)
        q += k
    return np.array(out, dtype=np.int64).reshape(len(gk) * M, N)


def test_brute_force_tiny(orc):
    g = np.random.default_rng(1)
    cases = 0
    for G, M, N in itertools.product([1, 2, 3], [1, 3, 5], [1, 2, 4]):
        gk = g.integers(0, 5, size=G).astype(np.int32)
        K = int(gk.sum()) + int(g.integers(0, 3))          # spare columns are never read
        A = g.integers(-128, 128, size=(M, max(K, 1))).astype(np.int8)
        B = g.integers(-128, 128, size=(max(K, 1), N)).astype(np.int8)
        for tile, off, d in [((1, 1), 1, "zn"), ((2, 3), 2, "nz"), ((4, 4), 1, "raster")]:
            ref, den, acc = orc.grouped_gemm_slice_k(orc.I8, gk, A, B, M, N,
                                                     total_k=max(K, 1), tile=tile, off=off,
                                                     direction=d)
            want = brute(gk.tolist(), A.tolist(), B.tolist(), M, N)
            assert np.array_equal(acc, want), (G, M, N, gk, tile)
            assert np.array_equal(ref, want.astype(np.float64))
            absw = brute(gk.tolist(), np.abs(A.astype(np.int64)).tolist(),
                         np.abs(B.astype(np.int64)).tolist(), M, N)
            assert np.array_equal(den, absw.astype(np.float64))
            cases += 1
    assert cases == 81


def test_per_group_numpy_and_sum_identity(orc):
    g = np.random.default_rng(2)
    gk = np.array([48, 0, 160, 16, 1, 77], np.int32)
    M, N, K = 70, 90, int(gk.sum()) + 5
    A = g.integers(-127, 128, size=(M, K)).astype(np.int8)
    B = g.integers(-127, 128, size=(K, N)).astype(np.int8)
    _, _, acc = orc.grouped_gemm_slice_k(orc.I8, gk, A, B, M, N, total_k=K, tile=(32, 64),
                                         off=2)
    q = np.concatenate([[0], np.cumsum(gk)])
    A64, B64 = A.astype(np.int64), B.astype(np.int64)
    for i, k in enumerate(gk):
        want = A64[:, q[i]:q[i + 1]] @ B64[q[i]:q[i + 1]]
        assert np.array_equal(acc[i * M:(i + 1) * M], want), i
    # the groups partition K: their outputs sum to the product over all of it
    total = acc.reshape(len(gk), M, N).sum(axis=0)
    assert np.array_equal(total, A64[:, :q[-1]] @ B64[:q[-1]])


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_16bit_groups_match_numpy(orc, kind):
    g = np.random.default_rng(3)
    gk = np.array([64, 8, 0, 200], np.int32)
    M, N, K = 33, 40, int(gk.sum())
    x, y = g.uniform(-1, 1, size=(M, K)), g.uniform(-1, 1, size=(K, N))
    A = I.f16_bits(x) if kind == "f16" else I.bf16_bits(x)
    B = I.f16_bits(y) if kind == "f16" else I.bf16_bits(y)
    code = orc.F16 if kind == "f16" else orc.BF16
    ref, den, _ = orc.grouped_gemm_slice_k(code, gk, A, B, M, N, tile=(16, 16), off=3)
    Ad, Bd = orc.decode(kind, A), orc.decode(kind, B)
    q = np.concatenate([[0], np.cumsum(gk)])
    for i in range(len(gk)):
        want = Ad[:, q[i]:q[i + 1]] @ Bd[q[i]:q[i + 1]]
        wden = np.abs(Ad[:, q[i]:q[i + 1]]) @ np.abs(Bd[q[i]:q[i + 1]])
        got, gden = ref[i * M:(i + 1) * M], den[i * M:(i + 1) * M]
        # products of two 16-bit values are exact in fp64; only the summation
        # order differs from numpy's
        assert np.all(np.abs(got - want) <= 1e-12 * np.maximum(wden, 1e-300)), i
        assert np.allclose(gden, wden, rtol=1e-12, atol=0), i


def test_closed_forms(orc):
    gk = np.array([5, 0, 1, 12], np.int32)
    M, N, K = 9, 11, 18
    ones_a = np.ones((M, K), np.int8)
    ones_b = np.ones((K, N), np.int8)
    _, _, acc = orc.grouped_gemm_slice_k(orc.I8, gk, ones_a, ones_b, M, N, tile=(4, 8))
    for i, k in enumerate(gk):
        assert np.all(acc[i * M:(i + 1) * M] == k)      # all-ones: each output is k_g
    g = np.random.default_rng(4)
    A = g.integers(-9, 10, size=(M, K)).astype(np.int8)
    B = g.integers(-9, 10, size=(K, N)).astype(np.int8)
    ref, den, acc = orc.grouped_gemm_slice_k(orc.I8, gk, A, B, M, N, tile=(8, 8))
    # the empty group is all zeros, den included; the one-element group (K index 5) is the
    # outer product of A's column 5 and B's row 5
    assert np.all(acc[M:2 * M] == 0) and np.all(den[M:2 * M] == 0)
    assert np.array_equal(acc[2 * M:3 * M], np.outer(A[:, 5].astype(np.int64), B[5].astype(np.int64)))


def test_dequant_scales(orc):
    g = np.random.default_rng(5)
    gk = np.array([32, 16, 48], np.int32)
    M, N, K = 20, 24, 96
    A = g.integers(-127, 128, size=(M, K)).astype(np.int8)
    B = g.integers(-127, 128, size=(K, N)).astype(np.int8)
    # powers of two: the products are exact in fp64
    rs = np.exp2(g.integers(-6, 7, size=(3, M))).astype(np.float32)
    cs = np.exp2(g.integers(-6, 7, size=(3, N))).astype(np.float32)
    ref, den, acc = orc.grouped_gemm_slice_k(orc.I8, gk, A, B, M, N, row_scale=rs, col_scale=cs,
                                             tile=(16, 16))
    _, den0, acc0 = orc.grouped_gemm_slice_k(orc.I8, gk, A, B, M, N, tile=(16, 16))
    assert np.array_equal(acc, acc0)
    want = acc0.reshape(3, M, N) * rs[:, :, None] * cs[:, None, :]
    assert np.array_equal(ref, want.reshape(3 * M, N))
    wden = den0.reshape(3, M, N) * rs[:, :, None] * cs[:, None, :]
    assert np.array_equal(den, wden.reshape(3 * M, N))
    # a scale index that ignored the group would differ here: the groups' scales differ
    assert not np.array_equal(rs[0], rs[1]) and not np.array_equal(cs[0], cs[2])


def test_row_selection_and_order_invariance(orc):
    g = np.random.default_rng(6)
    gk = np.array([40, 24], np.int32)
    M, N = 50, 30
    A = g.integers(-127, 128, size=(M, 64)).astype(np.int8)
    B = g.integers(-127, 128, size=(64, N)).astype(np.int8)
    full = orc.grouped_gemm_slice_k(orc.I8, gk, A, B, M, N, tile=(16, 16))[2]
    rows = np.array([0, 17, 49, 50, 77, 99])
    part = orc.grouped_gemm_slice_k(orc.I8, gk, A, B, M, N, tile=(32, 8), off=2,
                                    direction="nz", rows=rows)[2]
    assert np.array_equal(part, full[rows])


def test_rejects_bad_arguments(orc):
    A = np.zeros((4, 8), np.int8)
    B = np.zeros((8, 4), np.int8)
    with pytest.raises(ValueError):
        orc.grouped_gemm_slice_k(orc.I8, np.array([4, -1], np.int32), A, B, 4, 4, total_k=8)
    with pytest.raises(ValueError):
        orc.grouped_gemm_slice_k(orc.I8, np.array([4, 5], np.int32), A, B, 4, 4, total_k=8)
    with pytest.raises(ValueError):   # scales with 16-bit operands
        orc.grouped_gemm_slice_k(orc.F16, np.array([8], np.int32), A.view(np.uint8), B, 4, 4,
                                 row_scale=np.ones((1, 4), np.float32),
                                 col_scale=np.ones((1, 4), np.float32))
