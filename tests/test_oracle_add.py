"""Pins of the oracle's matmul-add, C = A . B + X (the matmul-add example that
"Block Dispatch Policies" lists under its ping-pong policy; reading: X has C's
shape and type): closed forms with all-ones operands, a zero left operand (the
result is the addend, exactly), exact cancellation, the error scale, and an
integer brute force on tiny shapes."""
import itertools

import numpy as np


def f16(x):
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def test_all_ones_plus_constant(orc):
    # A . B = K everywhere; X = 0.5  ->  K + 0.5, scale K + 0.5
    M, N, K = 9, 13, 300
    X = f16(np.full((M, N), 0.5))
    ref, den = orc.gemm_add(orc.F16, f16(np.ones((M, K))), f16(np.ones((K, N))), X, "f16",
                            tile=(4, 8))
    assert np.all(ref == K + 0.5) and np.all(den == K + 0.5)


def test_zero_left_operand_gives_the_addend(orc):
    g = np.random.default_rng(3)
    M, N, K = 17, 23, 40
    X = f16(g.uniform(-4, 4, size=(M, N)))
    ref, den = orc.gemm_add(orc.F16, f16(np.zeros((M, K))), f16(g.uniform(-1, 1, (K, N))), X,
                            "f16", tile=(8, 8), off=2, direction="nz")
    x = orc.decode("f16", X)
    assert np.array_equal(ref, x) and np.array_equal(den, np.abs(x))


def test_cancellation_and_scale(orc):
    # A . B = K, X = -K  ->  exactly 0 with scale 2K (the compare then needs got == 0 only
    # to within 2K times the tolerance)
    M, N, K = 5, 6, 2048
    ref, den = orc.gemm_add(orc.F16, f16(np.ones((M, K))), f16(np.ones((K, N))),
                            f16(np.full((M, N), -K)), "f16", tile=(4, 4))
    assert not ref.any() and np.all(den == 2 * K)


def test_brute_force_tiny_int8_with_int32_addend(orc):
    """int8 operands with an int32 addend (the raw-accumulator output): Python integer sums."""
    g = np.random.default_rng(11)
    for M, N, K in itertools.product((1, 2, 3), (1, 3), (1, 2, 5)):
        a = g.integers(-127, 128, size=(M, K)).astype(np.int8)
        b = g.integers(-127, 128, size=(K, N)).astype(np.int8)
        x = g.integers(-2**20, 2**20, size=(M, N)).astype(np.int32)
        want = [[sum(int(a[i, k]) * int(b[k, j]) for k in range(K)) + int(x[i, j])
                 for j in range(N)] for i in range(M)]
        ref, den = orc.gemm_add(orc.I8, a, b, x, "i32", tile=(2, 2))
        assert ref.tolist() == want
        assert den.tolist() == [[sum(abs(int(a[i, k]) * int(b[k, j])) for k in range(K)) +
                                 abs(int(x[i, j])) for j in range(N)] for i in range(M)]


def test_selected_rows(orc):
    g = np.random.default_rng(5)
    M, N, K = 40, 24, 64
    A, B = f16(g.uniform(-1, 1, (M, K))), f16(g.uniform(-1, 1, (K, N)))
    X = f16(g.uniform(-1, 1, (M, N)))
    rows = np.array([0, 7, 39])
    full, fden = orc.gemm_add(orc.F16, A, B, X, "f16", tile=(16, 8))
    part, pden = orc.gemm_add(orc.F16, A, B, X[rows], "f16", tile=(16, 8), rows=rows)
    assert np.array_equal(part, full[rows]) and np.array_equal(pden, fden[rows])
