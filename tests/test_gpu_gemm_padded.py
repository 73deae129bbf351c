"""GPU parity of the padding GEMM (bst_gemm_padded): operands with odd row strides
and element-aligned (not 16-byte aligned) bases are repacked into the workspace and
multiplied; checked against the oracle reading the caller's original layout.  int8
raw int32 outputs are bit-exact."""
import numpy as np
import pytest

from gpu_util import TOL_16, check_close, codes, say, to_gpu

pytestmark = pytest.mark.gpu


def bst():
    import block_swizzle_tile_amd as m
    return m


def _f16(g, shape):
    return g.uniform(-1, 1, shape).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("M,N,K", [(200, 136, 250), (256, 256, 256), (33, 17, 9)])
@pytest.mark.parametrize("sched", [dict(tile=(64, 64)), dict(tile=(128, 128), split_k=2)])
def test_fp16_odd_strides_and_bases(orc, M, N, K, sched):
    import torch
    g = np.random.default_rng(M + N + K)
    Af = _f16(g, (M, K + 3))          # lda = K + 3 elements, base one element in
    Bf = _f16(g, (K, N + 5))          # ldb = N + 5, base two elements in
    ref, den = orc.gemm(orc.F16, Af.ravel()[1:], Bf.ravel()[2:], M=M, N=N, K=K, lda=K + 3,
                        ldb=N + 5)
    A = to_gpu(Af, "f16")[:, 1:K + 1]
    B = to_gpu(Bf, "f16")[:, 2:N + 2]
    assert A.data_ptr() % 16 != 0 and B.data_ptr() % 16 != 0
    say("padded fp16", M, N, K, sched)
    # C keeps whole 16-byte rows (only the operands are repacked)
    C = torch.empty((M, -(-N // 8) * 8), dtype=torch.float16, device="cuda")[:, :N]
    bst().gemm_padded(A, B, C, sched=bst().make_sched(**sched))
    check_close(orc, C, ref, den, TOL_16, str(sched))
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["f16", "i8"])
def test_padded_k_runs_lds_dma(orc, kind):
    """K = 250 is not a whole number of 16-byte chunks: the padding GEMM pads K
    too (zero columns of A meet zero rows of B), so with N aligned it runs the
    LDS-DMA kernels; results match the oracle on the caller's layout (int8
    bit-exact)."""
    import torch
    M, N, K = 200, 256, 250
    g = np.random.default_rng(31)
    ab = bst().F16 if kind == "f16" else bst().I8
    if kind == "f16":
        Af, Bf = _f16(g, (M, K + 3)), _f16(g, (K, N + 1))
    else:
        Af = g.integers(-127, 128, (M, K + 3)).astype(np.int8)
        Bf = g.integers(-127, 128, (K, N + 1)).astype(np.int8)
    code = orc.F16 if kind == "f16" else orc.I8
    res = orc.gemm(code, Af, Bf, M=M, N=N, K=K, lda=K + 3, ldb=N + 1, want_acc=kind == "i8")
    A, B = to_gpu(Af, kind)[:, :K], to_gpu(Bf, kind)[:, :N]
    for sched in [dict(tile=(64, 64)), dict(tile=(128, 128), split_k=2, xcd_remap=1)]:
        s = bst().make_sched(**sched)
        assert bst().effective_sched(2, ab, 1, M, N, K, s).path == 2
        say("padded K", kind, sched)
        C = bst().gemm_padded(A, B, sched=s)
        if kind == "f16":
            check_close(orc, C, res[0], res[1], TOL_16, str(sched))
        else:
            assert np.array_equal(codes(C).astype(np.int64), res[2]), sched
    torch.cuda.synchronize()


def test_int8_odd_stride_bit_exact(orc):
    import torch
    M, N, K = 160, 96, 300
    g = np.random.default_rng(21)
    Af = g.integers(-127, 128, (M, K + 1)).astype(np.int8)
    Bf = g.integers(-127, 128, (K, N + 3)).astype(np.int8)
    ref, _ = orc.gemm(orc.I8, Af.ravel()[1:], Bf.ravel()[3:], M=M, N=N, K=K, lda=K + 1,
                      ldb=N + 3)
    A = to_gpu(Af, "i8")[:, 1:K + 1]
    B = to_gpu(Bf, "i8")[:, 3:N + 3]
    for sched in [dict(tile=(64, 64)), dict(tile=(128, 128), split_k=3)]:
        C = bst().gemm_padded(A, B, sched=bst().make_sched(**sched))
        assert np.array_equal(codes(C).astype(np.int64), ref.astype(np.int64)), sched
    torch.cuda.synchronize()


def test_shared_workspace_keeps_split_counters_zero(orc):
    """A padded split-K call, then plain split-K calls on the same stream's cached workspace:
    the repacked operands never land on the split-K counter area."""
    import torch
    g = np.random.default_rng(5)
    M, N, K = 256, 256, 512
    Af, Bf = _f16(g, (M, K + 1)), _f16(g, (K, N + 1))
    refp, denp = orc.gemm(orc.F16, Af, Bf, M=M, N=N, K=K, lda=K + 1, ldb=N + 1)
    A2, B2 = _f16(g, (M, K)), _f16(g, (K, N))
    ref2, den2 = orc.gemm(orc.F16, A2, B2)
    s = bst().make_sched(tile=(128, 128), split_k=4)
    for _ in range(2):
        Cp = bst().gemm_padded(to_gpu(Af, "f16")[:, :K], to_gpu(Bf, "f16")[:, :N], sched=s)
        C2 = bst().gemm(to_gpu(A2, "f16"), to_gpu(B2, "f16"), sched=s)
        check_close(orc, Cp, refp, denp, TOL_16, "padded")
        check_close(orc, C2, ref2, den2, TOL_16, "plain after padded")
    torch.cuda.synchronize()
