"""GPU parity of the matmul-add entry point, C = A . B + X (bst_gemm_add), against the
oracle's gemm_add: the same tolerances as the plain GEMM, with the error scale
sum_k |a_ik b_kj| + |x_ij|; int8 raw int32 outputs with an int32 addend are bit-exact.
The addends are seeded like the operands (block_swizzle_tile_amd.inputs)."""
import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I
from gpu_util import TOL_16, TOL_8, check_close, codes, say, to_gpu

pytestmark = pytest.mark.gpu

X_STREAM = 7  # tensor id of the addends in the seeded generators


def bst():
    import block_swizzle_tile_amd as m
    return m


def take(t, rows):
    import torch
    return t[torch.as_tensor(rows, device=t.device)]


@pytest.mark.parametrize("sched", [dict(tile=(64, 64), offset=8, xcd_remap=1, shuffle_k=1),
                                   dict(tile=(128, 128), offset=2, split_k=2),
                                   dict(tile=(64, 64), offset=3, direction="nz")])
def test_fp16_2k_add(orc, sched):
    w = I.workload("fp16_2k")
    M, N = w["M"], w["N"]
    X = I.uniform_f16((M, N), I.WORKLOAD_IDS["fp16_2k"], X_STREAM, -4.0, 4.0)
    rows = np.array(sorted({0, 63, 64, 511, 512, 1000, 1023} | set(range(120, 136))), np.int64)
    ref, den = orc.gemm_add(orc.F16, w["A"], w["B"], X[rows], "f16", rows=rows)
    say("fp16 2k add", sched)
    C = bst().gemm(to_gpu(w["A"], "f16"), to_gpu(w["B"], "f16"), add=to_gpu(X, "f16"),
                   sched=bst().make_sched(**sched))
    check_close(orc, take(C, rows), ref, den, TOL_16, str(sched))


def test_in_place_accumulate(orc):
    """X may be C itself: C += A . B, run twice (the second adds onto the first)."""
    import torch
    M, N, K = 256, 192, 320
    A = I.uniform_f16((M, K), 9, 0)
    B = I.uniform_f16((K, N), 9, 1)
    X = I.uniform_f16((M, N), 9, X_STREAM)
    Cg = to_gpu(X, "f16").clone()
    s = bst().make_sched(tile=(64, 64), offset=2)
    bst().gemm(to_gpu(A, "f16"), to_gpu(B, "f16"), Cg, add=Cg, sched=s)
    ref, den = orc.gemm_add(orc.F16, A, B, X, "f16")
    check_close(orc, Cg, ref, den, TOL_16, "once")
    C1 = codes(Cg).copy()
    bst().gemm(to_gpu(A, "f16"), to_gpu(B, "f16"), Cg, add=Cg, sched=s)
    ref2, den2 = orc.gemm_add(orc.F16, A, B, C1, "f16")
    check_close(orc, Cg, ref2, den2, TOL_16, "twice")
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K", [(129, 136, 200), (64, 64, 64), (300, 40, 72), (1, 8, 8)])
def test_ragged_add_guard_band(orc, M, N, K):
    """Tails in M, N and K; nothing outside the M x N result is written."""
    import torch
    g = np.random.default_rng(M + 7 * N + 11 * K)
    ldc = N + 8
    A = I.f16_bits(g.uniform(-1, 1, (M, K)))
    B = I.f16_bits(g.uniform(-1, 1, (K, N)))
    X = I.f16_bits(g.uniform(-2, 2, (M, N)))
    ref, den = orc.gemm_add(orc.F16, A, B, X, "f16")
    for tile in [(64, 64), (128, 128)]:
        for split in [1, 3]:
            say("ragged add", M, N, K, tile, split)
            Cfull = torch.full((M + 2, ldc), float("nan"), dtype=torch.float16, device="cuda")
            C = Cfull[1:M + 1, :N]
            bst().gemm(to_gpu(A, "f16"), to_gpu(B, "f16"), C, add=to_gpu(X, "f16"),
                       sched=bst().make_sched(tile=tile, offset=2, split_k=split))
            check_close(orc, C, ref, den, TOL_16, "%s %s" % (tile, split))
            cf = codes(Cfull)
            assert np.all(np.isnan(orc.decode("f16", cf[0])))
            assert np.all(np.isnan(orc.decode("f16", cf[M + 1])))
            assert np.all(np.isnan(orc.decode("f16", cf[1:M + 1, N:])))


def test_bf16_with_f32_output(orc):
    import torch
    M, N, K = 192, 256, 384
    A = I.uniform_bf16((M, K), 10, 0)
    B = I.uniform_bf16((K, N), 10, 1)
    Xf = np.random.default_rng(10).uniform(-3, 3, (M, N)).astype(np.float32)
    ref, den = orc.gemm_add(orc.BF16, A, B, Xf.view(np.uint32), "f32")
    for sched in [dict(tile=(128, 128)), dict(tile=(64, 64), split_k=2)]:
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        bst().gemm(to_gpu(A, "bf16"), to_gpu(B, "bf16"), C,
                   add=torch.from_numpy(Xf).cuda(), sched=bst().make_sched(**sched))
        check_close(orc, C, ref, den, TOL_16, str(sched))


def test_mxfp8_add(orc):
    w = I.workload("mxfp8_4k", small=True)
    M, N = w["M"], w["N"]
    X = I.uniform_bf16((M, N), I.WORKLOAD_IDS["mxfp8_4k"], X_STREAM, -8.0, 8.0)
    ref, den = orc.gemm_add(orc.MXE4M3, w["A"], w["B"], X, "bf16", scale_a=w["scale_a"],
                            scale_b=w["scale_b"])
    A, B = to_gpu(w["A"], "e4m3"), to_gpu(w["B"], "e4m3")
    sa, sb = to_gpu(w["scale_a"], "u8"), to_gpu(w["scale_b"], "u8")
    for sched in [dict(tile=(64, 128), offset=8, xcd_remap=1), dict(tile=(128, 128), split_k=2)]:
        say("mxfp8 add", sched)
        C = bst().gemm(A, B, scale_a=sa, scale_b=sb, add=to_gpu(X, "bf16"),
                       sched=bst().make_sched(**sched))
        check_close(orc, C, ref, den, TOL_8, str(sched))


def test_int8_raw_plus_int32_bit_exact(orc):
    import torch
    M, N, K = 256, 384, 512
    A = I.int8_uniform((M, K), 11, 0)
    B = I.int8_uniform((K, N), 11, 1)
    X = np.random.default_rng(11).integers(-2**24, 2**24, (M, N)).astype(np.int32)
    ref, _ = orc.gemm_add(orc.I8, A, B, X, "i32")
    for sched in [dict(tile=(128, 128), offset=2), dict(tile=(128, 128), split_k=2, shuffle_k=1)]:
        C = torch.empty((M, N), dtype=torch.int32, device="cuda")
        bst().gemm(to_gpu(A, "i8"), to_gpu(B, "i8"), C, add=torch.from_numpy(X).cuda(),
                   sched=bst().make_sched(**sched))
        assert np.array_equal(codes(C).astype(np.int64), ref.astype(np.int64)), sched


def test_add_unsupported_tile_and_errors():
    import torch
    A = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    C = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(bst().BstError):
        bst().gemm(A, A, C, add=C, sched=bst().make_sched(tile=(256, 128)))   # no add instance
    with pytest.raises(TypeError):
        bst().gemm(A, A, C, add=torch.zeros((64, 64), dtype=torch.float32, device="cuda"))
