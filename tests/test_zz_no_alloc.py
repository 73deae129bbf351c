"""GPU test of bst_gemm_noalloc, the GEMM entry point that allocates nothing (its split-K
partials, counters and work queues live in the library's static device scratch).

Called through the C ABI and compared with bst_gemm (the same kernels with a caller
workspace) and with the oracle: two calls in a row, the second smaller, then an int8 call
(raw accumulators bit-exact) and a schedule too large for the scratch, which must be
refused before anything runs.
"""
import ctypes

import numpy as np
import pytest

from block_swizzle_tile_amd import inputs as I
from gpu_util import TOL_16, check_close, codes, say, to_gpu

pytestmark = pytest.mark.gpu


def _call_noalloc(L, ab, c, A, B, C, sched):
    import torch
    import block_swizzle_tile_amd as bst
    M, K = A.shape
    N = B.shape[1]
    return L.bst_gemm_noalloc(ab, c, M, N, K, ctypes.c_void_p(A.data_ptr()), A.stride(0),
                              ctypes.c_void_p(B.data_ptr()), B.stride(0),
                              ctypes.c_void_p(C.data_ptr()), C.stride(0), None, None,
                              ctypes.byref(sched),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_gemm(orc):
    import torch
    import block_swizzle_tile_amd as bst
    from block_swizzle_tile_amd import _lib
    L = _lib.lib()
    cases = [
        # (M, N, K, schedule): the first needs 16 MiB of partials, the second is smaller
        (1024, 1024, 2048, dict(tile=(128, 128), split_k=4, offset=2, xcd_remap=1)),
        (384, 256, 1024, dict(tile=(64, 64), split_k=3, offset=3, dynamic=1, grid=9)),
    ]
    for i, (M, N, K, sk) in enumerate(cases):
        A = I.uniform_f16((M, K), 81, 2 * i)
        B = I.uniform_f16((K, N), 81, 2 * i + 1)
        ref, den = orc.gemm(orc.F16, A, B, tile=(64, 64))
        At, Bt = to_gpu(A, "f16"), to_gpu(B, "f16")
        s = bst.make_sched(**sk)
        say("noalloc", M, N, K, sk)
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        assert _call_noalloc(L, _lib.F16, _lib.F16, At, Bt, C, s) == _lib.OK, L.bst_last_error()
        want = bst.gemm(At, Bt, sched=s)          # the same kernels with a caller workspace
        torch.cuda.synchronize()
        check_close(orc, C, ref, den, TOL_16, str(sk))
        assert np.array_equal(codes(C), codes(want)), sk
    # int8, raw accumulators: exact
    M, N, K = 256, 320, 1536
    A = I.int8_uniform((M, K), 82, 0)
    B = I.int8_uniform((K, N), 82, 1)
    _, _, acc = orc.gemm(orc.I8, A, B, tile=(64, 64), want_acc=True)
    C = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
    s = bst.make_sched(tile=(128, 128), split_k=2)
    assert _call_noalloc(L, _lib.I8, _lib.I32, to_gpu(A, "i8"), to_gpu(B, "i8"), C, s) == _lib.OK
    torch.cuda.synchronize()
    assert np.array_equal(codes(C), acc.astype(np.int32))
    # a schedule whose partials exceed the scratch: refused, nothing written
    M, N, K = 1024, 2048, 4096
    At = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    Bt = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    C = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    s = bst.make_sched(tile=(128, 128), split_k=8)
    assert bst.workspace_bytes(0, bst.F16, 1, M, N, K, s) > 32 << 20
    assert _call_noalloc(L, _lib.F16, _lib.F16, At, Bt, C, s) == _lib.E_WORKSPACE
    assert b"static scratch" in L.bst_last_error()
    torch.cuda.synchronize()
    assert bool((C == 3.0).all())
