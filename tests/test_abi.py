"""CPU tests of the C ABI: the library loads, exports every function that
include/bst.h declares, and its host-side validation rejects bad arguments
with the documented status before touching the GPU (all pointers here are
fake or NULL; no call reaches a launch)."""
import ctypes
import os
import re

import pytest

import block_swizzle_tile_amd as bst
from block_swizzle_tile_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced
FAKE2 = ctypes.c_void_p(0x20000)
ODD = ctypes.c_void_p(0x10008)         # not 16-byte aligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from block_swizzle_tile_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "bst.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bst_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert "bst_gemm" in names and "bst_grouped_gemm_slice_m" in names
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.EXPORTS) == names


def test_version(L):
    assert b"gfx950" in L.bst_version()


def S(**kw):
    return bst.make_sched(**kw)


def gemm(L, ab=_lib.F16, c=_lib.F16, M=64, N=64, K=64, A=FAKE, lda=None, B=FAKE, ldb=None,
         C=FAKE2, ldc=None, sa=None, sb=None, sched=None, ws=None, wsb=0):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return L.bst_gemm(ab, c, M, N, K, A, lda, B, ldb, C, ldc, sa, sb,
                      None if sched is None else ctypes.byref(sched), ws, wsb, None)


def test_validation_errors(L):
    assert gemm(L, sched=S(offset=0)) == _lib.E_INVAL            # offset 0 undefined
    assert gemm(L, sched=S(direction=3)) == _lib.E_INVAL         # no such direction
    assert gemm(L, sched=S(shuffle_k=2)) == _lib.E_INVAL         # ShuffleK is a flag
    assert gemm(L, M=-1) == _lib.E_INVAL
    assert gemm(L, A=None) == _lib.E_INVAL
    assert gemm(L, C=None) == _lib.E_INVAL
    assert gemm(L, lda=32) == _lib.E_INVAL                       # lda < K
    assert gemm(L, ldb=32) == _lib.E_INVAL
    assert gemm(L, ldc=32) == _lib.E_INVAL
    assert gemm(L, A=ODD) == _lib.E_ALIGN
    assert gemm(L, K=60, lda=60) == _lib.E_ALIGN                 # 120-byte rows
    assert gemm(L, sched=S(tile=(96, 96))) == _lib.E_UNSUPPORTED
    assert gemm(L, sched=S(tile=(128, 128), tile_k=32)) == _lib.E_UNSUPPORTED
    assert gemm(L, c=_lib.I32) == _lib.E_UNSUPPORTED             # int32 out needs int8 in
    assert gemm(L, ab=_lib.MXE4M3, c=_lib.BF16, K=48, lda=64, sa=FAKE, sb=FAKE) == _lib.E_INVAL
    assert gemm(L, ab=_lib.MXE4M3, c=_lib.BF16, K=64) == _lib.E_INVAL   # scales missing
    assert gemm(L, ab=_lib.I8, c=_lib.I32, K=131072, lda=131072) == _lib.E_INVAL
    assert gemm(L, ab=_lib.F16, sa=FAKE) == _lib.E_INVAL         # scales only for MX
    assert gemm(L, ab=9) == _lib.E_INVAL
    assert b"swizzle_offset" in gemm_msg(L, sched=S(offset=0))


def test_lds_dma_family_needs_c_tiles_within_2gib(L):
    """The LDS-DMA kernels store a C tile with 31-bit offsets: a row pitch that makes one tile's
    rows span 2 GiB or more rules them out (path 2 refused before any launch); the register-staged
    family takes it."""
    big = (1 << 31) // (64 * 2)          # fp16 elements: 64 rows of this pitch are exactly 2 GiB
    assert gemm(L, ldc=big, sched=S(tile=(64, 64), path=2)) == _lib.E_UNSUPPORTED
    assert b"LDS-DMA" in L.bst_last_error()
    assert gemm(L, ldc=big - 8, sched=S(tile=(64, 64), path=2)) != _lib.E_UNSUPPORTED


def gemm_msg(L, **kw):
    gemm(L, **kw)
    return L.bst_last_error()


def test_empty_problems_are_noops(L):
    assert gemm(L, M=0, A=None, B=None, C=None) == _lib.OK
    assert gemm(L, N=0, A=None, B=None, C=None) == _lib.OK
    assert L.bst_batched_gemm(_lib.F16, _lib.F16, 0, 64, 64, 64, None, 64, 0, None, 64, 0, None,
                              64, 0, None, None, 0, None) == _lib.OK


def test_workspace_required_for_split(L):
    s = S(tile=(128, 128), split_k=4)
    need = L.bst_workspace_bytes(0, _lib.F16, 1, 1024, 1024, 2048, ctypes.byref(s))
    assert need == 73728 + 4 * 64 * 128 * 128 * 4
    assert gemm(L, M=1024, N=1024, K=2048, sched=s) == _lib.E_WORKSPACE
    assert gemm(L, M=1024, N=1024, K=2048, sched=s, ws=FAKE, wsb=need - 1) == _lib.E_WORKSPACE
    assert L.bst_workspace_bytes(0, _lib.F16, 1, 1024, 1024, 2048,
                                 ctypes.byref(S(tile=(128, 128)))) == 0


def test_effective_sched_split_resolution(L):
    out = _lib.Sched()
    s = S(tile=(128, 128), split_k=16)
    assert L.bst_effective_sched(0, _lib.F16, 1, 1024, 1024, 256, ctypes.byref(s),
                                 ctypes.byref(out)) == _lib.OK
    assert out.split_k == 4 and out.tile_k == 64   # 4 stages of K: no empty slices
    s = S(tile=(128, 128), split_k=3)
    assert L.bst_effective_sched(0, _lib.F16, 1, 1024, 1024, 2048, ctypes.byref(s),
                                 ctypes.byref(out)) == _lib.OK
    assert out.split_k == 3 and out.grid >= 1 and out.path == 2
    # K not a whole number of 16-byte chunks: only the register-staged family
    assert L.bst_effective_sched(0, _lib.F16, 1, 64, 64, 60, ctypes.byref(S(tile=(64, 64))),
                                 ctypes.byref(out)) == _lib.OK and out.path == 1
    assert L.bst_effective_sched(0, _lib.F16, 1, 64, 64, 60,
                                 ctypes.byref(S(tile=(64, 64), path=2)),
                                 ctypes.byref(out)) == _lib.E_UNSUPPORTED
    assert L.bst_effective_sched(0, _lib.F16, 1, 64, 64, 64, ctypes.byref(S(path=4)),
                                 ctypes.byref(out)) == _lib.E_INVAL


def test_two_workgroup_family_selection(L):
    """path 3 (two resident workgroups per CU): chosen automatically at 128x128 when the launch
    has more units than CUs, on request otherwise; refused where no such instance exists."""
    out = _lib.Sched()

    def eff(kind, ab, count, M, N, K, **kw):
        st = L.bst_effective_sched(kind, ab, count, M, N, K, ctypes.byref(S(**kw)),
                                   ctypes.byref(out))
        return st, out.path
    # 1024 tiles of 128x128: more units than CUs
    for ab in (_lib.F16, _lib.BF16, _lib.I8):
        assert eff(0, ab, 1, 4096, 4096, 256, tile=(128, 128)) == (_lib.OK, 3)
        assert eff(0, ab, 1, 4096, 4096, 256, tile=(128, 128), path=2) == (_lib.OK, 2)
        # 64 tiles: one workgroup per CU with the deeper pipeline, unless asked
        assert eff(0, ab, 1, 1024, 1024, 256, tile=(128, 128)) == (_lib.OK, 2)
        assert eff(0, ab, 1, 1024, 1024, 256, tile=(128, 128), path=3) == (_lib.OK, 3)
        # grouped slice-M
        assert eff(1, ab, 8, 8192, 4096, 2048, tile=(128, 128)) == (_lib.OK, 3)
    # batched: 16 x 4 x 6 = 384 tiles
    assert eff(0, _lib.BF16, 16, 512, 768, 1024, tile=(128, 128)) == (_lib.OK, 3)
    # a split that brings the units above the CU count
    assert eff(0, _lib.F16, 1, 1024, 1024, 2048, tile=(128, 128), split_k=8) == (_lib.OK, 3)
    # no such instance: other tiles, slice-K, plain e4m3, matmul-add
    assert eff(0, _lib.F16, 1, 4096, 4096, 256, tile=(64, 64), path=3)[0] == _lib.E_UNSUPPORTED
    assert eff(0, _lib.F16, 1, 4096, 4096, 256, tile=(64, 64)) == (_lib.OK, 2)
    assert eff(3, _lib.I8, 8, 1024, 2048, 8192, tile=(128, 128), path=3)[0] == _lib.E_UNSUPPORTED
    assert eff(3, _lib.I8, 8, 1024, 2048, 8192, tile=(128, 128)) == (_lib.OK, 2)
    assert eff(0, _lib.MXE4M3, 1, 4096, 4096, 256, tile=(128, 128)) == (_lib.OK, 3)
    assert eff(0, _lib.MXE4M3, 1, 4096, 4096, 256, tile=(64, 128)) == (_lib.OK, 2)
    assert eff(0, _lib.E4M3, 1, 4096, 4096, 256, tile=(128, 128), path=3)[0] == _lib.E_UNSUPPORTED
    # a layout the LDS-DMA family cannot take: the register-staged family, and path 3 refused
    assert eff(0, _lib.F16, 1, 4096, 4096, 250, tile=(128, 128)) == (_lib.OK, 1)
    assert eff(0, _lib.F16, 1, 4096, 4096, 250, tile=(128, 128), path=3)[0] == _lib.E_UNSUPPORTED


def test_gemm_add_validation(L):
    """bst_gemm_add (C = A.B + X): validation before any launch."""
    def add(X=FAKE, ldx=64, sched=None, **kw):
        a = dict(ab=_lib.F16, c=_lib.F16, M=64, N=64, K=64, A=FAKE, lda=64, B=FAKE, ldb=64,
                 C=FAKE2, ldc=64)
        a.update(kw)
        return L.bst_gemm_add(a["ab"], a["c"], a["M"], a["N"], a["K"], a["A"], a["lda"],
                              a["B"], a["ldb"], X, ldx, a["C"], a["ldc"], None, None,
                              None if sched is None else ctypes.byref(sched), None, 0, None)
    assert add(X=None) == _lib.E_INVAL                       # the addend is required
    assert add(ldx=32) == _lib.E_INVAL                       # ldx < N
    assert add(X=ODD) == _lib.E_ALIGN
    assert add(ldx=68) == _lib.E_ALIGN                       # 136-byte rows
    assert add(sched=S(tile=(256, 128))) == _lib.E_UNSUPPORTED   # no matmul-add instance
    assert add(sched=S(tile=(64, 64), path=1)) == _lib.E_UNSUPPORTED  # LDS-DMA family only
    assert add(M=0, X=None) == _lib.OK                        # empty: nothing to add


def test_gemm_padded_validation(L):
    """bst_gemm_padded: workspace sizing and validation before any launch."""
    need = L.bst_workspace_bytes(2, _lib.F16, 1, 64, 64, 60, None)
    # 73728-byte counter area, then A 64 x 64 and B 64 x 64 fp16: rows padded to 16 bytes and
    # B's K padded the same way (4 zero rows)
    assert need == 73728 + 64 * 64 * 2 + 64 * 64 * 2
    assert L.bst_workspace_bytes(3, _lib.F16, 1, 64, 64, 60, None) == 0   # no such kind

    def pad(ws=None, wsb=0, ab=_lib.F16, c=_lib.F16, sa=None, sb=None, **kw):
        a = dict(M=64, N=64, K=60, A=ODD, lda=61, B=ODD, ldb=67, C=FAKE2, ldc=64)
        a.update(kw)
        return L.bst_gemm_padded(ab, c, a["M"], a["N"], a["K"], a["A"], a["lda"],
                                 a["B"], a["ldb"], a["C"], a["ldc"], sa, sb, None, ws, wsb,
                                 None)
    assert pad() == _lib.E_WORKSPACE                          # odd strides are fine, ws is not
    assert pad(ws=FAKE, wsb=need - 1) == _lib.E_WORKSPACE
    assert pad(ws=ODD, wsb=need) == _lib.E_ALIGN
    assert pad(lda=59) == _lib.E_INVAL                        # lda < K
    assert pad(A=None) == _lib.E_INVAL
    assert pad(M=0) == _lib.OK
    # Errors that only the GEMM's own checks find must still come before the
    # operand copies are enqueued: with fake operand pointers and a fake
    # workspace of the right size, a call that got as far as a launch would
    # fault or report BST_E_HIP, not the documented status.
    ws = dict(ws=FAKE, wsb=need)
    assert pad(c=_lib.I32, **ws) == _lib.E_UNSUPPORTED        # int32 out needs int8 in
    assert pad(C=None, **ws) == _lib.E_INVAL
    assert pad(C=ODD, **ws) == _lib.E_ALIGN
    assert pad(N=56, ldc=60, **ws) == _lib.E_ALIGN            # 120-byte rows of C
    assert pad(ldc=32, **ws) == _lib.E_INVAL                  # ldc < N
    mx_need = L.bst_workspace_bytes(2, _lib.MXE4M3, 1, 64, 64, 64, None)
    assert pad(ab=_lib.MXE4M3, c=_lib.BF16, K=64, lda=65, ws=FAKE,
               wsb=mx_need) == _lib.E_INVAL                   # MX scales missing
    assert pad(ab=_lib.MXE4M3, c=_lib.BF16, K=48, lda=65, sa=FAKE, sb=FAKE, ws=FAKE,
               wsb=1 << 20) == _lib.E_INVAL                   # MX needs K % 32 == 0


def test_gemm_padded_runs_the_dma_family(L):
    """The padding matmul pads K as well, so a K that is not a whole number of
    16-byte chunks still reaches the LDS-DMA kernels when N is aligned."""
    out = _lib.Sched()
    for ab, K in [(_lib.F16, 250), (_lib.BF16, 1001), (_lib.I8, 250), (_lib.E4M3, 120)]:
        assert L.bst_effective_sched(2, ab, 1, 200, 256, K, ctypes.byref(S(tile=(128, 128))),
                                     ctypes.byref(out)) == _lib.OK
        assert out.path == 2, (ab, K)
        assert L.bst_effective_sched(0, ab, 1, 200, 256, K, ctypes.byref(S(tile=(128, 128))),
                                     ctypes.byref(out)) == _lib.OK
        assert out.path == 1, (ab, K)          # the same K unpadded: register-staged only
    # N not aligned: the copies' extra columns would be outputs, so N is not padded
    assert L.bst_effective_sched(2, _lib.F16, 1, 200, 250, 256, None, ctypes.byref(out)) == _lib.OK
    assert out.path == 1


def test_batched_c_batches_may_not_overlap(L):
    def call(strideC):
        return L.bst_batched_gemm(_lib.F16, _lib.F16, 3, 64, 64, 64, FAKE, 64, 0, FAKE, 64,
                                  64 * 64, FAKE2, 72, strideC, None, None, 0, None)
    assert call(0) == _lib.E_INVAL
    assert call(63 * 72 + 56) == _lib.E_INVAL              # last row of batch b meets batch b+1
    assert b"overlap" in L.bst_last_error()
    # with no rows there is nothing to overlap
    assert L.bst_batched_gemm(_lib.F16, _lib.F16, 3, 0, 64, 64, FAKE, 64, 0, FAKE, 64, 0, FAKE2,
                              72, 0, None, None, 0, None) == _lib.OK


def test_task_count(L):
    n = ctypes.c_int64(-1)
    assert L.bst_task_count(0, _lib.F16, 3, 200, 136, ctypes.byref(S(tile=(64, 64))),
                            ctypes.byref(n)) == _lib.OK
    assert n.value == 3 * 4 * 3
    assert L.bst_task_count(1, _lib.I8, 8, 8192, 4096, ctypes.byref(S(tile=(256, 256))),
                            ctypes.byref(n)) == _lib.OK
    assert n.value == (32 + 8) * 16
    assert L.bst_task_count(0, _lib.F16, 1, 1024, 1024, None, ctypes.byref(n)) == _lib.OK
    assert n.value == 64                                     # default tile 128 x 128
    assert L.bst_task_count(0, _lib.F16, 1, 64, 64, ctypes.byref(S(tile=(96, 96))),
                            ctypes.byref(n)) == _lib.E_UNSUPPORTED
    assert L.bst_task_count(2, _lib.F16, 1, 64, 64, None, ctypes.byref(n)) == _lib.E_INVAL
    assert L.bst_task_count(0, _lib.F16, 1, 64, 64, None, None) == _lib.E_INVAL


def test_effective_sched_shuffle_k(L):
    """ShuffleK is applied by the LDS-DMA family only; the register-staged one runs stages in
    order and reports 0."""
    out = _lib.Sched()
    assert L.bst_effective_sched(0, _lib.F16, 1, 1024, 1024, 2048,
                                 ctypes.byref(S(tile=(64, 64), shuffle_k=1)),
                                 ctypes.byref(out)) == _lib.OK
    assert out.path == 2 and out.shuffle_k == 1
    assert L.bst_effective_sched(0, _lib.F16, 1, 1024, 1024, 2048,
                                 ctypes.byref(S(tile=(64, 64), shuffle_k=1, path=1)),
                                 ctypes.byref(out)) == _lib.OK
    assert out.path == 1 and out.shuffle_k == 0
    assert L.bst_effective_sched(0, _lib.F16, 1, 1024, 1024, 2048,
                                 ctypes.byref(S(tile=(64, 64))), ctypes.byref(out)) == _lib.OK
    assert out.shuffle_k == 0


def test_grouped_validation(L):
    def call(G=4, gm=FAKE, total_m=256, N=64, K=64, ab=_lib.I8, c=_lib.I32, rs=None, cs=None,
             strideB=None):
        strideB = K * N if strideB is None else strideB
        return L.bst_grouped_gemm_slice_m(ab, c, G, gm, total_m, N, K, FAKE, K, FAKE, N, strideB,
                                          FAKE2, N, rs, cs, None, None, 0, None)
    assert call(G=0) == _lib.E_INVAL
    assert call(G=1025) == _lib.E_INVAL
    assert call(gm=None) == _lib.E_INVAL
    assert call(rs=FAKE) == _lib.E_INVAL                 # one scale without the other
    assert call(rs=FAKE, cs=FAKE) == _lib.E_INVAL        # dequant into int32
    assert call(ab=_lib.E4M3, c=_lib.BF16) == _lib.E_UNSUPPORTED
    assert call(strideB=10) == _lib.E_INVAL
    assert call(total_m=0) == _lib.OK


def test_quant_requires_scales(L):
    r = L.bst_quant_gemm_per_token(64, 64, 64, FAKE, 64, FAKE, 64, None, None, FAKE2, 64,
                                   _lib.BF16, None, None, 0, None)
    assert r == _lib.E_INVAL


def test_slice_k_validation(L):
    """bst_grouped_gemm_slice_k: validation before any launch."""
    def call(G=4, gk=FAKE, total_k=256, M=64, N=64, ab=_lib.I8, c=_lib.I32, lda=None, ldc=64,
             strideC=None, rs=None, cs=None, A=FAKE, C=FAKE2, sched=None, ws=None, wsb=0):
        lda = total_k if lda is None else lda
        strideC = M * ldc if strideC is None else strideC
        return L.bst_grouped_gemm_slice_k(ab, c, G, gk, total_k, M, N, A, lda, FAKE, N, C, ldc,
                                          strideC, rs, cs,
                                          None if sched is None else ctypes.byref(sched), ws,
                                          wsb, None)
    assert call(G=0) == _lib.E_INVAL
    assert call(G=1025) == _lib.E_INVAL
    assert call(gk=None) == _lib.E_INVAL
    assert call(rs=FAKE) == _lib.E_INVAL                 # one scale without the other
    assert call(rs=FAKE, cs=FAKE) == _lib.E_INVAL        # dequant into int32
    assert call(ab=_lib.E4M3, c=_lib.BF16) == _lib.E_UNSUPPORTED
    assert call(ab=_lib.MXE4M3, c=_lib.BF16) == _lib.E_UNSUPPORTED
    assert call(ab=_lib.F16, c=_lib.I32) == _lib.E_UNSUPPORTED
    assert call(lda=200) == _lib.E_INVAL                 # lda < total_k
    assert call(ldc=32) == _lib.E_INVAL                  # ldc < N
    assert call(strideC=63 * 64 + 63) == _lib.E_INVAL    # outputs of groups overlap
    assert call(A=None) == _lib.E_INVAL
    assert call(C=ODD) == _lib.E_ALIGN
    assert call(lda=260) == _lib.E_ALIGN                 # 260-byte int8 rows
    assert call(M=0, C=None) == _lib.OK                  # no output
    s = S(tile=(128, 128), split_k=4)
    need = L.bst_workspace_bytes(3, _lib.I8, 4, 64, 64, 256, ctypes.byref(s))
    assert need == 73728 + 4 * 4 * 128 * 128 * 4         # 4 groups x 1 tile x 4 slices
    assert call(sched=s) == _lib.E_WORKSPACE
    assert call(sched=S(tile=(96, 96))) == _lib.E_UNSUPPORTED
    n = ctypes.c_int64(-1)
    assert L.bst_task_count(3, _lib.I8, 8, 1024, 2048, ctypes.byref(S(tile=(256, 256))),
                            ctypes.byref(n)) == _lib.OK and n.value == 8 * 4 * 8
    out = _lib.Sched()
    assert L.bst_effective_sched(3, _lib.I8, 8, 1024, 2048, 8192,
                                 ctypes.byref(S(tile=(256, 256))), ctypes.byref(out)) == _lib.OK
    assert out.path == 2 and out.split_k == 1
