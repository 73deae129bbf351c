"""Pins of the oracle's exact decoders: every code of fp16, bf16, OCP e4m3fn
and OCP e8m0 against torch / numpy dtype casts (an independent library)."""
import numpy as np
import torch


def _same(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    return np.all(both_nan | (a == b)) and np.array_equal(np.signbit(a) & ~both_nan,
                                                          np.signbit(b) & ~both_nan)


def test_f16_exhaustive(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert _same(orc.decode("f16", codes), codes.view(np.float16).astype(np.float64))


def test_bf16_exhaustive(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert _same(orc.decode("bf16", codes), ref)


def test_e4m3fn_exhaustive(orc):
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = orc.decode("e4m3", codes)
    assert _same(got, ref)
    assert np.nanmax(got) == 448.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[1] == 2.0 ** -9


def test_e8m0_exhaustive(orc):
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = orc.decode("e8m0", codes)
    assert _same(got, ref)
    assert got[127] == 1.0 and np.isnan(got[255])


def test_integer_and_float_kinds(orc):
    i8 = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    assert np.array_equal(orc.decode("i8", i8), i8.astype(np.float64))
    i32 = np.array([-2**31, -1, 0, 1, 2**31 - 1], np.int32)
    assert np.array_equal(orc.decode("i32", i32), i32.astype(np.float64))
    f32 = np.array([0.0, -0.0, 1.5, 3.4e38, 1e-45], np.float32)
    assert _same(orc.decode("f32", f32), f32.astype(np.float64))
