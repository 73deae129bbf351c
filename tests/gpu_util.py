"""Helpers for the GPU parity tests: move raw-code numpy arrays to the GPU as
typed tensors and bring results back as raw codes for the oracle."""
import sys

import numpy as np

TOL_16 = 2.0 ** -9   # fp16 / bf16 outputs: max |gpu - oracle| / sum_k |a_ik b_kj|
TOL_8 = 2.0 ** -7    # fp8 / MX-fp8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_gpu(arr, kind):
    import torch
    a = np.ascontiguousarray(arr)
    if kind in ("f16", "bf16"):
        t = torch.from_numpy(a.view(np.int16)).cuda()
        return t.view(torch.float16 if kind == "f16" else torch.bfloat16)
    if kind == "e4m3":
        return torch.from_numpy(a.view(np.uint8)).cuda().view(torch.float8_e4m3fn)
    if kind in ("u8", "e8m0"):
        return torch.from_numpy(a.view(np.uint8)).cuda()
    if kind == "i8":
        return torch.from_numpy(a.astype(np.int8)).cuda()
    if kind == "i32":
        return torch.from_numpy(a.astype(np.int32)).cuda()
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32)).cuda()
    raise KeyError(kind)


def codes(t):
    """Raw codes of a GPU result tensor as numpy (uint16 for 16-bit floats)."""
    import torch
    t = t.detach().cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def kind_of(t):
    import torch
    return {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32",
            torch.int32: "i32"}[t.dtype]


def check_close(orc, got_tensor, ref, den, tol, what=""):
    """Normalised error of a GPU result (tensor) against oracle (ref, den)."""
    got = orc.decode(kind_of(got_tensor), codes(got_tensor))
    e, at = orc.compare(got.reshape(ref.shape), ref, den)
    if not e <= tol:
        idx = np.unravel_index(at, ref.shape) if at >= 0 else None
        raise AssertionError("%s: normalised error %.3g > %.3g at %s (got %r, ref %r, den %r)" % (
            what, e, tol, idx, got.reshape(ref.shape)[idx] if idx else None,
            ref[idx] if idx else None, den[idx] if idx else None))
    return e


def check_close_rounded(orc, got_tensor, ref, den, tol, unit, what=""):
    """As check_close for outputs rounded to a format of unit roundoff `unit` (2^-8 for bf16,
    2^-11 for fp16): the rounding of the result itself, up to unit * |ref|, is allowed on top
    of tol * den.  A short sum of same-sign terms has |ref| close to den, and then that
    rounding alone exceeds tol * den."""
    got = orc.decode(kind_of(got_tensor), codes(got_tensor)).reshape(ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    excess = np.maximum(np.abs(got - ref) - unit * np.abs(ref), 0.0)
    e = np.where(den > 0, excess / np.where(den > 0, den, 1.0), np.where(got == 0, 0.0, np.inf))
    at = int(np.argmax(e))
    assert e.flat[at] <= tol, "%s: normalised error beyond the output rounding %.3g > %.3g at %s" % (
        what, e.flat[at], tol, np.unravel_index(at, ref.shape))
    return float(e.flat[at])
