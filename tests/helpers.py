"""Helpers for the GPU parity tests (not a test module)."""
import sys

import numpy as np

TOL = 1e-3  # max relative error of GEMV/GEMM outputs against the double-precision oracle


def say(*a):
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev_u16(a, dtype_name="float16"):
    """numpy uint16 patterns -> CUDA tensor of the given 16-bit float type."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return t.view(getattr(torch, dtype_name))


def host_u16(t):
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.contiguous().cpu().numpy()


def floored_rel_err(y, ref):
    """max_i |y_i - ref_i| / max(|ref_i|, 0.01 * rms(ref)), per output vector.

    An unfloored relative error is meaningless for outputs that are near zero
    by cancellation (any correct FP32 sum fails it); the floor ties those to
    the vector's RMS instead."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ref2 = np.atleast_2d(ref)
    y2 = np.atleast_2d(y)
    worst = 0.0
    for yr, rr in zip(y2, ref2):
        rms = np.sqrt(np.mean(rr * rr)) if rr.size else 0.0
        denom = np.maximum(np.abs(rr), 0.01 * rms)
        denom = np.where(denom == 0, 1.0, denom)
        worst = max(worst, float(np.max(np.abs(yr - rr) / denom)) if rr.size else 0.0)
    return worst


def assert_close(y, ref, what=""):
    e = floored_rel_err(y, ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert e <= TOL, f"{what}: floored relative error {e:.3e} > {TOL}"
    return e
