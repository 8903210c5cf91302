"""Helpers for the GPU parity tests (not a test module)."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

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


def full_weights(fmt, n, k, seed):
    """Seeded full-size weights for a GPU parity test: the values are drawn
    on the device (torch's seeded generator, as bench.py does), copied to
    the host and packed there by the oracle; the GPU gets the uploaded
    oracle codes, so both sides read the same codes and none of the
    oracle's inputs comes from the library.  Returns (device codes, device
    scales, host codes, host scales)."""
    import torch

    import oracle
    from bit_matmul_lowbit_amd import synth

    if fmt == "q1":
        w = synth.dev_fp16_normal((n, k), 0.1, seed)
        hw = host_u16(w)
        del w
        hc, hs = oracle.q1_quantize(hw)
        del hw
    else:
        t = synth.dev_ternary((n, k), seed)
        s = synth.dev_fp16_uniform((n, k // 128), 0.01, 0.2, seed + 1)
        ht, hsc = t.cpu().numpy(), host_u16(s)
        del t, s
        hc, hs = oracle.t2_pack(ht, hsc)
        del ht
    return torch.from_numpy(hc).cuda(), dev_u16(hs), hc, hs


def oracle_threads():
    """Threads for oracle calls: the host's CPUs, at most 16 (ctypes releases
    the GIL during each oracle call, so the calls run in parallel)."""
    return max(1, min(16, os.cpu_count() or 1))


def oracle_blocks(call, total, axis, block=None):
    """Concatenation along `axis` of call(start, count) over [0, total) in
    blocks, computed on a thread pool.  `call` is an oracle function of a
    row range; the blocks are independent, so the result equals one call
    over the whole range."""
    nt = oracle_threads()
    if block is None:
        block = max(1, -(-total // (4 * nt)))
    starts = list(range(0, total, block))
    with ThreadPoolExecutor(nt) as ex:
        parts = list(ex.map(lambda s0: call(s0, min(block, total - s0)), starts))
    return np.concatenate(parts, axis=axis)


GUARD = 4096      # bytes of known pattern on each side of a guarded output
GUARD_BYTE = 0xA5


def guarded(shape, dtype):
    """(raw, view): `view` is a device tensor of `shape` and `dtype` that sits
    inside `raw` with GUARD bytes of GUARD_BYTE before and after it (and is
    filled with GUARD_BYTE itself); 256-byte aligned like torch's own
    allocations."""
    import torch

    shape = tuple(shape)
    n = 1
    for d in shape:
        n *= d
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    raw = torch.full((GUARD + nbytes + GUARD,), GUARD_BYTE, dtype=torch.uint8, device="cuda")
    view = raw[GUARD:GUARD + nbytes].view(dtype).view(shape)
    return raw, view


def guards_intact(raw):
    """True if the GUARD bytes on both sides still hold GUARD_BYTE."""
    head = raw[:GUARD].cpu().numpy()
    tail = raw[-GUARD:].cpu().numpy()
    return bool((head == GUARD_BYTE).all() and (tail == GUARD_BYTE).all())
