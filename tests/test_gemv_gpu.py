"""GPU parity of the decode GEMV against the double-precision oracle.

y[i][n] = sum_g s[n][g] * sum_{k in g} t[n][k] * x[i][k]  [P1 section 7; P2
"Como funciona la compresion"].  FP32 outputs must stay within a floored
relative error of 1e-3 (see helpers.floored_rel_err); one-hot inputs read a
single weight back and must match bit for bit.
"""
import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import assert_close, dev_u16, say

pytestmark = pytest.mark.gpu


def _make(fmt, n, k, seed):
    g = synth.rng(seed)
    if fmt == "q1":
        w = synth.fp16_normal(g, (n, k), 0.1)
        codes, scales = oracle.q1_quantize(w)
    else:
        t = synth.ternary(g, (n, k))
        s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
        codes, scales = oracle.t2_pack(t, s)
    return g, codes, scales


def _gemv(fmt, codes, scales, n, k, x16):
    import torch

    y = lowbit.lowbit_gemv(fmt, torch.from_numpy(codes).cuda(), dev_u16(scales), n, k, dev_u16(x16))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("b", [1, 3, 8])
def test_one_hot_reads_single_weight_exactly(fmt, b):
    n, k = 70, 1280
    say(f"gemv one-hot {fmt} b={b}")
    g, codes, scales = _make(fmt, n, k, 500 + b)
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    dense = oracle.unpack(f, codes, scales, n, k).view(np.float16).astype(np.float64)
    for cols in ([0] * b, list(range(7, 7 + 130 * b, 130)), [k - 1] * b, [511, 512, 513, 1000, 1279, 640, 3, 129][:b]):
        x = np.zeros((b, k), np.uint16)
        for i, c in enumerate(cols):
            x[i, c] = 0x3C00
        y = _gemv(fmt, codes, scales, n, k, x)
        want = np.stack([dense[:, c] for c in cols])
        assert np.array_equal(y, want), (cols, np.abs(y - want).max())


# The same on the matrix-core persistent kernel (two-phase API, which always
# runs the table or matrix-core kernel; 34816 x 1280 at b >= 3 makes 272
# items, more than the CUs): one product per output, then the group scale
# applied once (1-bit codes, lookup expansion) or with the operand (ternary),
# so each output is the weight exactly.
@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("b", [3, 8])
def test_one_hot_exact_on_persistent_matrix_core_kernel(fmt, b):
    import torch

    n, k = 34816, 1280
    say(f"gemv one-hot persistent {fmt} b={b}")
    g, codes, scales = _make(fmt, n, k, 700 + b)
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    cols = [0, 129, 640, 1279, 511, 512, 3, 1000][:b]
    dense = oracle.unpack(f, codes, scales, n, k).view(np.float16)[:, cols].astype(np.float64)
    x = np.zeros((b, k), np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x3C00
    dc, ds, dx = torch.from_numpy(codes).cuda(), dev_u16(scales), dev_u16(x)
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(lowbit.lowbit_gemv_workspace_bytes(fmt, n, k, b), dtype=torch.uint8,
                     device="cuda")
    lowbit.lowbit_gemv_prepare(n, k, dx, y, ws)
    lowbit.lowbit_gemv_accumulate(fmt, dc, ds, n, k, b, y, ws)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, dense.T), np.abs(got - dense.T).max()


SHAPES = [(1, 128), (16, 128), (37, 384), (300, 1280), (1000, 2176), (129, 4224)]


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 8])
def test_small_shapes(fmt, n, k, b):
    say(f"gemv {fmt} n={n} k={k} b={b}")
    g, codes, scales = _make(fmt, n, k, 600 + n + k + b)
    x = synth.fp16_normal(g, (b, k))
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemv(f, codes, scales, n, k, x)
    y = _gemv(fmt, codes, scales, n, k, x)
    assert_close(y, ref, f"{fmt} {n}x{k} b={b}")


def _gemv_split(fmt, codes, scales, n, k, x16):
    """The two-phase API (prepare, then accumulate): always the table kernel
    (b <= 2) or the matrix-core kernel (b >= 3), whatever the size."""
    import torch

    b = x16.shape[0]
    c, s, x = torch.from_numpy(codes).cuda(), dev_u16(scales), dev_u16(x16)
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(lowbit.lowbit_gemv_workspace_bytes(fmt, n, k, b), dtype=torch.uint8,
                     device="cuda")
    lowbit.lowbit_gemv_prepare(n, k, x, y, ws)
    lowbit.lowbit_gemv_accumulate(fmt, c, s, n, k, b, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


# lowbit_gemv sends most of these shapes to the single-launch kernel; the
# two-phase calls keep the table (b <= 2) and matrix-core (b >= 3) kernels
# covered at the same shapes
@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("b", [1, 2, 3, 5, 8])
def test_small_shapes_two_phase(fmt, n, k, b):
    say(f"gemv two-phase {fmt} n={n} k={k} b={b}")
    g, codes, scales = _make(fmt, n, k, 650 + n + k + b)
    x = synth.fp16_normal(g, (b, k))
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemv(f, codes, scales, n, k, x)
    assert_close(_gemv_split(fmt, codes, scales, n, k, x), ref, f"two-phase {fmt} {n}x{k} b={b}")


# the single-launch kernel's limits: 16 waves (k = 8192) at b = 1, 8 waves
# (k = 4096) at b >= 2, n * k <= 32 Mi weights (b <= 2) or n * k * b <= 128 Mi
# (b >= 3); and the first shapes past them (table / matrix-core kernels)
EDGES = [(40, 8192, 1), (40, 4096, 2), (40, 8320, 1), (40, 4224, 2), (4096, 8192, 1),
         (4112, 8192, 1), (17, 7808, 1), (2049, 4096, 2), (40, 4096, 8), (40, 4224, 3),
         (6544, 4096, 5), (6600, 4096, 5), (7, 128, 8), (33, 640, 6)]


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("n,k,b", EDGES)
def test_single_launch_limits(fmt, n, k, b):
    say(f"gemv limits {fmt} n={n} k={k} b={b}")
    g, codes, scales = _make(fmt, n, k, 660 + n + k + b)
    x = synth.fp16_normal(g, (b, k))
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemv(f, codes, scales, n, k, x)
    assert_close(_gemv(fmt, codes, scales, n, k, x), ref, f"{fmt} {n}x{k} b={b}")


def test_zero_codes_and_zero_scales():
    n, k = 40, 512
    say("gemv zero codes / zero scales")
    g = synth.rng(700)
    s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
    codes, scales = oracle.t2_pack(np.zeros((n, k), np.int8), s)
    x = synth.fp16_normal(g, (2, k))
    assert not _gemv("t2", codes, scales, n, k, x).any()
    w = synth.fp16_normal(g, (n, k), 0.1)
    w[5] = 0  # all-zero row: scale 0, output exactly 0
    codes, scales = oracle.q1_quantize(w)
    y = _gemv("q1", codes, scales, n, k, x)
    assert not y[:, 5].any()


def test_repeated_calls_do_not_accumulate():
    import torch

    n, k = 256, 1024
    say("gemv repeated calls")
    g, codes, scales = _make("t2", n, k, 800)
    x = dev_u16(synth.fp16_normal(g, (1, k)))
    c, s = torch.from_numpy(codes).cuda(), dev_u16(scales)
    ws = torch.empty(lowbit.lowbit_gemv_workspace_bytes("t2", n, k, 1), dtype=torch.uint8, device="cuda")
    out = torch.full((1, n), 123.0, device="cuda")
    y1 = lowbit.lowbit_gemv("t2", c, s, n, k, x, out=out, workspace=ws).clone()
    y2 = lowbit.lowbit_gemv("t2", c, s, n, k, x, out=out, workspace=ws).clone()
    torch.cuda.synchronize()
    ref = oracle.gemv(oracle.T2, codes, scales, n, k, dev_host(x))
    assert_close(y1.cpu().numpy(), ref)
    assert_close(y2.cpu().numpy(), ref)


def dev_host(x):
    from tests.helpers import host_u16

    return host_u16(x)


# full-size decode shapes, generated on the device, every output checked:
# configs 0 and 1 at b = 1, the 27B-class fused gate+up and down matrices at
# every batch the bench reports (1, 2, 5, 8; 5 = verify of k = 4 drafts),
# and the ternary LM head
FULL = [
    ("q1", 2048, 2048, 1),
    ("t2", 6144, 2048, 1),
    ("t2", 2048, 6144, 1),
    ("q1", 34816, 5120, 1),
    ("q1", 34816, 5120, 2),
    ("q1", 34816, 5120, 5),
    ("q1", 34816, 5120, 8),
    ("q1", 5120, 17408, 1),
    ("q1", 5120, 17408, 2),
    ("q1", 5120, 17408, 5),
    ("q1", 5120, 17408, 8),
    ("t2", 151936, 5120, 1),
]


@pytest.mark.parametrize("fmt,n,k,b", FULL)
def test_full_size(fmt, n, k, b):
    import torch

    from tests.helpers import full_weights, host_u16, oracle_blocks

    say(f"gemv full {fmt} n={n} k={k} b={b}")
    seed = 1000 + n + k + b
    codes, scales, hc, hs = full_weights(fmt, n, k, seed)
    x = synth.dev_fp16_normal((b, k), 1.0, seed + 2)
    y = lowbit.lowbit_gemv(fmt, codes, scales, n, k, x)
    torch.cuda.synchronize()
    hx = host_u16(x)
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle_blocks(lambda r0, r: oracle.gemv(f, hc, hs, n, k, hx, row0=r0, nrows=r), n, axis=1)
    assert_close(y.cpu().numpy(), ref, f"full {fmt} {n}x{k} b={b}")


# the largest K the library accepts (2^22): 32768 groups, 4096 K-slices of
# the table kernel, a 128 MB matrix-core workspace; offsets near 2^27 bytes
@pytest.mark.parametrize("fmt,b", [("q1", 1), ("t2", 2), ("q1", 5)])
def test_max_k(fmt, b):
    n, k = 16, 1 << 22
    say(f"gemv max k {fmt} n={n} k={k} b={b}")
    g, codes, scales = _make(fmt, n, k, 4242 + b)
    x = synth.fp16_normal(g, (b, k))
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemv(f, codes, scales, n, k, x)
    y = _gemv(fmt, codes, scales, n, k, x)
    assert_close(y, ref, f"{fmt} max k b={b}")
