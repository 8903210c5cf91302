"""GPU parity of the prefill GEMM against the double-precision oracle.

Y[i][n] = RNE_bf16(sum_g s[n][g] * sum_{k in g} X[i][k] * t[n][k])  [P1
section 7; P2 "Como funciona la compresion" and "Rendimiento ..."].

* the FP32-output entry point must be within a floored relative error of 1e-3
  of the oracle (the 1e-3 target cannot apply to BF16 outputs, whose own
  rounding step is 2^-8 relative);
* the BF16-output entry point must equal, bit for bit, the nearest-even
  rounding of the FP32-output entry point's values (same kernel, same
  summation order), and lie within one BF16 ulp of the rounded oracle value;
* one-hot rows of X read single weights back exactly.
"""
import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import TOL, assert_close, dev_u16, full_weights, host_u16, oracle_blocks, say

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


def _run(fmt, codes, scales, n, k, x16):
    import torch

    c, s, x = torch.from_numpy(codes).cuda(), dev_u16(scales), dev_u16(x16, "bfloat16")
    yf = lowbit.lowbit_gemm_f32(fmt, c, s, n, k, x)
    yb = lowbit.lowbit_gemm(fmt, c, s, n, k, x)
    torch.cuda.synchronize()
    return yf.cpu().numpy(), host_u16(yb)


def _rne_f32_to_bf16(f32):
    """Nearest-even rounding of FP32 values to BF16 patterns (torch's cast)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _bf16_ulp_ok(yb, ref64):
    """|y - ref| <= one BF16 ulp at |ref| + TOL * 0.01 * rms(row of ref).

    y is the nearest-even rounding of the FP32 sum (checked bit for bit
    separately), so |y - ref| <= ulp/2 + |FP32 sum - ref|; the FP32 error is
    bounded by the floored tolerance, whose floor is 1% of the row's RMS.  For
    ordinary outputs the ulp term dominates; outputs near zero by cancellation
    (below the floor) get the FP32 bound, which a BF16 ulp there can be far
    smaller than."""
    import torch

    y = torch.from_numpy(yb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    a = np.abs(ref64)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.exp2(np.maximum(e, -126) - 7)
    r2 = np.atleast_2d(ref64)
    rms = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True)).reshape(ref64.shape[:-1] + (1,)) \
        if ref64.ndim else np.float64(0.0)
    return np.all(np.abs(y - ref64) <= ulp * 1.0000001 + TOL * 0.01 * rms + 1e-30)


SHAPES = [(1, 16, 128), (5, 37, 384), (64, 128, 256), (130, 200, 640), (256, 129, 1280), (300, 300, 2048)]


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_small_shapes(fmt, m, n, k):
    say(f"gemm {fmt} m={m} n={n} k={k}")
    g, codes, scales = _make(fmt, n, k, 900 + m + n + k)
    x = synth.bf16_normal(g, (m, k))
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemm(f, codes, scales, n, k, x)
    yf, yb = _run(fmt, codes, scales, n, k, x)
    assert_close(yf, ref, f"gemm f32 {fmt} {m}x{n}x{k}")
    assert np.array_equal(yb, _rne_f32_to_bf16(yf))
    assert _bf16_ulp_ok(yb, ref)


@pytest.mark.parametrize("fmt", ["q1", "t2"])
def test_one_hot_rows_read_weights_exactly(fmt):
    m, n, k = 136, 144, 640
    say(f"gemm one-hot {fmt}")
    g, codes, scales = _make(fmt, n, k, 950)
    cols = np.random.default_rng(5).integers(0, k, m)
    x = np.zeros((m, k), np.uint16)
    x[np.arange(m), cols] = 0x3F80  # BF16 1.0
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    dense = oracle.unpack(f, codes, scales, n, k).view(np.float16).astype(np.float64)
    yf, yb = _run(fmt, codes, scales, n, k, x)
    assert np.array_equal(yf.astype(np.float64), dense[:, cols].T)


# Ragged shapes that reach each tile configuration of the launcher on a
# 256-CU part: 64 x 64 tiles, one team (600 x 2000); 128 x 96 tiles filling
# whole rounds of the CUs (500 x 6100: 64 x 4 = 256 tiles, last tile 52
# columns and 116 rows; 450 x 6144: 4 x 64 tiles): one K-group takes the
# twelve-wave kernel, more take the team kernel, whose K-teams run
# half-group stages unrolled six at a time -- 2 groups (two stages per
# team: a tail only), 3 (the second team's last group is past the end), 6
# (one unrolled pass), 10 (a pass and a four-stage tail); 128 x 128 tiles
# (2100 x 4100: 561 tiles).  Grids of one round with a multiple of 8 tiles
# take their tiles in die order: the 128 x 96 shapes above, and 64 x 64
# tiles with two K-teams at 500 x 2000 (8 x 32 = 256 tiles, last tile 52
# rows and 16 columns) and 500 x 500 (64 tiles).
# Smaller shapes above take 64 x 64 tiles with two K-teams.
CONFIG_SHAPES = [(600, 2000, 384), (450, 6144, 128), (500, 6100, 256), (500, 6100, 384),
                 (500, 6100, 768), (512, 6144, 1280), (2100, 4100, 128), (500, 2000, 384),
                 (500, 500, 256)]


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("m,n,k", CONFIG_SHAPES)
def test_tile_configs(fmt, m, n, k):
    say(f"gemm config {fmt} m={m} n={n} k={k}")
    g, codes, scales = _make(fmt, n, k, 960 + m + n + k)
    x = synth.bf16_normal(g, (m, k))
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemm(f, codes, scales, n, k, x)
    yf, yb = _run(fmt, codes, scales, n, k, x)
    assert_close(yf, ref, f"gemm f32 {fmt} {m}x{n}x{k}")
    assert np.array_equal(yb, _rne_f32_to_bf16(yf))
    assert _bf16_ulp_ok(yb, ref)


FULL = [("t2", 512, 6144, 2048), ("q1", 512, 2048, 6144)]


@pytest.mark.parametrize("fmt,m,n,k", FULL)
def test_full_pp512(fmt, m, n, k):
    import torch

    say(f"gemm full {fmt} m={m} n={n} k={k}")
    seed = 1004 + n
    codes, scales, hc, hs = full_weights(fmt, n, k, seed)
    x = synth.dev_bf16_normal((m, k), 1.0, seed + 2)
    yf = lowbit.lowbit_gemm_f32(fmt, codes, scales, n, k, x)
    yb = lowbit.lowbit_gemm(fmt, codes, scales, n, k, x)
    torch.cuda.synchronize()
    hx = host_u16(x)
    yf, yb = yf.cpu().numpy(), host_u16(yb)
    assert np.array_equal(yb, _rne_f32_to_bf16(yf))
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    # every one of the 512 rows (the oracle runs on a thread pool)
    ref = oracle_blocks(lambda m0, mr: oracle.gemm(f, hc, hs, n, k, hx, m0=m0, mrows=mr), m,
                        axis=0, block=8)
    assert_close(yf, ref, f"gemm full {fmt}")
    assert _bf16_ulp_ok(yb, ref)


@pytest.mark.parametrize("fmt", ["q1", "t2"])
def test_max_k(fmt):
    # the largest K the library accepts (2^22): 32768 K-groups, X rows of 8 MB
    m, n, k = 3, 16, 1 << 22
    say(f"gemm max k {fmt} m={m} n={n} k={k}")
    g, codes, scales = _make(fmt, n, k, 4343)
    x = synth.bf16_normal(g, (m, k))
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemm(f, codes, scales, n, k, x)
    yf, yb = _run(fmt, codes, scales, n, k, x)
    assert_close(yf, ref, f"gemm f32 {fmt} max k")
    assert np.array_equal(yb, _rne_f32_to_bf16(yf))
