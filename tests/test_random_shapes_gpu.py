"""Seeded random-shape sweep of the GEMV, GEMM and decode FFN against the
double-precision oracle.

The hand-picked shapes in the other GPU tests sit on the launch
configurations' boundaries by design; this sweep draws ragged row counts,
K multiples of 128 and every batch size from a fixed seed, so that a shape
nobody thought of still meets the same bars: the floored relative error
1e-3 for FP32 outputs [P1 section 7; P2 "Como funciona la compresion"],
BF16 outputs equal to the nearest-even rounding of the FP32 entry point's,
and the FFN bound derived in test_ffn_gpu.
"""
import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import assert_close, dev_u16, host_u16, say
from tests.test_ffn_gpu import _ffn_ok

pytestmark = pytest.mark.gpu


def _draw(seed, count, m_max, n_max, kg_max, b_max):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        out.append((int(g.integers(1, m_max + 1)), int(g.integers(1, n_max + 1)),
                    128 * int(g.integers(1, kg_max + 1)), int(g.integers(1, b_max + 1))))
    return out


def _weights(fmt, g, n, k):
    if fmt == "q1":
        return oracle.q1_quantize(synth.fp16_normal(g, (n, k), 0.1))
    return oracle.t2_pack(synth.ternary(g, (n, k)), synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2))


GEMV_CASES = _draw(4242, 16, 1, 3000, 40, 8)


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("case", range(len(GEMV_CASES)))
def test_gemv_random_shapes(fmt, case):
    import torch

    _, n, k, b = GEMV_CASES[case]
    say(f"random gemv {fmt} n={n} k={k} b={b}")
    g = synth.rng(5000 + 97 * case + (fmt == "t2"))
    codes, scales = _weights(fmt, g, n, k)
    x = synth.fp16_normal(g, (b, k))
    of = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemv(of, codes, scales, n, k, x)
    y = lowbit.lowbit_gemv(fmt, torch.from_numpy(codes).cuda(), dev_u16(scales), n, k, dev_u16(x))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy().astype(np.float64), ref, f"gemv {fmt} {n}x{k} b={b}")


GEMM_CASES = _draw(4343, 8, 600, 1600, 8, 1)


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("case", range(len(GEMM_CASES)))
def test_gemm_random_shapes(fmt, case):
    import torch

    m, n, k, _ = GEMM_CASES[case]
    say(f"random gemm {fmt} m={m} n={n} k={k}")
    g = synth.rng(6000 + 97 * case + (fmt == "t2"))
    codes, scales = _weights(fmt, g, n, k)
    x = synth.bf16_normal(g, (m, k))
    of = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemm(of, codes, scales, n, k, x)
    c, s, xd = torch.from_numpy(codes).cuda(), dev_u16(scales), dev_u16(x, "bfloat16")
    yf = lowbit.lowbit_gemm_f32(fmt, c, s, n, k, xd)
    yb = lowbit.lowbit_gemm(fmt, c, s, n, k, xd)
    torch.cuda.synchronize()
    yf = yf.cpu().numpy()
    assert_close(yf, ref, f"gemm f32 {fmt} {m}x{n}x{k}")
    want = torch.from_numpy(np.ascontiguousarray(yf, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    assert np.array_equal(host_u16(yb), want), f"gemm bf16 {fmt} {m}x{n}x{k}"


# k = 128 * (1..12), f = 128 * (1..12); batch sizes fixed so that both z
# paths (formed inside the down GEMV for b <= 2, its own launch for b >= 3)
# are drawn
FFN_CASES = [(1, fg, k, b) for (_, fg, k, _), b in zip(_draw(4444, 6, 1, 12, 12, 8), (1, 2, 1, 2, 3, 8))]


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("case", range(len(FFN_CASES)))
def test_ffn_random_shapes(fmt, case):
    import torch

    _, fg, k, b = FFN_CASES[case]
    f = 128 * fg
    say(f"random ffn {fmt} k={k} f={f} b={b}")
    g = synth.rng(7000 + 97 * case + (fmt == "t2"))
    gu = _weights(fmt, g, 2 * f, k)
    dn = _weights(fmt, g, k, f)
    x = synth.fp16_normal(g, (b, k))
    of = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.ffn(of, gu[0], gu[1], dn[0], dn[1], k, f, x)
    y = lowbit.lowbit_ffn(fmt, torch.from_numpy(gu[0]).cuda(), dev_u16(gu[1]),
                          torch.from_numpy(dn[0]).cuda(), dev_u16(dn[1]), k, f, dev_u16(x))
    torch.cuda.synchronize()
    _ffn_ok(y.cpu().numpy(), ref, f"ffn {fmt} k={k} f={f} b={b}")
