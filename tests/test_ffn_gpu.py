"""GPU parity of the decode FFN (gated MLP) against the double-precision oracle.

y = W_dn RNE_fp16(SiLU(W_gate x) * (W_up x)), gate and up stacked in one
[2f][k] matrix [P2 "Como funciona la compresion": the MLP projections are
low-bit; P5 "Detalles tecnicos": FFN-level decode kernels].

Tolerances, from the arithmetic:
* lowbit_silu_mul, given h exactly, computes SiLU and the product in FP32
  (a few FP32 ulps, well under 1e-6 relative) and rounds once to FP16: its
  output must be the FP16 rounding of the exact double value, except where
  that value lies within 1e-6 (relative) of an FP16 rounding boundary,
  where either neighbour is accepted; a value that rounds to zero keeps the
  sign of the product (checked on its own at the edge values);
* the whole chain adds the FP32 GEMV error to h, so a z value whose exact
  double lies near an FP16 rounding boundary can round one FP16 ulp the
  other way.  Each such flip moves an output by |w| * ulp(z) and the flips
  are few and of random sign: their sum stays below 2e-4 * rms(y) at every
  shape here (at f = 17408 a CPU model of the FP32 chain puts it at
  ~2e-5 * rms(y)).  So every output must satisfy
    |y - y_oracle| <= 1e-3 * max(|y_oracle|, 0.01 rms(y_oracle)) + 2e-4 rms(y_oracle),
  the GEMV's floored bound plus that FP16-intermediate term.  A wrong gate,
  order, scale or layout errs by O(rms(y)).
"""
import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import TOL, dev_u16, full_weights, host_u16, say

pytestmark = pytest.mark.gpu

FFN_TERM = 2e-4  # FP16-intermediate allowance, relative to rms(y) per output vector


def _ffn_ok(y, ref, what):
    y = np.atleast_2d(np.asarray(y, np.float64))
    ref = np.atleast_2d(ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    for i, (yr, rr) in enumerate(zip(y, ref)):
        rms = np.sqrt(np.mean(rr * rr))
        bound = TOL * np.maximum(np.abs(rr), 0.01 * rms) + FFN_TERM * rms
        worst = np.max(np.abs(yr - rr) - bound)
        assert worst <= 0, f"{what} batch row {i}: exceeds the bound by {worst:.3e} (rms {rms:.3e})"


def _fp16_bracket(z64, rho=1e-6):
    """FP16 roundings of z64 * (1 -+ rho): equal unless z64 is within rho of a
    rounding boundary."""
    a = oracle.f64_to_fp16_rne_array(z64 * (1 - rho))
    b = oracle.f64_to_fp16_rne_array(z64 * (1 + rho))
    return a, b


def test_silu_mul_matches_oracle():
    import torch

    say("silu_mul b=3 f=1024 plus edge values")
    g = np.random.default_rng(71)
    b, f = 3, 1024
    h = (g.standard_normal((b, 2 * f)) * 6).astype(np.float32)
    # edges: zeros of both signs, exp overflow (v < -88), large products
    # (beyond the FP16 range), tiny products (FP16 subnormals)
    h[0, :8] = [0.0, -0.0, -100.0, -88.5, 88.0, 300.0, 1e-4, -1e-4]
    h[0, f:f + 8] = [1.5, -2.0, 3.0, -1.0, 2.0, 400.0, 1e-3, 2e-3]
    z = host_u16(lowbit.lowbit_silu_mul(torch.from_numpy(h).cuda()))
    torch.cuda.synchronize()
    h64 = h.astype(np.float64)
    z64 = np.array([[oracle.silu(v) for v in row] for row in h64[:, :f]]) * h64[:, f:]
    lo, hi = _fp16_bracket(z64)
    # zeros must carry the IEEE sign of the product: SiLU(-100) is -0 in FP32
    # (e^100 overflows) and a tiny negative number in double; both round to
    # the FP16 pattern 0x8000 once multiplied by 3
    ok = (z == lo) | (z == hi)
    bad = np.argwhere(~ok)[:4].tolist()
    assert ok.all(), (f"{(~ok).sum()} values off, first at {bad}: got "
                      f"{[hex(z[i, j]) for i, j in bad]}, want {[hex(lo[i, j]) for i, j in bad]}")
    assert (lo != hi).sum() < 0.01 * z.size  # the allowance is rarely used
    assert z[0, 5] == 0x7C00  # SiLU(300) * 400 is beyond FP16: +inf
    assert z[0, 2] == 0x8000  # SiLU(-100) * 3 = -0
    assert z[0, 0] == 0x0000 and z[0, 1] == 0x0000  # SiLU(+0) * 1.5 = +0, SiLU(-0) * -2 = +0



# shapes whose matrices are both small run the two single-launch GEMVs;
# f = 8320 (> 8192) or, for b >= 2, f = 4224 (> 4096) puts the down matrix
# past that kernel's limit, so those shapes run the table (b <= 2) or
# matrix-core (b >= 3) chain.  The table chain's gate+up GEMV leaves one
# plane of partial sums per K-slice (1024 weights of K at b = 1, 512 at
# b = 2) for the down GEMV to add up: k = 256 / 128 give one plane, 2176 at
# b = 1 three (the last slice ragged: 2 of 8 groups), 1024 at b = 2 two,
# 5120 at b = 2 ten (more planes than the 8 waves that load them).  The
# matrix-core chain's gate+up GEMV leaves one plane per K-piece (4 groups
# on these shapes) for the SiLU launch to add up: k = 128 / 256 one, 1024
# two and 2048 four (one item per work-group), 4096 eight (the persistent
# kernel: 264 items).
SMALL = [(128, 128, 1), (256, 384, 2), (384, 256, 3), (512, 640, 5), (1024, 512, 8),
         (256, 1024, 1), (640, 256, 4), (2048, 6144, 2), (256, 8320, 1), (128, 8320, 2),
         (2176, 8320, 1), (1024, 8320, 2), (5120, 4224, 2),
         (256, 4224, 3), (128, 4224, 5), (256, 4224, 8), (1024, 4224, 8), (2048, 4224, 5),
         (4096, 4224, 3)]


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("k,f,b", SMALL)
def test_ffn_small_shapes(fmt, k, f, b):
    import torch

    say(f"ffn {fmt} k={k} f={f} b={b}")
    g = synth.rng(2000 + k + f + b)
    if fmt == "q1":
        gu = oracle.q1_quantize(synth.fp16_normal(g, (2 * f, k), 0.1))
        dn = oracle.q1_quantize(synth.fp16_normal(g, (k, f), 0.1))
    else:
        gu = oracle.t2_pack(synth.ternary(g, (2 * f, k)), synth.fp16_uniform(g, (2 * f, k // 128), 0.01, 0.2))
        dn = oracle.t2_pack(synth.ternary(g, (k, f)), synth.fp16_uniform(g, (k, f // 128), 0.01, 0.2))
    x = synth.fp16_normal(g, (b, k))
    of = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.ffn(of, gu[0], gu[1], dn[0], dn[1], k, f, x)
    y = lowbit.lowbit_ffn(fmt, torch.from_numpy(gu[0]).cuda(), dev_u16(gu[1]),
                          torch.from_numpy(dn[0]).cuda(), dev_u16(dn[1]), k, f, dev_u16(x))
    torch.cuda.synchronize()
    _ffn_ok(y.cpu().numpy(), ref, f"ffn {fmt} k={k} f={f} b={b}")


@pytest.mark.parametrize("k,f,b", [(256, 256, 1), (256, 256, 2), (256, 256, 3), (2176, 8320, 1),
                                   (1024, 8320, 2), (256, 4224, 3), (2048, 4224, 4)])
def test_ffn_zero_gate_gives_exact_zeros(k, f, b):
    """SiLU(0) * up = 0 exactly, through every z path: formed by the
    single-launch down GEMV (f = 256), inside the down table GEMV from the
    summed planes of partial sums (f = 8320, b <= 2), by its own launch
    from one or several planes (f = 4224, b >= 3)."""
    import torch

    say(f"ffn zero gate k={k} f={f} b={b}")
    g = synth.rng(2100 + b + k + f)
    t = synth.ternary(g, (2 * f, k))
    t[:f] = 0
    gu = oracle.t2_pack(t, synth.fp16_uniform(g, (2 * f, k // 128), 0.01, 0.2))
    dn = oracle.t2_pack(synth.ternary(g, (k, f)), synth.fp16_uniform(g, (k, f // 128), 0.01, 0.2))
    x = synth.fp16_normal(g, (b, k))
    y = lowbit.lowbit_ffn("t2", torch.from_numpy(gu[0]).cuda(), dev_u16(gu[1]),
                          torch.from_numpy(dn[0]).cuda(), dev_u16(dn[1]), k, f, dev_u16(x))
    torch.cuda.synchronize()
    assert not y.cpu().numpy().any()


FULL = [("q1", 5120, 17408, 1), ("q1", 5120, 17408, 2), ("q1", 5120, 17408, 5),
        ("t2", 2048, 6144, 1)]


@pytest.mark.parametrize("fmt,k,f,b", FULL)
def test_ffn_full_shapes(fmt, k, f, b):
    import torch

    say(f"ffn full {fmt} k={k} f={f} b={b}")
    seed = 3000 + k + f + b
    guc, gus, hguc, hgus = full_weights(fmt, 2 * f, k, seed)
    dnc, dns, hdnc, hdns = full_weights(fmt, k, f, seed + 7)
    x = synth.dev_fp16_normal((b, k), 1.0, seed + 3)
    y = lowbit.lowbit_ffn(fmt, guc, gus, dnc, dns, k, f, x)
    torch.cuda.synchronize()
    of = oracle.Q1 if fmt == "q1" else oracle.T2
    hx = host_u16(x)
    # every output (the bound needs rms(y) of the whole vector); the oracle
    # takes a few seconds at these sizes
    ref = oracle.ffn(of, hguc, hgus, hdnc, hdns, k, f, hx)
    _ffn_ok(y.cpu().numpy(), ref, f"ffn full {fmt} k={k} f={f} b={b}")
