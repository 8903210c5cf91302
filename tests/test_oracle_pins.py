"""Pins for the CPU oracle: each test checks it against something other than
itself -- numbers the pages print, library routines (numpy / torch), exhaustive
enumeration of FP16 patterns, closed forms, invariants and a hand-derived
layout fixture.  A plausible slip anywhere in oracle.c (a dropped scale, a
wrong sign rule, a transposed index, a wrong bit order) fails at least one.

Pages: [P1] 7minutos.es tutorial "Bonsai 1-bit LLM en CUDA con GGUF", section 7
"Q1_0_g128 Cuantizacion"; [P2] 7minutos.es "PrismML lanza Bonsai 27B", section
"Como funciona la compresion".
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# number formats

def test_fp16_to_f64_exhaustive_matches_numpy():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_f64(int(h)) for h in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero preserved
    assert math.copysign(1.0, oracle.fp16_to_f64(0x8000)) == -1.0


def test_bf16_to_f64_exhaustive_matches_torch():
    import torch

    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(int(h)) for h in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _bf16_rne_fraction(v: float) -> float:
    """Textbook round-to-nearest-even to 8 significant bits with exact
    rationals (independent of oracle.c); normal range only."""
    if v == 0:
        return v
    a = Fraction(abs(v))
    e = math.floor(math.log2(abs(v)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    q = a / ulp
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = float(fl * ulp)
    return -r if v < 0 else r


def test_f64_to_bf16_rne_against_torch_and_rationals():
    import torch

    g = np.random.default_rng(7)
    # values exactly representable in binary32: torch's cast is one rounding
    vals = np.concatenate([
        g.standard_normal(4000).astype(np.float32).astype(np.float64),
        (g.standard_normal(1000) * 1e-38).astype(np.float32).astype(np.float64),
        np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8), 3.3895313892515355e38,
                  2.0**-133, 2.0**-134, 3 * 2.0**-134, 1e-45, 0.0, -0.0]),
    ])
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_rne_array(vals)
    assert np.array_equal(got, ref)
    # doubles that binary32 cannot hold: single rounding must be used
    for v in [1.0 + 2.0**-8 + 2.0**-40, 1.0 + 2.0**-8 - 2.0**-40, -(1.0 + 2.0**-8 + 2.0**-45),
              12345.678901234567, -0.000123456789012345, 1.0 / 3.0]:
        expect = _bf16_rne_fraction(v)
        got_v = oracle.bf16_to_f64(oracle.f64_to_bf16_rne(v))
        assert got_v == expect, (v, got_v, expect)
    assert oracle.f64_to_bf16_rne(1.0 + 2.0**-8 + 2.0**-40) == 0x3F81
    assert oracle.f64_to_bf16_rne(1e39) == 0x7F80
    assert oracle.f64_to_bf16_rne(float("nan")) & 0x7FFF > 0x7F80


# --------------------------------------------------------------------------
# sizes printed on the pages

def test_format_sizes_match_printed_numbers():
    n, k = 4096, 8192
    q1_bytes = oracle.codes_bytes(oracle.Q1, n, k) + 2 * oracle.scales_count(n, k)
    t2_bytes = oracle.codes_bytes(oracle.T2, n, k) + 2 * oracle.scales_count(n, k)
    # [P1 s.7] 1 bit + 16/128 bits = 1.125 bpw; 18 B per group of 128
    assert q1_bytes * 8 / (n * k) == 1.125
    assert q1_bytes == 18 * n * k // 128
    # [P1 s.7] FP16 256 B vs 18 B per group: "14,2x" (printed with one decimal)
    assert f"{(128 * 2) / (128 / 8 + 2):.1f}" == "14.2"
    # [P1 s.7 box] Bonsai-1.7B: FP16 3.44 GB -> Q1_0_g128 0.24 GB
    params = 3.44e9 / 2
    assert round(params * 1.125 / 8 / 1e9, 2) == 0.24
    # [P2] ternary: log2(3) + 16/128 ~ 1.71 bpw, ~9.4x vs FP16 (entropy bound);
    # this library stores 2 bits + 16/128 = 2.125 bpw, 34 B per group
    assert round(math.log2(3) + 16 / 128, 2) == 1.71
    assert round(16 / (math.log2(3) + 16 / 128), 1) == 9.4
    assert t2_bytes * 8 / (n * k) == 2.125
    assert t2_bytes == 34 * n * k // 128
    # ragged rows are padded to a multiple of 16
    assert oracle.codes_bytes(oracle.Q1, 17, 128) == 32 * 128 // 8
    assert oracle.codes_bytes(oracle.Q1, 16, 100) == 0


# --------------------------------------------------------------------------
# Q1 quantiser  [P1 s.7]

def test_quantize_bit_rule_and_scale_exhaustive_fp16():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    n, k = 512, 128  # every FP16 pattern exactly once, one group per row
    w = pats.reshape(n, k)
    codes, scales = oracle.q1_quantize(w)
    dense = oracle.unpack(oracle.Q1, codes, scales, n, k)
    vals = w.view(np.float16).astype(np.float64)
    want_bit = vals >= 0  # IEEE comparison; NaN -> False, -0 -> True
    s_rows = np.array([oracle.fp16_to_f64(s) for s in scales[: n]])  # placeholder sizes
    del s_rows
    for row in range(n):
        srow = scales[(row // 16) * 16 + row % 16]  # G = 1: element tile*16 + r
        row_vals = vals[row]
        if np.isnan(row_vals).any():
            nan_mags = (w[row][np.isnan(row_vals)] & 0x7FFF).max()
            assert srow == nan_mags
        else:
            assert np.float16(np.abs(row_vals).max()).view(np.uint16) == srow
        got_bit = dense[row] == srow  # +s for bit 1, s^0x8000 for bit 0
        assert np.array_equal(got_bit, want_bit[row]), row
        assert np.array_equal(dense[row][~want_bit[row]], np.full((~want_bit[row]).sum(), srow ^ 0x8000, np.uint16))


def test_quantize_random_ragged_matches_numpy_semantics():
    g = synth.rng(11)
    n, k = 37, 384  # ragged rows (37 = 2*16 + 5), 3 groups
    w = synth.fp16_normal(g, (n, k), 0.1)
    codes, scales = oracle.q1_quantize(w)
    dense = oracle.unpack(oracle.Q1, codes, scales, n, k)
    v = w.view(np.float16).astype(np.float64)
    s = np.abs(v).reshape(n, k // 128, 128).max(axis=2)
    s16 = s.astype(np.float16).view(np.uint16)
    assert np.array_equal(s.astype(np.float16).astype(np.float64), s)  # max of FP16 is FP16
    s_full = np.repeat(s16, 128, axis=1)
    want = np.where(v >= 0, s_full, s_full ^ 0x8000).astype(np.uint16)
    assert np.array_equal(dense, want)
    # pad rows are zero
    np_ = 48
    assert oracle.codes_bytes(oracle.Q1, n, k) == np_ * k // 8
    tile2 = codes.reshape(np_ // 16, k // 8, 16)[2]
    assert not tile2[:, 5:].any()


def test_quantize_edge_groups():
    k = 128
    rows = []
    rows.append(np.zeros(k, np.uint16))                                   # all +0
    rows.append(np.full(k, 0x8000, np.uint16))                            # all -0
    r = np.full(k, 0x8001, np.uint16); r[5] = 0x0001; rows.append(r)      # negative subnormals
    r = np.full(k, 0x3C00, np.uint16); r[127] = 0xFC00; rows.append(r)    # -inf at the end
    r = np.full(k, 0xB800, np.uint16); r[0] = 0x7E00; rows.append(r)      # NaN first
    for pos in (0, 63, 127):                                              # single max anywhere
        r = np.full(k, 0x2E66, np.uint16); r[pos] = 0xC500; rows.append(r)
    w = np.stack(rows)
    n = w.shape[0]
    codes, scales = oracle.q1_quantize(w)
    dense = oracle.unpack(oracle.Q1, codes, scales, n, k)
    sc = [scales[(i // 16) * 16 + i % 16] for i in range(n)]
    assert sc[0] == 0 and (dense[0] == 0).all()                 # bit 1, +0 scale
    assert sc[1] == 0 and (dense[1] == 0).all()                 # -0 >= 0 -> bit 1
    assert sc[2] == 0x0001                                      # subnormal magnitude kept
    assert dense[2][5] == 0x0001 and (np.delete(dense[2], 5) == 0x8001).all()
    assert sc[3] == 0x7C00 and dense[3][127] == 0xFC00 and dense[3][0] == 0x7C00
    assert sc[4] == 0x7E00 and dense[4][0] == 0xFE00           # NaN -> bit 0
    for i in (5, 6, 7):
        assert sc[i] == 0x4500                                  # |-5.0|


def test_page_worked_example_seed42():
    """[P1 s.7] the demonstration: random.seed(42), 128 values of
    gauss(0, 0.1), scale = largest |w|, bit = 1 for w >= 0, 18 B per group.
    Inputs are rounded to FP16 first (the library's input type)."""
    random.seed(42)
    vals = [random.gauss(0, 0.1) for _ in range(128)]
    w = np.array(vals).astype(np.float16).view(np.uint16).reshape(1, 128)
    codes, scales = oracle.q1_quantize(w)
    v16 = w.view(np.float16).astype(np.float64)[0]
    assert oracle.fp16_to_f64(scales[0]) == max(abs(a) for a in v16)
    dense = oracle.unpack(oracle.Q1, codes, scales, 1, 128).view(np.float16).astype(np.float64)[0]
    assert all((d > 0) == (a >= 0) for d, a in zip(dense, v16))
    assert set(np.abs(dense)) == {oracle.fp16_to_f64(scales[0])}
    # the double-precision inputs and their FP16 roundings give the same bits
    assert all((a >= 0) == (b >= 0) for a, b in zip(vals, v16))
    assert codes.nbytes // 16 * 16 / 16 == 16  # 16 code bytes for this row tile
    assert 128 // 8 + 2 == 18

    # The values the demonstration produces when run (the page shows the
    # code, not its output): scale = max|w| = 0.2619945... in double, which
    # is 0.261962890625 (pattern 0x3431) once the inputs are FP16; the first
    # eight bits 0,0,0,1,0,0,1,0; 68 ones among the 128; reconstruction
    # MSE 0.038976; 256 B of FP16 against 18 B, "14,2x".
    assert scales[0] == 0x3431 and oracle.fp16_to_f64(scales[0]) == 0.261962890625
    bits = [1 if d > 0 else 0 for d in dense]
    assert bits[:8] == [0, 0, 0, 1, 0, 0, 1, 0]
    assert sum(bits) == 68
    # the oracle's scale is the FP16 rounding of the page's double scale
    # (|ds| = 3.2e-5); MSE(s) = mean((|w| - s)^2) moves by at most
    # 2 s |ds| = 1.7e-5 between the two scales
    mse = sum((a - d) ** 2 for a, d in zip(vals, dense)) / 128
    assert abs(mse - 0.038976) <= 2e-5, mse
    assert round(256 / (128 // 8 + 2), 1) == 14.2


# --------------------------------------------------------------------------
# ternary pack / unpack  [P2]

def test_t2_pack_unpack_is_t_times_s():
    g = synth.rng(12)
    n, k = 21, 256
    t = synth.ternary(g, (n, k))
    t[0, :10] = [3, -7, 127, -128, 1, -1, 0, 2, -2, 0]  # out-of-range values clamp by sign
    s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
    codes, scales = oracle.t2_pack(t, s)
    dense = oracle.unpack(oracle.T2, codes, scales, n, k)
    s_full = np.repeat(s, 128, axis=1)
    want = np.where(t > 0, s_full, np.where(t < 0, s_full ^ 0x8000, 0)).astype(np.uint16)
    assert np.array_equal(dense, want)
    vals = set(np.unique(dense.view(np.float16).astype(np.float64) / s_full.view(np.float16).astype(np.float64)))
    assert vals <= {-1.0, 0.0, 1.0}


def test_layout_golden_fixture():
    with open(os.path.join(GOLDEN, "layout_v1.json")) as f:
        fx = json.load(f)
    q = fx["q1"]
    w = np.full((q["n"], q["k"]), int(q["fill_fp16"], 16), np.uint16)
    for r, c, h in q["weights"]:
        w[r, c] = int(h, 16)
    codes, scales = oracle.q1_quantize(w)
    assert codes.nbytes == q["codes_bytes"] and scales.size == q["scales_count"]
    for off, val in q["bytes"]:
        assert codes[off] == int(val, 16), off
    for off, val in q["scales"]:
        assert scales[off] == int(val, 16), off
    t2 = fx["t2"]
    n, k = t2["n"], t2["k"]
    t = np.zeros((n, k), np.int8)
    for r, c, v in t2["t"]:
        t[r, c] = v
    s = np.array([[2 * r + gg + 1 for gg in range(k // 128)] for r in range(n)], np.float64)
    s16 = s.astype(np.float16).view(np.uint16)
    codes, scales = oracle.t2_pack(t, s16)
    assert codes.nbytes == t2["codes_bytes"]
    listed = {off for off, _ in t2["bytes"]}
    for off, val in t2["bytes"]:
        assert codes[off] == int(val, 16), off
    others = np.delete(codes, sorted(listed))
    assert not others.any()
    for off, val in t2["scales"]:
        assert scales[off] == int(val, 16), off


# --------------------------------------------------------------------------
# products

def _dense_q1(w16):
    v = w16.view(np.float16).astype(np.float64)
    n, k = v.shape
    s = np.abs(v).reshape(n, k // 128, 128).max(axis=2)
    return np.where(v >= 0, 1.0, -1.0) * np.repeat(s, 128, axis=1)


def _dense_t2(t, s16):
    return t.astype(np.float64) * np.repeat(s16.view(np.float16).astype(np.float64), 128, axis=1)


@pytest.mark.parametrize("fmt", [oracle.Q1, oracle.T2])
def test_gemv_matches_numpy_dense(fmt):
    g = synth.rng(13)
    n, k, b = 45, 512, 3
    if fmt == oracle.Q1:
        w = synth.fp16_normal(g, (n, k), 0.1)
        codes, scales = oracle.q1_quantize(w)
        W = _dense_q1(w)
    else:
        t = synth.ternary(g, (n, k))
        s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
        codes, scales = oracle.t2_pack(t, s)
        W = _dense_t2(t, s)
    x = synth.fp16_normal(g, (b, k))
    y = oracle.gemv(fmt, codes, scales, n, k, x)
    ref = x.view(np.float16).astype(np.float64) @ W.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # a row sub-range gives the same numbers
    ys = oracle.gemv(fmt, codes, scales, n, k, x, row0=17, nrows=11)
    assert np.array_equal(ys, y[:, 17:28])


def test_gemv_closed_forms():
    g = synth.rng(14)
    n, k = 33, 640
    # Q1, x = 1: y_n = sum_g s_g (2 * #(w >= 0) - 128)
    w = synth.fp16_normal(g, (n, k), 0.1)
    codes, scales = oracle.q1_quantize(w)
    v = w.view(np.float16).astype(np.float64).reshape(n, k // 128, 128)
    s = np.abs(v).max(axis=2)
    pop = (v >= 0).sum(axis=2)
    ones = np.full((1, k), 0x3C00, np.uint16)
    y = oracle.gemv(oracle.Q1, codes, scales, n, k, ones)[0]
    assert np.array_equal(y, (s * (2 * pop - 128)).sum(axis=1))
    # x = e_j: y_n is exactly the dequantised weight (n, j)
    for j in (0, 7, 8, 127, 128, 639):
        e = np.zeros((1, k), np.uint16); e[0, j] = 0x3C00
        yj = oracle.gemv(oracle.Q1, codes, scales, n, k, e)[0]
        want = np.where(v.reshape(n, k)[:, j] >= 0, 1.0, -1.0) * s[:, j // 128]
        assert np.array_equal(yj, want), j
    # T2, x = 1: y_n = sum_g s_g (n+ - n-); all-zero codes give exact zeros
    t = synth.ternary(g, (n, k))
    sc = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
    codes, scales = oracle.t2_pack(t, sc)
    y = oracle.gemv(oracle.T2, codes, scales, n, k, ones)[0]
    tt = t.reshape(n, k // 128, 128)
    want = (sc.view(np.float16).astype(np.float64) * ((tt > 0).sum(2) - (tt < 0).sum(2))).sum(1)
    assert np.array_equal(y, want)
    z_codes, z_scales = oracle.t2_pack(np.zeros((n, k), np.int8), sc)
    x = synth.fp16_normal(g, (2, k))
    assert not oracle.gemv(oracle.T2, z_codes, z_scales, n, k, x).any()


def test_gemv_invariants():
    g = synth.rng(15)
    n, k = 20, 256
    t = synth.ternary(g, (n, k))
    s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
    codes, scales = oracle.t2_pack(t, s)
    x = synth.fp16_normal(g, (2, k))
    y = oracle.gemv(oracle.T2, codes, scales, n, k, x)
    # x -> -x gives exactly -y
    assert np.array_equal(oracle.gemv(oracle.T2, codes, scales, n, k, x ^ 0x8000), -y)
    # t -> -t gives exactly -y
    c2, s2 = oracle.t2_pack(-t, s)
    assert np.array_equal(oracle.gemv(oracle.T2, c2, s2, n, k, x), -y)
    # s -> 2s (exact in FP16 here) gives exactly 2y
    s_dbl = (s.view(np.float16).astype(np.float64) * 2).astype(np.float16).view(np.uint16)
    c3, s3 = oracle.t2_pack(t, s_dbl)
    assert np.array_equal(oracle.gemv(oracle.T2, c3, s3, n, k, x), 2 * y)
    # changing row 7 leaves the other rows untouched
    t4 = t.copy(); t4[7] = -t4[7]
    c4, s4 = oracle.t2_pack(t4, s)
    y4 = oracle.gemv(oracle.T2, c4, s4, n, k, x)
    assert np.array_equal(np.delete(y4, 7, axis=1), np.delete(y, 7, axis=1))
    assert np.array_equal(y4[:, 7], -y[:, 7])


@pytest.mark.parametrize("fmt", [oracle.Q1, oracle.T2])
def test_gemm_matches_numpy_and_gemv(fmt):
    g = synth.rng(16)
    n, k, m = 24, 384, 5
    if fmt == oracle.Q1:
        w = synth.fp16_normal(g, (n, k), 0.1)
        codes, scales = oracle.q1_quantize(w)
        W = _dense_q1(w)
    else:
        t = synth.ternary(g, (n, k))
        s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
        codes, scales = oracle.t2_pack(t, s)
        W = _dense_t2(t, s)
    x = synth.bf16_normal(g, (m, k))
    import torch
    X = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    y = oracle.gemm(fmt, codes, scales, n, k, x)
    ref = X @ W.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    for i in range(m):
        assert np.array_equal(y[i], oracle.gemv_f64x(fmt, codes, scales, n, k, X[i])[0])
    ys = oracle.gemm(fmt, codes, scales, n, k, x, m0=2, mrows=2, row0=5, nrows=9)
    assert np.array_equal(ys, y[2:4, 5:14])


# --------------------------------------------------------------------------
# decode FFN: y = W_dn RNE_fp16(SiLU(W_gate x) * (W_up x))

def test_f64_to_fp16_rne_matches_numpy():
    # every finite FP16 value round-trips, and every midpoint between two
    # neighbours rounds as numpy's direct double -> half conversion does
    # (nearest, ties to even); random doubles over the whole range too
    h = np.arange(0x7C00, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    assert np.array_equal(oracle.f64_to_fp16_rne_array(v), h)
    assert np.array_equal(oracle.f64_to_fp16_rne_array(-v), h | 0x8000)
    mid = (v[:-1] + v[1:]) / 2  # exact in double
    want = mid.astype(np.float16).view(np.uint16)
    got = oracle.f64_to_fp16_rne_array(mid)
    assert np.array_equal(got, want)
    assert np.array_equal(got & 1, np.zeros_like(got))  # ties went to even
    g = np.random.default_rng(21)
    r = g.standard_normal(20000) * np.exp2(g.integers(-30, 18, 20000))
    with np.errstate(over="ignore"):
        want = r.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f64_to_fp16_rne_array(r), want)
    assert oracle.f64_to_fp16_rne(65519.99) == 0x7BFF and oracle.f64_to_fp16_rne(65520.0) == 0x7C00


def test_silu_against_expit_and_identities():
    from scipy.special import expit
    g = np.random.default_rng(22)
    vs = np.concatenate([g.standard_normal(500) * 8, [0.0, 1e-300, -745.0, 745.0, 30.0, -30.0]])
    for v in vs:
        s = oracle.silu(v)
        assert s == pytest.approx(v * expit(v), rel=1e-14, abs=1e-300)
        # v * sigmoid(v) - (-v) * sigmoid(-v) = v
        assert s - oracle.silu(-v) == pytest.approx(v, rel=1e-13, abs=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(-1000.0) == 0.0  # e^1000 overflows to inf: v / inf


def _ffn_weights(fmt, g, k, f):
    """Stacked gate+up [2f][k] and down [k][f] weights with dense copies."""
    if fmt == oracle.Q1:
        wgu = synth.fp16_normal(g, (2 * f, k), 0.1)
        wdn = synth.fp16_normal(g, (k, f), 0.1)
        gu = oracle.q1_quantize(wgu)
        dn = oracle.q1_quantize(wdn)
        return gu, dn, _dense_q1(wgu), _dense_q1(wdn)
    tgu, tdn = synth.ternary(g, (2 * f, k)), synth.ternary(g, (k, f))
    sgu = synth.fp16_uniform(g, (2 * f, k // 128), 0.01, 0.2)
    sdn = synth.fp16_uniform(g, (k, f // 128), 0.01, 0.2)
    return (oracle.t2_pack(tgu, sgu), oracle.t2_pack(tdn, sdn),
            _dense_t2(tgu, sgu), _dense_t2(tdn, sdn))


@pytest.mark.parametrize("fmt", [oracle.Q1, oracle.T2])
def test_ffn_matches_numpy_dense(fmt):
    from scipy.special import expit
    g = synth.rng(23)
    k, f, b = 256, 384, 3
    (gc, gs), (dc, ds), Wgu, Wdn = _ffn_weights(fmt, g, k, f)
    x = synth.fp16_normal(g, (b, k))
    X = x.view(np.float16).astype(np.float64)
    h = X @ Wgu.T
    zz = h[:, :f] * expit(h[:, :f]) * h[:, f:]
    z16 = zz.astype(np.float16)
    z = oracle.ffn_hidden(fmt, gc, gs, k, f, x)
    assert np.array_equal(z, z16.view(np.uint16))
    y = oracle.ffn(fmt, gc, gs, dc, ds, k, f, x)
    ref = z16.astype(np.float64) @ Wdn.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    ys = oracle.ffn(fmt, gc, gs, dc, ds, k, f, x, row0=100, nrows=30, z=z)
    assert np.array_equal(ys, y[:, 100:130])


def test_ffn_closed_forms():
    g = synth.rng(24)
    k, f = 128, 256
    tgu, tdn = synth.ternary(g, (2 * f, k)), synth.ternary(g, (k, f))
    sgu = synth.fp16_uniform(g, (2 * f, 1), 0.01, 0.2)
    sdn = synth.fp16_uniform(g, (k, f // 128), 0.01, 0.2)
    dc, ds = oracle.t2_pack(tdn, sdn)
    x = synth.fp16_normal(g, (2, k))
    # zero gate rows: SiLU(0) = 0, so z and y are exact zeros (z = -0.0
    # where the up value is negative)
    t0 = tgu.copy(); t0[:f] = 0
    gc0, gs0 = oracle.t2_pack(t0, sgu)
    assert not (oracle.ffn_hidden(oracle.T2, gc0, gs0, k, f, x) & 0x7FFF).any()
    assert not oracle.ffn(oracle.T2, gc0, gs0, dc, ds, k, f, x).any()
    # x = e_j: h is column j of the dequantised stacked matrix, exactly, so
    # z[f'] = RNE_fp16(SiLU(w_gate) * w_up) from math.exp and numpy's rounding
    gc, gs = oracle.t2_pack(tgu, sgu)
    sv = sgu.view(np.float16).astype(np.float64)[:, 0]
    for j in (0, 5, 127):
        e = np.zeros((1, k), np.uint16); e[0, j] = 0x3C00
        wg = tgu[:f, j] * sv[:f]
        wu = tgu[f:, j] * sv[f:]
        want = np.array([a / (1.0 + math.exp(-a)) * c for a, c in zip(wg, wu)]).astype(np.float16)
        assert np.array_equal(oracle.ffn_hidden(oracle.T2, gc, gs, k, f, e)[0], want.view(np.uint16))
    # gate and up are not interchangeable: the stacked order matters
    sw = np.concatenate([tgu[f:], tgu[:f]])
    gsw = np.concatenate([sgu[f:], sgu[:f]])
    gc2, gs2 = oracle.t2_pack(sw, gsw)
    assert not np.array_equal(oracle.ffn_hidden(oracle.T2, gc2, gs2, k, f, x),
                              oracle.ffn_hidden(oracle.T2, gc, gs, k, f, x))


# --------------------------------------------------------------------------
# ternary quantiser (rule: s = max|w|, t = sign(w) iff 2|w| > s, ties to 0)
# and base-3 storage (five trits per byte)

def test_t2_quantize_rule_exhaustive_magnitudes():
    # every FP16 magnitude m <= S against several group maxima S, decided
    # with exact rationals; both signs
    mags = np.arange(0x7C01, dtype=np.uint32).astype(np.uint16)  # 0 .. +inf
    for S in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x3C01, 0x5BFF, 0x7BFF, 0x7C00):
        cand = mags[mags <= S]
        sgn = (np.arange(cand.size) % 2).astype(np.uint16) << 15
        vals = cand | sgn
        per = 127
        groups = (vals.size + per - 1) // per
        w = np.zeros((groups, 128), np.uint16)
        w[:, 0] = S  # the group maximum
        flat = np.zeros(groups * per, np.uint16)
        flat[:vals.size] = vals
        w[:, 1:] = flat.reshape(groups, per)
        t, s = oracle.t2_quantize(w.reshape(1, -1))
        t = t.reshape(groups, 128)
        assert (s == S).all()
        sv = Fraction(oracle.fp16_to_f64(S)) if S != 0x7C00 else None
        for gi in range(groups):
            for j in range(1, 128):
                h = int(w[gi, j])
                m = h & 0x7FFF
                if sv is None:  # s = inf: 2|w| > inf never holds
                    want = 0
                else:
                    av = Fraction(oracle.fp16_to_f64(m)) if m != 0x7C00 else None
                    want = 0 if (av is None or not 2 * av > sv) else (-1 if h & 0x8000 else 1)
                assert t[gi, j] == want, (hex(S), hex(h))


def test_t2_quantize_nearest_and_worked_group():
    g = synth.rng(41)
    w = synth.fp16_normal(g, (7, 384), 0.1)
    t, s = oracle.t2_quantize(w)
    v = w.view(np.float16).astype(np.float64)
    sv = np.repeat(s.view(np.float16).astype(np.float64), 128, axis=1)
    assert np.array_equal(s, (v.reshape(7, 3, 128).__abs__().max(axis=2)).astype(np.float16).view(np.uint16))
    # s * t is a nearest point of {-s, 0, +s} (exact in double for FP16 values)
    d = np.stack([np.abs(v - sv * c) for c in (-1, 0, 1)])
    assert np.all(np.abs(v - sv * t) <= d.min(axis=0))
    # hand-built group: s = 1 (first weight), ties to 0, subnormals, -0
    vals = [1.0, 0.5, np.nextafter(np.float16(0.5), np.float16(1)), np.nextafter(np.float16(0.5), np.float16(0)),
            -0.75, -0.5, 0.0, -0.0, 6e-8, -1.0]
    wg = np.zeros((1, 128), np.float16)
    wg[0, :len(vals)] = vals
    t1, s1 = oracle.t2_quantize(wg.view(np.uint16))
    assert s1[0, 0] == 0x3C00
    assert list(t1[0, :len(vals)]) == [1, 0, 1, 0, -1, 0, 0, 0, 0, -1]
    assert not t1[0, len(vals):].any()
    # quantise -> pack -> read codes back gives t; unpack gives s * t exactly
    codes, scales = oracle.t2_pack(t, s)
    assert np.array_equal(oracle.t2_codes_to_trits(codes, 7, 384), t)


def test_base3_closed_forms_and_sizes():
    k = 10
    rows = np.array([[-1] * 10, [0] * 10, [1] * 10,
                     [1, -1, -1, -1, -1, -1, 1, -1, -1, -1],
                     [0, 0, 0, 0, 1, 1, 1, 1, 1, 1]], np.int8)
    b = oracle.base3_pack(rows)
    assert b.shape == (5, 2)
    assert b.tolist() == [[0, 0], [121, 121], [242, 242], [2, 6], [202, 242]]
    # k = 128: 25 full bytes and one holding three trits plus two padding
    # zeros (digit 1): for an all -1 row that byte is 27 + 81 = 108
    b128 = oracle.base3_pack(np.full((1, 128), -1, np.int8))
    assert b128.shape == (1, 26) and b128[0, 25] == 108 and not b128[0, :25].any()
    # round trip
    g = synth.rng(42)
    t = synth.ternary(g, (9, 640))
    assert np.array_equal(oracle.base3_unpack(oracle.base3_pack(t), 9, 640), t)
    # the pages' arithmetic: log2(3) + 16/128 ~ 1.71 bits per weight is the
    # bound; five trits per byte gives 8/5 + 16/128 = 1.725 (0.9 % above it)
    assert oracle.base3_row_bytes(5120) == 1024
    bpw = 8 * oracle.base3_row_bytes(5120) / 5120 + 16 / 128
    assert bpw == 1.725 and round(math.log2(3) + 16 / 128, 2) == 1.71
    assert bpw / (math.log2(3) + 16 / 128) < 1.01
    # a byte the packer never writes (243..255) decodes with its fifth digit mod 3
    assert oracle.base3_unpack(np.array([[243]], np.uint8), 1, 5).tolist() == [[-1, -1, -1, -1, -1]]
