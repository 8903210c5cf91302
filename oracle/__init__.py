"""CPU oracle for the group-scaled 1-bit / ternary y = W.x path.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``bit_matmul_lowbit_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain scalar C, double precision); this
module only builds that file with gcc and marshals numpy arrays through ctypes.
Every function documents the passage it follows:

* [P1] 7minutos.es, "Un tutorial de codificacion para ejecutar PrismML Bonsai
  1-bit LLM en CUDA con GGUF", section 7 "Q1_0_g128 Cuantizacion".
* [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", section "Como funciona la
  compresion".

Pins (what checks this code against something other than itself) are in
``tests/test_oracle_pins.py``; every function here is pinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q1 = 1
T2 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# tests/test_oracle_mutations.py points this at deliberately broken builds
# of oracle.c to show that the pins catch each mistake
_OVERRIDE = os.environ.get("LOWBIT_ORACLE_LIB_OVERRIDE")
_LIB = _OVERRIDE or os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if _OVERRIDE:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.orc_fp16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_fp16_to_f64.restype = ctypes.c_double
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = ctypes.c_double
        lib.orc_f64_to_bf16_rne.argtypes = [ctypes.c_double]
        lib.orc_f64_to_bf16_rne.restype = ctypes.c_uint16
        lib.orc_codes_bytes.argtypes = [ctypes.c_int, i64, i64]
        lib.orc_codes_bytes.restype = i64
        lib.orc_scales_count.argtypes = [i64, i64]
        lib.orc_scales_count.restype = i64
        lib.orc_code_value.argtypes = [ctypes.c_int, p, i64, i64, i64]
        lib.orc_code_value.restype = ctypes.c_int
        lib.orc_q1_quantize.argtypes = [p, i64, i64, p, p]
        lib.orc_q1_quantize.restype = None
        lib.orc_t2_pack.argtypes = [p, p, i64, i64, p, p]
        lib.orc_t2_pack.restype = None
        lib.orc_unpack.argtypes = [ctypes.c_int, p, p, i64, i64, p]
        lib.orc_unpack.restype = None
        lib.orc_gemv_rows_f64x.argtypes = [ctypes.c_int, p, p, i64, i64, p, i64, i64, i64, p]
        lib.orc_gemv_rows_f64x.restype = None
        lib.orc_gemv_rows.argtypes = [ctypes.c_int, p, p, i64, i64, p, i64, i64, i64, p, p]
        lib.orc_gemv_rows.restype = None
        lib.orc_gemm_rows.argtypes = [ctypes.c_int, p, p, i64, i64, p, i64, i64, i64, i64, p, p]
        lib.orc_gemm_rows.restype = None
        lib.orc_f64_to_fp16_rne.argtypes = [ctypes.c_double]
        lib.orc_f64_to_fp16_rne.restype = ctypes.c_uint16
        lib.orc_silu.argtypes = [ctypes.c_double]
        lib.orc_silu.restype = ctypes.c_double
        lib.orc_ffn_hidden.argtypes = [ctypes.c_int, p, p, i64, i64, p, i64, p, p, p]
        lib.orc_ffn_hidden.restype = None
        lib.orc_t2_quantize.argtypes = [p, i64, i64, p, p]
        lib.orc_t2_quantize.restype = None
        lib.orc_base3_row_bytes.argtypes = [i64]
        lib.orc_base3_row_bytes.restype = i64
        lib.orc_base3_pack.argtypes = [p, i64, i64, p]
        lib.orc_base3_pack.restype = None
        lib.orc_base3_unpack.argtypes = [p, i64, i64, p]
        lib.orc_base3_unpack.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


# --------------------------------------------------------------------------
# number formats

def fp16_to_f64(h: int) -> float:
    """binary16 pattern -> exact double."""
    return _load().orc_fp16_to_f64(int(h))


def bf16_to_f64(h: int) -> float:
    """bfloat16 pattern -> exact double."""
    return _load().orc_bf16_to_f64(int(h))


def f64_to_bf16_rne(v: float) -> int:
    """double -> bfloat16 pattern, nearest-even, single rounding."""
    return int(_load().orc_f64_to_bf16_rne(float(v)))


def f64_to_bf16_rne_array(v: np.ndarray) -> np.ndarray:
    f = _load().orc_f64_to_bf16_rne
    flat = np.asarray(v, dtype=np.float64).ravel()
    return np.array([f(float(a)) for a in flat], dtype=np.uint16).reshape(np.shape(v))


# --------------------------------------------------------------------------
# layout

def f64_to_fp16_rne(v: float) -> int:
    """double -> FP16 pattern, nearest-even (|v| >= 65520 -> infinity)."""
    return int(_load().orc_f64_to_fp16_rne(float(v)))


def f64_to_fp16_rne_array(v: np.ndarray) -> np.ndarray:
    f = _load().orc_f64_to_fp16_rne
    flat = np.asarray(v, dtype=np.float64).ravel()
    return np.array([f(float(a)) for a in flat], dtype=np.uint16).reshape(np.shape(v))


def silu(v: float) -> float:
    """SiLU(v) = v / (1 + e^-v) in double."""
    return float(_load().orc_silu(float(v)))


def codes_bytes(fmt: int, n: int, k: int) -> int:
    return int(_load().orc_codes_bytes(fmt, n, k))


def scales_count(n: int, k: int) -> int:
    return int(_load().orc_scales_count(n, k))


def code_value(fmt: int, codes: np.ndarray, k: int, row: int, col: int) -> int:
    """t in {-1,0,+1} of weight (row, col) read from the packed code plane."""
    return int(_load().orc_code_value(fmt, _ptr(codes), k, row, col))


# --------------------------------------------------------------------------
# packing

def q1_quantize(w_fp16: np.ndarray):
    """[P1 s.7] scale = max|w| per 128 along K, bit = 1 iff w >= 0.

    w_fp16: uint16 [n][k] FP16 patterns.  Returns (codes uint8, scales uint16).
    """
    w = np.ascontiguousarray(w_fp16, dtype=np.uint16)
    n, k = w.shape
    codes = np.zeros(codes_bytes(Q1, n, k), dtype=np.uint8)
    scales = np.zeros(scales_count(n, k), dtype=np.uint16)
    _load().orc_q1_quantize(_ptr(w), n, k, _ptr(codes), _ptr(scales))
    return codes, scales


def t2_pack(t: np.ndarray, s_fp16: np.ndarray):
    """[P2] ternary codes sign(t) plus the FP16 group scales, packed."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    s = np.ascontiguousarray(s_fp16, dtype=np.uint16)
    n, k = t.shape
    assert s.shape == (n, k // 128)
    codes = np.zeros(codes_bytes(T2, n, k), dtype=np.uint8)
    scales = np.zeros(scales_count(n, k), dtype=np.uint16)
    _load().orc_t2_pack(_ptr(t), _ptr(s), n, k, _ptr(codes), _ptr(scales))
    return codes, scales


def unpack(fmt: int, codes: np.ndarray, scales: np.ndarray, n: int, k: int) -> np.ndarray:
    """[P1 s.7, P2] dense FP16 patterns [n][k]: +-s (Q1) or s*t (T2)."""
    out = np.zeros((n, k), dtype=np.uint16)
    _load().orc_unpack(fmt, _ptr(np.ascontiguousarray(codes)),
                       _ptr(np.ascontiguousarray(scales)), n, k, _ptr(out))
    return out


# --------------------------------------------------------------------------
# products (double precision)

def gemv(fmt, codes, scales, n, k, x_fp16, row0=0, nrows=None) -> np.ndarray:
    """y[b][rows] = sum_g s * sum_k t * x, exact in double; x is FP16 [b][k]."""
    x = np.ascontiguousarray(np.atleast_2d(x_fp16), dtype=np.uint16)
    b = x.shape[0]
    assert x.shape[1] == k
    if nrows is None:
        nrows = n - row0
    y = np.zeros((b, nrows), dtype=np.float64)
    xbuf = np.zeros(b * k, dtype=np.float64)
    _load().orc_gemv_rows(fmt, _ptr(np.ascontiguousarray(codes)),
                          _ptr(np.ascontiguousarray(scales)), n, k, _ptr(x), b,
                          row0, nrows, _ptr(xbuf), _ptr(y))
    return y


def gemv_f64x(fmt, codes, scales, n, k, x64, row0=0, nrows=None) -> np.ndarray:
    """Same as gemv with x given as doubles [b][k]."""
    x = np.ascontiguousarray(np.atleast_2d(x64), dtype=np.float64)
    b = x.shape[0]
    if nrows is None:
        nrows = n - row0
    y = np.zeros((b, nrows), dtype=np.float64)
    _load().orc_gemv_rows_f64x(fmt, _ptr(np.ascontiguousarray(codes)),
                               _ptr(np.ascontiguousarray(scales)), n, k, _ptr(x), b,
                               row0, nrows, _ptr(y))
    return y


def gemm(fmt, codes, scales, n, k, x_bf16, m0=0, mrows=None, row0=0, nrows=None) -> np.ndarray:
    """Y[m][rows] in double for X BF16 [m][k]; one GEMV sum per X row."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    m = x.shape[0]
    assert x.shape[1] == k
    if mrows is None:
        mrows = m - m0
    if nrows is None:
        nrows = n - row0
    y = np.zeros((mrows, nrows), dtype=np.float64)
    xbuf = np.zeros(k, dtype=np.float64)
    _load().orc_gemm_rows(fmt, _ptr(np.ascontiguousarray(codes)),
                          _ptr(np.ascontiguousarray(scales)), n, k, _ptr(x), m0, mrows,
                          row0, nrows, _ptr(xbuf), _ptr(y))
    return y


# --------------------------------------------------------------------------
# decode FFN (gated MLP of the Qwen-derived models the pages compress)
#
# [P2] "Como funciona la compresion" and [P4] "Configuracion multimodal y de
# bajo bit de extremo a extremo": the MLP projections are low-bit like every
# other matrix.  [P5] "Detalles tecnicos": decode kernels were tuned at the
# matvec / FFN level.  The pages do not spell out the MLP; it is read as the
# gated form of the Qwen family, y = W_dn (SiLU(W_gate x) * (W_up x)), with
# gate and up stacked in one [2f][k] matrix (gate rows first) and the
# elementwise product rounded to FP16, the activation type every GEMV of the
# path reads.

def ffn_hidden(fmt, gu_codes, gu_scales, k, f, x_fp16) -> np.ndarray:
    """z[b][f] FP16 patterns: RNE_fp16(SiLU(h_gate) * h_up), h = W_gu x exact."""
    x = np.ascontiguousarray(np.atleast_2d(x_fp16), dtype=np.uint16)
    b = x.shape[0]
    assert x.shape[1] == k
    z = np.zeros((b, f), dtype=np.uint16)
    xbuf = np.zeros(b * k, dtype=np.float64)
    hbuf = np.zeros(b * 2 * f, dtype=np.float64)
    _load().orc_ffn_hidden(fmt, _ptr(np.ascontiguousarray(gu_codes)),
                           _ptr(np.ascontiguousarray(gu_scales)), k, f, _ptr(x), b,
                           _ptr(xbuf), _ptr(hbuf), _ptr(z))
    return z


def ffn(fmt, gu_codes, gu_scales, dn_codes, dn_scales, k, f, x_fp16, row0=0, nrows=None,
        z=None) -> np.ndarray:
    """y[b][rows] of the decode FFN in double; W_dn is [k][f] (rows = outputs).
    A precomputed z from ffn_hidden may be passed to sample several row sets."""
    if z is None:
        z = ffn_hidden(fmt, gu_codes, gu_scales, k, f, x_fp16)
    return gemv(fmt, dn_codes, dn_scales, k, f, z, row0=row0, nrows=nrows)


# --------------------------------------------------------------------------
# ternary quantiser and base-3 storage
#
# [P2] "Como funciona la compresion": log2(3) bits per ternary weight plus
# one FP16 scale per 128, ~1.71 bits per weight.  The pages give no ternary
# rounding rule; this build reads it as s = max |w| of the group and t the
# nearest of {-1, 0, +1} to w / s, ties to 0 (t = sign(w) iff 2|w| > s).

def t2_quantize(w_fp16: np.ndarray):
    """FP16 [n][k] -> (t int8 [n][k], s FP16 [n][k/128]) by the rule above."""
    w = np.ascontiguousarray(w_fp16, dtype=np.uint16)
    n, k = w.shape
    t = np.zeros((n, k), dtype=np.int8)
    s = np.zeros((n, k // 128), dtype=np.uint16)
    _load().orc_t2_quantize(_ptr(w), n, k, _ptr(t), _ptr(s))
    return t, s


def base3_row_bytes(k: int) -> int:
    return int(_load().orc_base3_row_bytes(k))


def base3_pack(t: np.ndarray) -> np.ndarray:
    """int8 t [n][k] -> uint8 [n][ceil(k/5)], five trits per byte."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    n, k = t.shape
    out = np.zeros((n, base3_row_bytes(k)), dtype=np.uint8)
    _load().orc_base3_pack(_ptr(t), n, k, _ptr(out))
    return out


def base3_unpack(b: np.ndarray, n: int, k: int) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    t = np.zeros((n, k), dtype=np.int8)
    _load().orc_base3_unpack(_ptr(b), n, k, _ptr(t))
    return t


def t2_codes_to_trits(codes: np.ndarray, n: int, k: int) -> np.ndarray:
    """The t values [n][k] held by ternary codes (layout v1), via the
    per-weight code reader."""
    f = _load().orc_code_value
    c = np.ascontiguousarray(codes)
    t = np.zeros((n, k), dtype=np.int8)
    for r in range(n):
        for j in range(k):
            t[r, j] = f(T2, _ptr(c), k, r, j)
    return t
