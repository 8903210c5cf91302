"""CPU checks of liblowbit.so: it loads, exports every symbol include/lowbit.h
declares, answers its host-only queries, and rejects bad arguments on the host
before any launch.  No call here reaches a kernel: every device entry point
is called only with arguments that fail validation, so the tests run without
a GPU.
"""
import ctypes
import math
import os
import re

import pytest

from bit_matmul_lowbit_amd import lowbit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lowbit.h")

OK, ARG, SHAPE, ALIGN, UNSUP, HIP, WS, SCRATCH = 0, 1, 2, 3, 4, 5, 6, 7
Q1, T2 = 1, 2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lowbit.LIB_PATH):
        from bit_matmul_lowbit_amd import build

        build.build()
    return lowbit.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w \*]*?\b(lowbit_\w+)\s*\(", text, flags=re.M)


def test_header_declares_what_binding_lists():
    assert declared_symbols() == lowbit.SYMBOLS


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.lowbit_version() == 1
    for s in range(8):
        assert lowbit.status_str(s) != "unknown status"
    assert lowbit.status_str(99) == "unknown status"


def test_size_queries(lib):
    for n, k in [(2048, 2048), (151936, 5120), (34816, 5120), (5120, 17408), (37, 384)]:
        np_ = (n + 15) // 16 * 16
        assert lowbit.lowbit_codes_bytes("q1", n, k) == np_ * k // 8
        assert lowbit.lowbit_codes_bytes("t2", n, k) == np_ * k // 4
        assert lowbit.lowbit_scales_bytes("q1", n, k) == np_ * (k // 128) * 2
        assert lowbit.lowbit_scales_bytes("t2", n, k) == np_ * (k // 128) * 2
    # the pages' per-group byte counts: 18 B (1-bit), 34 B (2-bit ternary codes)
    n, k = 4096, 4096
    q1 = lowbit.lowbit_codes_bytes("q1", n, k) + lowbit.lowbit_scales_bytes("q1", n, k)
    t2 = lowbit.lowbit_codes_bytes("t2", n, k) + lowbit.lowbit_scales_bytes("t2", n, k)
    assert q1 == 18 * n * k // 128 and q1 * 8 / (n * k) == 1.125
    assert t2 == 34 * n * k // 128 and t2 * 8 / (n * k) == 2.125
    # bad formats / shapes give 0
    assert lowbit.lowbit_codes_bytes(3, 16, 128) == 0
    assert lowbit.lowbit_codes_bytes("q1", 0, 128) == 0
    assert lowbit.lowbit_codes_bytes("q1", 16, 100) == 0
    assert lowbit.lowbit_codes_bytes("q1", 16, 0) == 0
    assert lowbit.lowbit_scales_bytes("t2", -1, 256) == 0


def test_workspace_query(lib):
    # b = 1, 2: a copy of x (the kernel builds its subset-sum tables from it)
    for b in (1, 2):
        for k in (128, 5120, 17408):
            assert lowbit.lowbit_gemv_workspace_bytes("t2", 151936, k, b) == b * k * 2
    # b >= 3 (matrix cores): x staged as MFMA operands, 4 KB per 128-weight group
    for b in (3, 4, 5, 8):
        for k in (128, 5120, 17408):
            assert lowbit.lowbit_gemv_workspace_bytes("q1", 2048, k, b) == (k // 128) * 4096
    assert lowbit.lowbit_gemv_workspace_bytes("q1", 16, 128, 0) == 0
    assert lowbit.lowbit_gemv_workspace_bytes("q1", 16, 128, 9) == 0


P = ctypes.c_void_p


def test_validation_returns_before_launch(lib):
    good = P(0x10000)  # never dereferenced: every call below fails validation
    bad_align = P(0x10008)
    null = P(0)
    st = P(0)
    # quantize
    assert lib.lowbit_quantize_q1(null, 16, 128, good, good, st) == ARG
    assert lib.lowbit_quantize_q1(good, 16, 100, good, good, st) == SHAPE
    assert lib.lowbit_quantize_q1(good, 0, 128, good, good, st) == SHAPE
    assert lib.lowbit_quantize_q1(bad_align, 16, 128, good, good, st) == ALIGN
    # pack
    assert lib.lowbit_pack_t2(good, null, 16, 128, good, good, st) == ARG
    assert lib.lowbit_pack_t2(good, good, 16, 129, good, good, st) == SHAPE
    assert lib.lowbit_pack_t2(good, good, 16, 128, bad_align, good, st) == ALIGN
    assert lib.lowbit_pack(Q1, good, good, 16, 128, good, good, st) == ARG  # Q1 takes no scales
    assert lib.lowbit_pack(7, good, null, 16, 128, good, good, st) == ARG
    # unpack
    assert lib.lowbit_unpack(0, good, good, 16, 128, good, st) == ARG
    assert lib.lowbit_unpack(T2, good, good, 16, 64, good, st) == SHAPE
    assert lib.lowbit_unpack(T2, good, bad_align, 16, 128, good, st) == ALIGN
    # gemv
    for b in (0, 9, -1):
        assert lib.lowbit_gemv(Q1, good, good, 16, 128, good, b, good, good, 1 << 20, st) == ARG
    assert lib.lowbit_gemv(Q1, good, good, 16, 120, good, 1, good, good, 1 << 20, st) == SHAPE
    assert lib.lowbit_gemv(Q1, good, good, 16, 128, good, 1, bad_align, good, 1 << 20, st) == ALIGN
    assert lib.lowbit_gemv(Q1, good, good, 16, 128, good, 1, good, null, 1 << 20, st) == WS
    assert lib.lowbit_gemv(Q1, good, good, 16, 128, good, 1, good, good, 16, st) == WS
    assert lib.lowbit_gemv(Q1, null, good, 16, 128, good, 1, good, good, 1 << 20, st) == ARG
    assert lib.lowbit_gemv_prepare(16, 128, null, 1, good, good, 1 << 20, st) == ARG
    assert lib.lowbit_gemv_prepare(16, 128, good, 9, good, good, 1 << 20, st) == ARG
    assert lib.lowbit_gemv_prepare(16, 136, good, 1, good, good, 1 << 20, st) == SHAPE
    assert lib.lowbit_gemv_prepare(16, 128, good, 1, good, good, 8, st) == WS
    assert lib.lowbit_gemv_accumulate(0, good, good, 16, 128, 1, good, good, 1 << 20, st) == ARG
    assert lib.lowbit_gemv_accumulate(T2, good, good, 16, 128, 1, bad_align, good, 1 << 20, st) == ALIGN
    assert lib.lowbit_gemv_accumulate(T2, good, good, 16, 128, 1, good, null, 1 << 20, st) == WS
    # gemm
    assert lib.lowbit_gemm(Q1, good, good, 16, 128, good, 0, good, st) == ARG
    assert lib.lowbit_gemm(T2, good, good, 16, 130, good, 4, good, st) == SHAPE
    assert lib.lowbit_gemm_f32(T2, good, good, 16, 128, bad_align, 4, good, st) == ALIGN
    assert lib.lowbit_gemm_f32(T2, good, null, 16, 128, good, 4, good, st) == ARG
    # a huge shape is refused, not overflowed
    assert lib.lowbit_gemv(Q1, good, good, 1 << 40, 128, good, 1, good, good, 1 << 20, st) == SHAPE


def test_ffn_workspace_query_and_validation(lib):
    def a256(v):
        return (v + 255) // 256 * 256
    # [h as P planes FP32 b x 2f][z prepared for W_dn], 256-aligned parts.
    # P: the gate+up table GEMV's K-slices for b <= 2 (1024 weights of K at
    # b = 1, 512 at b = 2); for b >= 3 the most K-pieces (at least 4 groups
    # = 512 weights each) the matrix-core GEMV can take.  b <= 2 forms z
    # inside the down GEMV and has no z part
    for b in (1, 2, 5, 8):
        for k, f in ((5120, 17408), (2048, 6144), (128, 128), (2176, 8320)):
            planes = -(-k // (1024 if b == 1 else 512))
            want = (a256(planes * b * 2 * f * 4)
                    + (a256(lowbit.lowbit_gemv_workspace_bytes("q1", k, f, b)) if b >= 3 else 0))
            assert lowbit.lowbit_ffn_workspace_bytes("q1", k, f, b) == want, (k, f, b)
    assert lowbit.lowbit_ffn_workspace_bytes("q1", 5120, 100, 1) == 0   # f % 128
    assert lowbit.lowbit_ffn_workspace_bytes("q1", 5000, 128, 1) == 0   # k % 128
    assert lowbit.lowbit_ffn_workspace_bytes("q1", 128, 128, 9) == 0
    assert lowbit.lowbit_ffn_workspace_bytes("q1", 128, 1 << 62, 1) == 0
    good, bad_align, null, st = P(0x10000), P(0x10008), P(0), P(0)
    big = 1 << 30
    assert lib.lowbit_ffn(Q1, good, good, good, good, 128, 128, good, 0, good, good, big, st) == ARG
    assert lib.lowbit_ffn(Q1, good, good, null, good, 128, 128, good, 1, good, good, big, st) == ARG
    assert lib.lowbit_ffn(Q1, good, good, good, good, 128, 200, good, 1, good, good, big, st) == SHAPE
    assert lib.lowbit_ffn(Q1, good, good, good, good, 130, 128, good, 1, good, good, big, st) == SHAPE
    assert lib.lowbit_ffn(Q1, good, good, good, good, 128, 128, bad_align, 1, good, good, big, st) == ALIGN
    assert lib.lowbit_ffn(Q1, good, good, good, good, 128, 128, good, 1, good, good, 64, st) == WS
    assert lib.lowbit_ffn(Q1, good, good, good, good, 128, 128, good, 1, good, null, big, st) == WS
    # silu_mul
    assert lib.lowbit_silu_mul(null, 128, 1, good, st) == ARG
    assert lib.lowbit_silu_mul(good, 128, 0, good, st) == ARG
    assert lib.lowbit_silu_mul(good, 12, 1, good, st) == SHAPE
    assert lib.lowbit_silu_mul(good, 128, 1, bad_align, st) == ALIGN


def test_ends_of_step_queries_and_validation(lib):
    # argmax parts: ceil(n / 1024) capped at 256, 8 bytes each per batch row
    for n, b in ((151936, 1), (151936, 8), (1000, 3), (1, 1)):
        parts = min(256, max(1, (n + 1023) // 1024))
        assert lowbit.load().lowbit_argmax_workspace_bytes(n, b) == (b * parts * 8 + 255) // 256 * 256
    assert lowbit.load().lowbit_argmax_workspace_bytes(0, 1) == 0
    assert lowbit.load().lowbit_argmax_workspace_bytes(1 << 31, 1) == 0
    g = lowbit.lowbit_gemv_workspace_bytes("t2", 151936, 5120, 1)
    assert lowbit.lowbit_lm_head_workspace_bytes("t2", 151936, 5120, 1) == (
        (g + 255) // 256 * 256 + lowbit.load().lowbit_argmax_workspace_bytes(151936, 1))
    assert lowbit.lowbit_lm_head_workspace_bytes("t2", 151936, 5120, 9) == 0
    good, bad_align, null, st = P(0x10000), P(0x10008), P(0), P(0)
    odd = P(0x10002)
    big = 1 << 30
    # embed
    assert lib.lowbit_embed(Q1, good, good, 16, 128, null, 4, good, st) == ARG
    assert lib.lowbit_embed(Q1, good, good, 16, 128, good, 0, good, st) == ARG
    assert lib.lowbit_embed(Q1, good, good, 16, 100, good, 4, good, st) == SHAPE
    assert lib.lowbit_embed(Q1, good, good, 16, 128, odd, 4, good, st) == ALIGN
    assert lib.lowbit_embed(T2, good, good, 16, 128, good, 4, bad_align, st) == ALIGN
    # argmax
    assert lib.lowbit_argmax(null, 16, 1, good, good, good, big, st) == ARG
    assert lib.lowbit_argmax(good, 16, 0, good, good, good, big, st) == ARG
    assert lib.lowbit_argmax(good, 0, 1, good, good, good, big, st) == SHAPE
    assert lib.lowbit_argmax(odd, 16, 1, good, good, good, big, st) == ALIGN
    assert lib.lowbit_argmax(good, 16, 1, good, good, good, 8, st) == WS
    # lm head
    assert lib.lowbit_lm_head(Q1, good, good, 16, 128, good, 9, good, good, good, good, big, st) == ARG
    assert lib.lowbit_lm_head(Q1, good, good, 16, 128, good, 1, good, null, good, good, big, st) == ARG
    assert lib.lowbit_lm_head(Q1, good, good, 16, 120, good, 1, good, good, good, good, big, st) == SHAPE
    assert lib.lowbit_lm_head(Q1, good, good, 16, 128, good, 1, good, good, good, good, 8, st) == WS


def test_ternary_storage_queries_and_validation(lib):
    assert lowbit.load().lowbit_base3_bytes(151936, 5120) == 151936 * 1024
    assert lowbit.load().lowbit_base3_bytes(3, 128) == 3 * 26
    assert lowbit.load().lowbit_base3_bytes(3, 100) == 0
    good, bad_align, null, st, odd = P(0x10000), P(0x10008), P(0), P(0), P(0x10001)
    assert lib.lowbit_quantize_t2(null, 16, 128, good, good, st) == ARG
    assert lib.lowbit_quantize_t2(good, 16, 120, good, good, st) == SHAPE
    assert lib.lowbit_quantize_t2(good, 16, 128, bad_align, good, st) == ALIGN
    assert lib.lowbit_t2_to_base3(good, good, 16, 128, null, good, st) == ARG
    assert lib.lowbit_t2_to_base3(good, odd, 16, 128, good, good, st) == ALIGN
    assert lib.lowbit_t2_to_base3(good, good, 0, 128, good, good, st) == SHAPE
    assert lib.lowbit_base3_to_t2(good, good, 16, 128, bad_align, good, st) == ALIGN
    assert lib.lowbit_base3_to_t2(good, good, 16, 130, good, good, st) == SHAPE


def test_binding_rejects_short_buffers(lib):
    # the C interface takes no buffer lengths: the binding checks them on the
    # host (plain CPU tensors stand in for device buffers here)
    import torch

    n, k = 40, 256
    cb = lowbit.lowbit_codes_bytes("t2", n, k)
    sb = lowbit.lowbit_scales_bytes("t2", n, k)
    lowbit._need_planes("t2", n, k, torch.empty(cb, dtype=torch.uint8), torch.empty(sb // 2))
    with pytest.raises(ValueError):
        # Q1-sized codes passed as ternary would be read past their end
        lowbit._need_planes("t2", n, k, torch.empty(lowbit.lowbit_codes_bytes("q1", n, k)),
                            torch.empty(sb // 2))
    with pytest.raises(ValueError):
        lowbit._need_planes("q1", n, k, torch.empty(cb), torch.empty(sb // 2 - 1))
    with pytest.raises(ValueError):
        lowbit._need_numel(torch.empty(3, 7), 22, "out")
    with pytest.raises(ValueError):
        lowbit._need_shape(torch.empty(7, 3), (3, 7), "out")


def test_noalloc_limits_are_checked_on_the_host(lib):
    # lowbit_gemv_noalloc rejects, before touching any device, a request whose
    # scratch exceeds its 1 MiB static array (the pointers here are never
    # dereferenced)
    good = ctypes.c_void_p(1 << 20)
    st = ctypes.c_void_p(0)
    assert lib.lowbit_gemv_noalloc(Q1, good, good, 16, 65536, good, 3, good, st) == SCRATCH
    assert lib.lowbit_gemv_noalloc(T2, good, good, 16, 1 << 19, good, 2, good, st) == SCRATCH
    assert lib.lowbit_gemv_noalloc(T2, good, good, 16, 128, good, 9, good, st) == ARG
    assert lib.lowbit_gemv_noalloc(T2, good, good, 16, 130, good, 1, good, st) == SHAPE
    assert lib.lowbit_gemv_noalloc(T2, ctypes.c_void_p(8), good, 16, 128, good, 1, good, st) == ALIGN
    assert lib.lowbit_gemv_noalloc(3, good, good, 16, 128, good, 1, good, st) == ARG
    # the limit sits where the header says: 2*b*k bytes for b <= 2, 32*k for b >= 3
    for b, k in ((1, 1 << 19), (2, 1 << 18), (3, 1 << 15), (8, 1 << 15)):
        assert lowbit.lowbit_gemv_workspace_bytes("q1", 16, k, b) == 1 << 20


def test_probe_header_and_exports(lib):
    text = open(os.path.join(ROOT, "include", "lowbit_probes.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(lowbit_probe_\w+)\s*\(", text, flags=re.M)
    assert names == lowbit.PROBE_SYMBOLS
    for name in names:
        assert hasattr(lib, name), name
    good = ctypes.c_void_p(1 << 20)
    st = ctypes.c_void_p(0)
    assert lib.lowbit_probe_stream_read(good, 100, 4, 0, good, st) == SHAPE
    assert lib.lowbit_probe_stream_read(good, 1 << 20, 0, 0, good, st) == ARG
    assert lib.lowbit_probe_stream_read(good, 1 << 20, 4, 2, good, st) == ARG
    assert lib.lowbit_probe_stream_read(ctypes.c_void_p(8), 1 << 20, 4, 1, good, st) == ALIGN
    assert lib.lowbit_probe_mfma_bf16(0, 2, good, st) == ARG
    assert lib.lowbit_probe_mfma_bf16(100, 9, good, st) == ARG
    assert lib.lowbit_probe_lds_read(100, 5, good, st) == ARG
    assert lib.lowbit_probe_lds_read(0, 2, good, st) == ARG
    assert lib.lowbit_probe_expand_mfma(3, 100, 2, good, st) == ARG
    assert lib.lowbit_probe_expand_mfma(2, 101, 2, good, st) == ARG  # mode 2: iters % 4
    assert lib.lowbit_probe_expand_mfma(1, 0, 2, good, st) == ARG
    assert lib.lowbit_probe_expand_mfma(1, 100, 5, good, st) == ARG
    assert lib.lowbit_probe_expand_mfma(1, 100, 2, ctypes.c_void_p(6), st) == ALIGN
