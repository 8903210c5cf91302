"""GPU parity of the packing kernels against the CPU oracle: bit-exact.

Q1 quantiser [P1: 7minutos.es tutorial, section 7], ternary packer and the
unpacker [P2: "PrismML lanza Bonsai 27B", "Como funciona la compresion"].
"""
import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import dev_u16, host_u16, host_u8, say

pytestmark = pytest.mark.gpu


def _q1_gpu(w16):
    import torch

    n, k = w16.shape
    codes, scales = lowbit.lowbit_quantize_q1(dev_u16(w16))
    torch.cuda.synchronize()
    return host_u8(codes), host_u16(scales)


def test_quantize_all_fp16_patterns():
    say("quantize_q1: all 65536 FP16 patterns as 512 x 128")
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 128)
    c, s = _q1_gpu(w)
    oc, os_ = oracle.q1_quantize(w)
    assert np.array_equal(c, oc)
    assert np.array_equal(s, os_)
    # shuffled across groups too
    g = np.random.default_rng(3)
    w2 = g.permutation(w.ravel()).reshape(256, 256)
    c, s = _q1_gpu(w2)
    oc, os_ = oracle.q1_quantize(w2)
    assert np.array_equal(c, oc) and np.array_equal(s, os_)


@pytest.mark.parametrize("n,k", [(1, 128), (15, 128), (16, 256), (37, 384), (100, 2048), (513, 4224)])
def test_quantize_random_shapes(n, k):
    say(f"quantize_q1 random n={n} k={k}")
    g = synth.rng(100 + n)
    w = synth.fp16_normal(g, (n, k), 0.1)
    w[0, :5] = [0x0000, 0x8000, 0x8001, 0x0001, 0x7E00]  # +0, -0, -subnormal, +subnormal, NaN
    c, s = _q1_gpu(w)
    oc, os_ = oracle.q1_quantize(w)
    assert np.array_equal(c, oc)
    assert np.array_equal(s, os_)


def test_quantize_full_lm_head_shape():
    """The 151936 x 5120 FP16 N(0, 0.02) matrix, byte-exact."""
    import torch

    from bit_matmul_lowbit_amd import synth as sy

    n, k = 151936, 5120
    say(f"quantize_q1 full {n}x{k}")
    w = sy.dev_fp16_normal((n, k), 0.02, seed=1003)
    codes, scales = lowbit.lowbit_quantize_q1(w)
    torch.cuda.synchronize()
    wh = host_u16(w)
    oc, os_ = oracle.q1_quantize(wh)
    assert np.array_equal(host_u8(codes), oc)
    assert np.array_equal(host_u16(scales), os_)


@pytest.mark.parametrize("n,k", [(1, 128), (16, 128), (37, 384), (300, 1280), (2048, 6144)])
def test_pack_t2(n, k):
    import torch

    say(f"pack_t2 n={n} k={k}")
    g = synth.rng(200 + n)
    t = synth.ternary(g, (n, k))
    t[0, :6] = [5, -3, 127, -128, 0, 1]
    s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
    codes, scales = lowbit.lowbit_pack_t2(torch.from_numpy(t).cuda(), dev_u16(s))
    torch.cuda.synchronize()
    oc, os_ = oracle.t2_pack(t, s)
    assert np.array_equal(host_u8(codes), oc)
    assert np.array_equal(host_u16(scales), os_)


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("n,k", [(1, 128), (37, 384), (300, 1280)])
def test_unpack(fmt, n, k):
    import torch

    say(f"unpack {fmt} n={n} k={k}")
    g = synth.rng(300 + n)
    if fmt == "q1":
        w = synth.fp16_normal(g, (n, k), 0.1)
        oc, os_ = oracle.q1_quantize(w)
        f = oracle.Q1
    else:
        t = synth.ternary(g, (n, k))
        s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
        oc, os_ = oracle.t2_pack(t, s)
        f = oracle.T2
    # the unpacker reads the oracle-packed planes; (1,1) T2 code pairs decode as 0
    if fmt == "t2":
        oc = oc.copy()
        oc[0] |= 0x01
        oc[16] |= 0x01
    dense = lowbit.lowbit_unpack(fmt, torch.from_numpy(oc).cuda(), dev_u16(os_), n, k)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(dense), oracle.unpack(f, oc, os_, n, k))


def test_roundtrip_on_device():
    import torch

    n, k = 48, 512
    say("quantize -> unpack round trip on device")
    g = synth.rng(400)
    w = synth.fp16_normal(g, (n, k), 0.1)
    codes, scales = lowbit.lowbit_quantize_q1(dev_u16(w))
    dense = host_u16(lowbit.lowbit_unpack("q1", codes, scales, n, k))
    torch.cuda.synchronize()
    v = w.view(np.float16).astype(np.float64)
    s = np.abs(v).reshape(n, k // 128, 128).max(axis=2).astype(np.float16).view(np.uint16)
    s_full = np.repeat(s, 128, axis=1)
    assert np.array_equal(dense, np.where(v >= 0, s_full, s_full ^ 0x8000))
