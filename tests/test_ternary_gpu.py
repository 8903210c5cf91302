"""GPU parity of the ternary quantiser and the base-3 storage conversions
against the oracle, bit for bit.

[P2 "Como funciona la compresion": w = s t with t in {-1, 0, +1}, one FP16
scale per 128, ~1.71 bits per weight.]  The rounding rule is this
library's reading (the pages give none): s = max |w|, t = sign(w) iff
2|w| > s (ties to 0).
"""
import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import dev_u16, host_u16, host_u8, say

pytestmark = pytest.mark.gpu


def _oracle_codes(w16):
    t, s = oracle.t2_quantize(w16)
    return (t, s) + oracle.t2_pack(t, s)


@pytest.mark.parametrize("n,k", [(16, 128), (37, 384), (1, 1280), (200, 640)])
def test_quantize_t2_matches_oracle(n, k):
    import torch

    say(f"quantize_t2 n={n} k={k}")
    g = synth.rng(600 + n + k)
    w = synth.fp16_normal(g, (n, k), 0.1)
    _, _, oc, os_ = _oracle_codes(w)
    codes, scales = lowbit.lowbit_quantize_t2(dev_u16(w))
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(codes), oc)
    assert np.array_equal(host_u16(scales), os_)


def test_quantize_t2_edge_groups():
    import torch

    say("quantize_t2 edge groups")
    # every FP16 magnitude against a few group maxima (first weight), both
    # signs; plus ties, zeros, subnormals, infinities and NaNs
    mags = np.arange(0x7C01, dtype=np.uint32).astype(np.uint16)
    rows = []
    for S in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x3C01, 0x7BFF, 0x7C00):
        cand = mags[mags <= S]
        vals = cand | ((np.arange(cand.size) % 2).astype(np.uint16) << 15)
        per = 127
        groups = (vals.size + per - 1) // per
        flat = np.zeros(groups * per, np.uint16)
        flat[:vals.size] = vals
        grp = np.zeros((groups, 128), np.uint16)
        grp[:, 0] = S
        grp[:, 1:] = flat.reshape(groups, per)
        rows.append(grp.reshape(-1))
    special = np.zeros(128 * 4, np.uint16)
    special[:6] = [0x3C00, 0x3800, 0xB800, 0x3801, 0x0000, 0x8000]   # ties +-0.5, just above, +-0
    special[384:387] = [0x3C00, 0x7E00, 0xBC00]                       # a NaN weight in the group
    special[128:131] = [0xFE00, 0x3C00, 0x0001]                       # NaN maximum
    special[256:259] = [0xFC00, 0x7BFF, 0x0400]                       # -inf maximum
    rows.append(special)
    width = max(r.size for r in rows)
    width = (width + 127) // 128 * 128
    w = np.zeros((len(rows), width), np.uint16)
    for i, r in enumerate(rows):
        w[i, :r.size] = r
    _, _, oc, os_ = _oracle_codes(w)
    codes, scales = lowbit.lowbit_quantize_t2(dev_u16(w))
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(scales), os_)
    assert np.array_equal(host_u8(codes), oc)


def test_quantize_t2_full_lm_head_size():
    import torch

    n, k = 151936, 5120
    say(f"quantize_t2 full n={n} k={k}")
    w = synth.dev_fp16_normal((n, k), 0.02, 1950)
    codes, scales = lowbit.lowbit_quantize_t2(w)
    torch.cuda.synchronize()
    hw = host_u16(w)
    del w
    _, _, oc, os_ = _oracle_codes(hw)
    assert np.array_equal(host_u16(scales), os_)
    assert np.array_equal(host_u8(codes), oc)


# (37, 2944): two whole 1280-weight blocks of the conversion kernels plus a
# partial one, and 589 bytes per row (rows start at unaligned addresses)
@pytest.mark.parametrize("n,k", [(16, 128), (37, 384), (5, 1280), (333, 640), (37, 2944)])
def test_base3_round_trip_matches_oracle(n, k):
    import torch

    say(f"base3 n={n} k={k}")
    g = synth.rng(700 + n + k)
    t = synth.ternary(g, (n, k))
    s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
    oc, os_ = oracle.t2_pack(t, s)
    b3, srm = lowbit.lowbit_t2_to_base3(torch.from_numpy(oc).cuda(), dev_u16(os_), n, k)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(b3), oracle.base3_pack(t))
    assert np.array_equal(host_u16(srm), s)
    # back to two planes: the oracle's packing of the decoded trits
    bb = oracle.base3_pack(t)
    bb[0, 0] = 250  # a byte the packer never writes: fifth digit mod 3
    codes, scales = lowbit.lowbit_base3_to_t2(torch.from_numpy(bb).cuda(), dev_u16(s), n, k)
    torch.cuda.synchronize()
    want_c, want_s = oracle.t2_pack(oracle.base3_unpack(bb, n, k), s)
    assert np.array_equal(host_u8(codes), want_c)
    assert np.array_equal(host_u16(scales), want_s)
