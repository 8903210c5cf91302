"""Guard canaries: every device output of the library, at ragged sizes, sits
between 4 KiB of a known byte pattern on each side; after the call the
pattern must be intact (no kernel wrote outside its output), and FP32
outputs must hold no element left at the fill pattern (every element was
written).  Bounds and pad-row guards of the kernels are observed directly
here; the values are checked against the oracle in the other GPU tests."""
import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import dev_u16, guarded, guards_intact, say

pytestmark = pytest.mark.gpu

FILL32 = 0xA5A5A5A5


def _all_written_f32(t):
    import torch

    return not bool((t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32) == FILL32).any())


def _weights(fmt, n, k, seed):
    import torch

    g = synth.rng(seed)
    if fmt == "q1":
        c, s = oracle.q1_quantize(synth.fp16_normal(g, (n, k), 0.1))
    else:
        c, s = oracle.t2_pack(synth.ternary(g, (n, k)), synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2))
    return g, torch.from_numpy(c).cuda(), dev_u16(s)


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("n,k", [(37, 384), (1, 128), (300, 1280), (1001, 2176)])
def test_pack_outputs_stay_in_bounds(fmt, n, k):
    import torch

    say(f"canary pack {fmt} n={n} k={k}")
    g = synth.rng(5000 + n + k)
    cb = lowbit.lowbit_codes_bytes(fmt, n, k)
    sb = lowbit.lowbit_scales_bytes(fmt, n, k)
    rc, codes = guarded((cb,), torch.uint8)
    rs, scales = guarded((sb // 2,), torch.float16)
    if fmt == "q1":
        lowbit.lowbit_quantize_q1(dev_u16(synth.fp16_normal(g, (n, k), 0.1)), codes, scales)
    else:
        t = torch.from_numpy(synth.ternary(g, (n, k))).cuda()
        lowbit.lowbit_pack_t2(t, dev_u16(synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)), codes, scales)
    torch.cuda.synchronize()
    assert guards_intact(rc) and guards_intact(rs)
    ro, out = guarded((n, k), torch.float16)
    lowbit.lowbit_unpack(fmt, codes, scales, n, k, out)
    torch.cuda.synchronize()
    assert guards_intact(ro)
    if fmt == "t2":
        rq, qc = guarded((cb,), torch.uint8)
        rqs, qs = guarded((sb // 2,), torch.float16)
        lowbit.lowbit_quantize_t2(dev_u16(synth.fp16_normal(g, (n, k), 0.1)), qc, qs)
        r3, b3 = guarded((n, (k + 4) // 5), torch.uint8)
        r3s, b3s = guarded((n, k // 128), torch.float16)
        lowbit.lowbit_t2_to_base3(codes, scales, n, k, b3, b3s)
        rb, back = guarded((cb,), torch.uint8)
        rbs, backs = guarded((sb // 2,), torch.float16)
        lowbit.lowbit_base3_to_t2(b3, b3s, n, k, back, backs)
        torch.cuda.synchronize()
        for r in (rq, rqs, r3, r3s, rb, rbs):
            assert guards_intact(r)
        assert torch.equal(back, codes)


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("n,k,b", [(37, 384, 1), (1001, 2176, 2), (300, 1280, 5), (129, 4224, 8),
                                   (16, 128, 3)])
def test_gemv_outputs_stay_in_bounds(fmt, n, k, b):
    import torch

    say(f"canary gemv {fmt} n={n} k={k} b={b}")
    g, c, s = _weights(fmt, n, k, 5100 + n + b)
    x = dev_u16(synth.fp16_normal(g, (b, k)))
    ry, y = guarded((b, n), torch.float32)
    rw, ws = guarded((lowbit.lowbit_gemv_workspace_bytes(fmt, n, k, b),), torch.uint8)
    lowbit.lowbit_gemv(fmt, c, s, n, k, x, out=y, workspace=ws)
    torch.cuda.synchronize()
    assert guards_intact(ry) and guards_intact(rw) and _all_written_f32(y)
    ry2, y2 = guarded((b, n), torch.float32)
    lowbit.lowbit_gemv_noalloc(fmt, c, s, n, k, x, out=y2)
    torch.cuda.synchronize()
    assert guards_intact(ry2) and _all_written_f32(y2)
    ri, idx = guarded((b,), torch.int32)
    rv, val = guarded((b,), torch.float32)
    rl, yl = guarded((b, n), torch.float32)
    rlw, lws = guarded((lowbit.lowbit_lm_head_workspace_bytes(fmt, n, k, b),), torch.uint8)
    lowbit.lowbit_lm_head(fmt, c, s, n, k, x, out=yl, idx=idx, val=val, workspace=lws)
    torch.cuda.synchronize()
    for r in (ri, rv, rl, rlw):
        assert guards_intact(r)
    assert _all_written_f32(yl) and _all_written_f32(val)
    ids = torch.tensor([0, n - 1, n // 2, n, -1], dtype=torch.int32, device="cuda")
    re, emb = guarded((ids.numel(), k), torch.float16)
    lowbit.lowbit_embed(fmt, c, s, n, k, ids, out=emb)
    torch.cuda.synchronize()
    assert guards_intact(re)


# shapes that reach every GEMM configuration (including the team kernel at
# 512 x 6144 and 500 x 6100) with ragged m and n
@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("m,n,k", [(3, 37, 256), (130, 300, 384), (500, 6100, 384),
                                   (512, 6144, 1280), (600, 2000, 384), (450, 6144, 128)])
def test_gemm_outputs_stay_in_bounds(fmt, m, n, k):
    import torch

    say(f"canary gemm {fmt} m={m} n={n} k={k}")
    g, c, s = _weights(fmt, n, k, 5200 + m + n)
    x = dev_u16(synth.bf16_normal(g, (m, k)), "bfloat16")
    rb, yb = guarded((m, n), torch.bfloat16)
    rf, yf = guarded((m, n), torch.float32)
    lowbit.lowbit_gemm(fmt, c, s, n, k, x, out=yb)
    lowbit.lowbit_gemm_f32(fmt, c, s, n, k, x, out=yf)
    torch.cuda.synchronize()
    assert guards_intact(rb) and guards_intact(rf) and _all_written_f32(yf)


@pytest.mark.parametrize("fmt,k,f,b", [("q1", 256, 384, 1), ("t2", 384, 640, 2), ("q1", 640, 384, 5)])
def test_ffn_outputs_stay_in_bounds(fmt, k, f, b):
    import torch

    say(f"canary ffn {fmt} k={k} f={f} b={b}")
    g, gc, gs = _weights(fmt, 2 * f, k, 5300 + f)
    _, dc, ds = _weights(fmt, k, f, 5301 + f)
    x = dev_u16(synth.fp16_normal(g, (b, k)))
    ry, y = guarded((b, k), torch.float32)
    rw, ws = guarded((lowbit.lowbit_ffn_workspace_bytes(fmt, k, f, b),), torch.uint8)
    lowbit.lowbit_ffn(fmt, gc, gs, dc, ds, k, f, x, out=y, workspace=ws)
    h = torch.from_numpy(np.random.default_rng(1).standard_normal((b, 2 * f)).astype(np.float32)).cuda()
    rz, z = guarded((b, f), torch.float16)
    lowbit.lowbit_silu_mul(h, out=z)
    torch.cuda.synchronize()
    assert guards_intact(ry) and guards_intact(rw) and guards_intact(rz) and _all_written_f32(y)
