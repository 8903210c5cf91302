"""GPU check of lowbit_gemv_noalloc, the decode GEMV that allocates nothing
(its scratch is a static device array instead of a caller workspace).

Through the C ABI (the Python binding passes raw device pointers), its
output must agree with lowbit_gemv's on the same inputs to the GEMV's bar
(floored relative error 1e-3: both sum K-slices with FP32 atomics, so the
last bits may differ between calls), and with the double-precision oracle.
Two calls in a row share the static array; the second has a smaller input,
so it must not pick up anything the first left behind.  Covered for both
codes and for both scratch layouts (b <= 2: a copy of x; b >= 3: x in
matrix-core operand order).
"""
import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import assert_close, dev_u16, say

pytestmark = pytest.mark.gpu

# (n, k, b) of the first, larger call and of the second, smaller one
PAIRS = [
    ((3000, 8192, 1), (700, 1280, 1)),
    ((2500, 6144, 2), (129, 384, 2)),
    ((2000, 4096, 5), (300, 1024, 3)),
    ((1500, 32768, 8), (37, 128, 8)),
]


def _inputs(fmt, n, k, b, seed):
    g = synth.rng(seed)
    if fmt == "q1":
        codes, scales = oracle.q1_quantize(synth.fp16_normal(g, (n, k), 0.1))
    else:
        codes, scales = oracle.t2_pack(synth.ternary(g, (n, k)),
                                       synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2))
    return codes, scales, synth.fp16_normal(g, (b, k))


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_gemv_on_two_calls(fmt, first, second):
    import torch

    for i, (n, k, b) in enumerate((first, second)):
        say(f"gemv_noalloc {fmt} call {i + 1}: n={n} k={k} b={b}")
        codes, scales, x = _inputs(fmt, n, k, b, 9100 + 31 * i + n + b)
        c, s, xd = torch.from_numpy(codes).cuda(), dev_u16(scales), dev_u16(x)
        y_na = lowbit.lowbit_gemv_noalloc(fmt, c, s, n, k, xd)
        y_ws = lowbit.lowbit_gemv(fmt, c, s, n, k, xd)
        torch.cuda.synchronize()
        y_na, y_ws = y_na.cpu().numpy(), y_ws.cpu().numpy()
        assert_close(y_na, y_ws.astype(np.float64), f"noalloc vs gemv {fmt} {n}x{k} b={b}")
        f = oracle.Q1 if fmt == "q1" else oracle.T2
        assert_close(y_na, oracle.gemv(f, codes, scales, n, k, x), f"noalloc vs oracle {fmt}")


def test_noalloc_rejects_requests_beyond_its_scratch():
    import torch

    # b >= 3 stages 32 bytes per k: k = 65536 needs 2 MiB > 1 MiB
    n, k, b = 16, 65536, 3
    say("gemv_noalloc scratch limit")
    c = torch.zeros(lowbit.lowbit_codes_bytes("q1", n, k), dtype=torch.uint8, device="cuda")
    s = torch.zeros(lowbit.lowbit_scales_bytes("q1", n, k) // 2, dtype=torch.float16, device="cuda")
    x = torch.zeros((b, k), dtype=torch.float16, device="cuda")
    with pytest.raises(lowbit.LowbitError) as e:
        lowbit.lowbit_gemv_noalloc("q1", c, s, n, k, x)
    assert e.value.status == 7
