"""The ceiling probes (include/lowbit_probes.h) on the GPU: each launches,
returns LOWBIT_OK, and leaves its sink as it was (a sink is written only if
a fold of the probe's data equals a fixed constant, which these runs never
produce).  Their rates are bench.py's business; here only that they run.
"""
import pytest

from bit_matmul_lowbit_amd import lowbit
from tests.helpers import say

pytestmark = pytest.mark.gpu


def test_probes_run_and_leave_their_sinks():
    import torch

    cus = lowbit.lowbit_probe_cu_count()
    assert 1 <= cus <= 1024
    buf = torch.ones(1 << 24, dtype=torch.uint8, device="cuda")
    for order in (0, 1):
        say(f"probe stream read order {order}")
        sink = torch.zeros(2 * cus, dtype=torch.int32, device="cuda")
        lowbit.lowbit_probe_stream_read(buf, 2, sink, order)
        torch.cuda.synchronize()
        assert int(sink.abs().sum()) == 0
    say("probe lds read")
    sink = torch.zeros(cus * 256, dtype=torch.int32, device="cuda")
    assert lowbit.lowbit_probe_lds_read(10, 1, sink) == cus * 256 * 10 * 8 * 16
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    say("probe mfma bf16")
    fsink = torch.zeros(cus * 256, dtype=torch.float32, device="cuda")
    assert lowbit.lowbit_probe_mfma_bf16(10, 1, fsink) == cus * 4 * 10 * 4 * 2 * 32 * 32 * 16
    torch.cuda.synchronize()
    assert float(fsink.abs().sum()) == 0.0
    for mode in (0, 1, 2):
        say(f"probe expand+mfma mode {mode}")
        fsink = torch.zeros(2 * cus * 256, dtype=torch.float32, device="cuda")
        assert lowbit.lowbit_probe_expand_mfma(mode, 12, 2, fsink) == 2 * 12 * 16
        torch.cuda.synchronize()
        assert float(fsink.abs().sum()) == 0.0
