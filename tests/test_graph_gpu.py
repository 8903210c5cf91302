"""HIP graph capture of the decode GEMV and FFN.

Each call is captured once and the graph replayed several times, with eager
work on the same output and workspace between the replays (the output
filled with a different value, the workspace with a byte pattern), and every
replay is checked against the double-precision oracle.  The library records
only kernel launches (y and h are zeroed by its own kernels, never by a
memset node), so every replay must give the result of a fresh call.  Cases
cover each GEMV path (single launch, subset-sum tables, matrix cores), the
allocation-free entry point, and the three FFN chains.
"""
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import assert_close, dev_u16, say
from tests.test_ffn_gpu import _ffn_ok

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _weights(fmt, n, k, g):
    if fmt == "q1":
        return oracle.q1_quantize(synth.fp16_normal(g, (n, k), 0.1))
    t = synth.ternary(g, (n, k))
    s = synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2)
    return oracle.t2_pack(t, s)


def _capture(fn):
    import torch

    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            fn()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    return graph


# (fmt, n, k, b, path lowbit_gemv takes)
GEMV = [("q1", 2048, 2048, 1, "single launch"), ("t2", 6144, 2048, 5, "single launch, x in LDS"),
        ("t2", 4096, 2048, 2, "single launch, half tiles"), ("q1", 8192, 2048, 1, "single launch, whole tiles"),
        ("q1", 1024, 12288, 1, "tables"),
        ("t2", 1040, 12288, 2, "tables"), ("q1", 2048, 8192, 5, "matrix cores"),
        ("t2", 4112, 4224, 8, "matrix cores")]


@pytest.mark.parametrize("fmt,n,k,b,path", GEMV)
@pytest.mark.parametrize("entry", ["lowbit_gemv", "lowbit_gemv_noalloc"])
def test_gemv_graph_replays(fmt, n, k, b, path, entry):
    import torch

    say(f"graph {entry} {fmt} {n}x{k} b={b} ({path})")
    g = synth.rng(5000 + n + k + b)
    codes, scales = _weights(fmt, n, k, g)
    x = synth.fp16_normal(g, (b, k))
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemv(f, codes, scales, n, k, x)
    c, s, xd = torch.from_numpy(codes).cuda(), dev_u16(scales), dev_u16(x)
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(lowbit.lowbit_gemv_workspace_bytes(fmt, n, k, b), 16), dtype=torch.uint8,
                     device="cuda")
    if entry == "lowbit_gemv":
        def call():
            lowbit.lowbit_gemv(fmt, c, s, n, k, xd, out=y, workspace=ws)
    else:
        def call():
            lowbit.lowbit_gemv_noalloc(fmt, c, s, n, k, xd, out=y)
    call()  # eager first: loads the library and, for the no-alloc entry, its scratch address
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), ref, f"eager {entry} {fmt} {n}x{k} b={b}")
    graph = _capture(call)
    for rep in range(REPLAYS):
        y.fill_(float(rep) + 7.0)
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy(), ref, f"replay {rep} {entry} {fmt} {n}x{k} b={b}")


# (fmt, k, f, b, chain)
FFN = [("t2", 1024, 4096, 1, "two single-launch GEMVs"), ("q1", 2176, 8320, 1, "table chain"),
       ("q1", 2048, 4224, 3, "matrix-core chain")]


@pytest.mark.parametrize("fmt,k,f,b,chain", FFN)
def test_ffn_graph_replays(fmt, k, f, b, chain):
    import torch

    say(f"graph ffn {fmt} k={k} f={f} b={b} ({chain})")
    g = synth.rng(5100 + k + f + b)
    gu = _weights(fmt, 2 * f, k, g)
    dn = _weights(fmt, k, f, g)
    x = synth.fp16_normal(g, (b, k))
    of = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.ffn(of, gu[0], gu[1], dn[0], dn[1], k, f, x)
    guc, gus = torch.from_numpy(gu[0]).cuda(), dev_u16(gu[1])
    dnc, dns = torch.from_numpy(dn[0]).cuda(), dev_u16(dn[1])
    xd = dev_u16(x)
    y = torch.empty((b, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(lowbit.lowbit_ffn_workspace_bytes(fmt, k, f, b), dtype=torch.uint8,
                     device="cuda")

    def call():
        lowbit.lowbit_ffn(fmt, guc, gus, dnc, dns, k, f, xd, out=y, workspace=ws)

    call()
    torch.cuda.synchronize()
    _ffn_ok(y.cpu().numpy(), ref, f"eager ffn {fmt} k={k} f={f} b={b}")
    graph = _capture(call)
    for rep in range(REPLAYS):
        y.fill_(float(rep) - 3.0)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _ffn_ok(y.cpu().numpy(), ref, f"replay {rep} ffn {fmt} k={k} f={f} b={b}")
