#!/usr/bin/env python3
"""Benchmark of the group-scaled 1-bit / ternary y = W.x path on one MI355X.

Default workload ``t2_lmhead_152k``: the ternary g128 LM-head decode GEMV,
W 151936 x 5120 (2.125 bits per weight: 206,632,960 bytes of codes + scales),
x FP16 [1][5120], y FP32.  One step = one full decode product: the table
preparation of x (lowbit_gemv_prepare) and the weight-streaming accumulation
(lowbit_gemv_accumulate), on the next of R distinct device copies of the
packed weights (R copies >= 1 GiB, four times the 256 MB last-level cache, so
every step reads its weights from HBM).  Inputs are resident in HBM before the
timed region.

Printed: one JSON line with
  value      effective weight GB/s of whole steps (codes + scale bytes / time)
  step_us_stats  min / median / p90 of the per-step time over chains of one
             step per rotated copy (HIP events at the chain boundaries)
  roofline   weight-streaming kernel: algorithmic bytes per launch / its mean
             duration from HIP events recorded on its launch stream (>= 10
             back-to-back chains; min / median / p90 in kernel_us_stats),
             against the 8 TB/s HBM peak and against the measured
             streaming-read ceiling; `traffic` is the HBM bytes per launch that
             rocprofv3 counters gave for the same kernel source, or null
  ceilings   measured on this GPU: a streaming read of 4 GiB (best of a sweep
             of launch shapes), LDS read bandwidth, and a BF16 matrix-core
             loop (include/lowbit_probes.h)
  provenance seeds, SHA-256 of the inputs, library and device versions
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload,
             on all host threads (at most 16) and on one; plus oracle GEMM
             GFLOPS and the CPU FP16 -> Q1 quantisation time
  secondary  the other workloads: decode GEMVs (fused FFN shapes, batch
             sweep), the decode FFN chain (gate+up GEMV, SiLU-gated
             product, down GEMV; eager and as a graph), the two ends of
             a decode step (8-row embedding gather; LM head with top-1
             against the GEMV alone), the ternary quantiser and base-3
             storage conversions, the FP16 -> Q1
             quantiser and the pp512 prefill GEMMs;
             for the GEMVs also the per-step time of a HIP graph that holds
             one step per rotated copy (small matrices are otherwise timed
             by the host's launch rate); the GEMMs' `us` is the median device
             time per GEMM of a replayed graph with one launch per rotated
             set of codes, scales, X and Y (>= 1 GiB: cold), `hot_us` the
             same for 50 launches on one set (cache-resident), and
             `dense_bf16_torch_matmul` a library GEMM on dense BF16 operands
             of the same shape (context)
``--gpus N`` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode GEMV effective weight GB/s (% of MI355X HBM peak); prefill GEMM TFLOPS"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 1 << 30

MAIN_KERNEL = "gemv_main_kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(path):
    """Fingerprint of a kernel source's code: sha256 prefix of the text with
    comments removed and whitespace collapsed, so that the recorded HBM
    counters stay valid across comment-only edits and lapse on any change
    to the code itself."""
    import re

    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# workload construction (device-side seeded generators)

def make_weights(fmt, n, k, seed):
    from bit_matmul_lowbit_amd import lowbit, synth

    if fmt == "q1":
        w = synth.dev_fp16_normal((n, k), 0.1, seed)
        codes, scales = lowbit.lowbit_quantize_q1(w)
        del w
    else:
        t = synth.dev_ternary((n, k), seed)
        s = synth.dev_fp16_uniform((n, k // 128), 0.01, 0.2, seed + 1)
        codes, scales = lowbit.lowbit_pack_t2(t, s)
        del t, s
    return codes, scales


def rotated_copies(codes, scales):
    nbytes = codes.numel() + scales.numel() * 2
    r = max(1, math.ceil(ROTATE_BYTES / nbytes))
    return [(codes.clone(), scales.clone()) for _ in range(r)], nbytes


def sha256_dev(t):
    """SHA-256 (hex prefix) of a device tensor's bytes."""
    import torch

    return hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()[:16]


def provenance(sha, seeds):
    import numpy as np
    import torch

    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"seeds": seeds, "input_sha256": sha, "numpy": np.__version__, "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None), "rocm": rocm,
            "device": torch.cuda.get_device_name(0)}


def stats(xs):
    """min / median / p90 / mean of a list of numbers (rounded for the JSON)."""
    import numpy as np

    a = np.asarray(xs, dtype=np.float64)
    return {"n": int(a.size), "min": float(a.min()), "median": float(np.median(a)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean())}


def rounded(d, nd=3):
    return {k: (round(v, nd) if isinstance(v, float) else v) for k, v in d.items()}


# ---------------------------------------------------------------------------
# GEMV timing

def time_gemv(fmt, n, k, b, seed, steps, warmup, with_kernel_events=True, with_graph=False,
              with_hash=False):
    """Returns dict with step GB/s, ms/step and the mean accumulate-kernel time;
    with_graph adds the per-step time of a HIP graph holding one step per
    rotated copy (no host work between launches).  A step is one lowbit_gemv
    call: prepare + accumulate, or for small matrices the single-launch
    kernel.  The kernel times are those of the two-phase API's accumulate
    kernel (the table or matrix-core kernel)."""
    import torch

    from bit_matmul_lowbit_amd import lowbit, synth

    codes, scales = make_weights(fmt, n, k, seed)
    x = synth.dev_fp16_normal((b, k), 1.0, seed + 2)
    sha = {"codes": sha256_dev(codes), "scales": sha256_dev(scales), "x": sha256_dev(x)} \
        if with_hash else None
    copies, wbytes = rotated_copies(codes, scales)
    del codes, scales
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(lowbit.lowbit_gemv_workspace_bytes(fmt, n, k, b), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()

    def step(i):
        c, s = copies[i % len(copies)]
        lowbit.lowbit_gemv(fmt, c, s, n, k, x, out=y, workspace=ws, stream=st)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # whole steps, wall clock bracketed by device synchronisation; HIP events
    # on the launch stream at every chain boundary (one chain = one step per
    # rotated copy) give the spread of the per-step time over the chains
    nc = len(copies)
    marks = []
    t0 = time.perf_counter()
    for i in range(steps):
        if i % nc == 0:
            marks.append((i, torch.cuda.Event(enable_timing=True)))
            marks[-1][1].record(st)
        step(warmup + i)
    marks.append((steps, torch.cuda.Event(enable_timing=True)))
    marks[-1][1].record(st)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    chain_step_ms = [a[1].elapsed_time(b_[1]) / (b_[0] - a[0]) for a, b_ in zip(marks, marks[1:])
                     if b_[0] - a[0] == nc]

    kernel_ms = kernel_stats = None
    if with_kernel_events:
        # the weight-streaming kernel alone: back-to-back chains of
        # accumulate launches (one per rotated copy), each chain between two
        # HIP events recorded on the launch stream so that dispatch gaps are
        # amortised; at least 10 chains and as many launches as timed steps
        lowbit.lowbit_gemv_prepare(n, k, x, y, ws, stream=st)
        nchains = max(10, -(-steps // nc))
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nchains + 1)]
        evs[0].record(st)
        for j in range(nchains):
            for i in range(nc):
                c, s = copies[i]
                lowbit.lowbit_gemv_accumulate(fmt, c, s, n, k, b, y, ws, stream=st)
            evs[j + 1].record(st)
        torch.cuda.synchronize()
        per = [evs[j].elapsed_time(evs[j + 1]) / nc for j in range(nchains)]
        kernel_ms = sum(per) / len(per)
        kernel_stats = stats([v * 1e3 for v in per])

    graph_ms = None
    if with_graph:
        # one captured step per rotated copy (>= 1 GiB of weights, so still
        # cold), replayed a few times; no host work sits between the launches
        nc = len(copies)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(nc):
                    c, s = copies[i]
                    lowbit.lowbit_gemv(fmt, c, s, n, k, x, out=y, workspace=ws)
        torch.cuda.current_stream().wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        reps = 3
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) / (reps * nc) * 1e3
        del g

    out = {
        "weight_bytes": wbytes,
        "copies": len(copies),
        "ms_per_step": elapsed / steps * 1e3,
        "gbs": wbytes * steps / elapsed / 1e9,
        "kernel_ms": kernel_ms,
        "kernel_us_stats": kernel_stats,
        "step_us_stats": stats([v * 1e3 for v in chain_step_ms]) if chain_step_ms else None,
        "graph_ms_per_step": graph_ms,
        "sha256": sha,
    }
    del copies
    torch.cuda.empty_cache()
    return out


def time_ffn(fmt, k, f, b, seed, steps, warmup):
    """Decode FFN (lowbit_ffn: gate+up GEMV, SiLU-gated product, down GEMV)
    over rotated copies of both matrices: per-step time of eager calls and
    of a HIP graph holding one step per copy."""
    import torch

    from bit_matmul_lowbit_amd import lowbit, synth

    gu_c, gu_s = make_weights(fmt, 2 * f, k, seed)
    dn_c, dn_s = make_weights(fmt, k, f, seed + 7)
    wbytes = gu_c.numel() + gu_s.numel() * 2 + dn_c.numel() + dn_s.numel() * 2
    r = max(1, math.ceil(ROTATE_BYTES / wbytes))
    copies = [(gu_c.clone(), gu_s.clone(), dn_c.clone(), dn_s.clone()) for _ in range(r)]
    del gu_c, gu_s, dn_c, dn_s
    x = synth.dev_fp16_normal((b, k), 1.0, seed + 3)
    y = torch.empty((b, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(lowbit.lowbit_ffn_workspace_bytes(fmt, k, f, b), dtype=torch.uint8, device="cuda")

    def step(i, stream=None):
        a, bs, c, d = copies[i % len(copies)]
        lowbit.lowbit_ffn(fmt, a, bs, c, d, k, f, x, out=y, workspace=ws, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / steps * 1e3

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(len(copies)):
                step(i, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    g.replay()
    torch.cuda.synchronize()
    reps = 3
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) / (reps * len(copies)) * 1e3
    del g, copies
    torch.cuda.empty_cache()
    return {"weight_bytes": wbytes, "eager_us": round(eager_ms * 1e3, 2),
            "graph_us_per_step": round(graph_ms * 1e3, 2),
            "graph_gbs": round(wbytes / (graph_ms * 1e-3) / 1e9, 1)}


def time_ends(n, k, seed):
    """The two ends of a decode step on the ternary LM-head-sized matrix:
    gathering 8 embedding rows, and the LM head with its top-1 (GEMV +
    argmax) against the GEMV alone; graphs over rotated weight copies."""
    import torch

    from bit_matmul_lowbit_amd import lowbit, synth

    codes, scales = make_weights("t2", n, k, seed)
    copies, wbytes = rotated_copies(codes, scales)
    del codes, scales
    x = synth.dev_fp16_normal((1, k), 1.0, seed + 2)
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    val = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(lowbit.lowbit_lm_head_workspace_bytes("t2", n, k, 1), dtype=torch.uint8, device="cuda")
    ids = torch.tensor([11, 4093, 77777, 151000, 5, 99999, 123456, 2048], dtype=torch.int32, device="cuda")
    emb = torch.empty((ids.numel(), k), dtype=torch.float16, device="cuda")

    def graph_us(body):
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(len(copies)):
                    body(i, cap)
        torch.cuda.current_stream().wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / (3 * len(copies)) * 1e6
        del g
        return round(us, 2)

    def lm_head(i, st):
        c, s = copies[i]
        lowbit.lowbit_lm_head("t2", c, s, n, k, x, out=y, idx=idx, val=val, workspace=ws, stream=st)

    def gemv_only(i, st):
        c, s = copies[i]
        lowbit.lowbit_gemv("t2", c, s, n, k, x, out=y, workspace=ws, stream=st)

    def embed(i, st):
        c, s = copies[i]
        lowbit.lowbit_embed("t2", c, s, n, k, ids, out=emb, stream=st)

    out = {"lm_head_argmax_us": graph_us(lm_head), "lm_head_gemv_only_us": graph_us(gemv_only),
           "embed_8_rows_us": graph_us(embed)}
    del copies
    torch.cuda.empty_cache()
    return out


def time_ternary(n, k, seed, steps=10):
    """FP16 -> ternary quantiser and the base-3 storage conversions on an
    LM-head-sized matrix: HBM bytes moved (read + written) per second."""
    import torch

    from bit_matmul_lowbit_amd import lowbit, synth

    w = synth.dev_fp16_normal((n, k), 0.02, seed)
    codes, scales = lowbit.lowbit_quantize_t2(w)
    b3, srm = lowbit.lowbit_t2_to_base3(codes, scales, n, k)
    torch.cuda.synchronize()
    cb, sb = codes.numel(), scales.numel() * 2
    jobs = {
        "quantize_t2": (lambda: lowbit.lowbit_quantize_t2(w, codes, scales), n * k * 2 + cb + sb),
        "t2_to_base3": (lambda: lowbit.lowbit_t2_to_base3(codes, scales, n, k, b3, srm),
                        cb + sb + b3.numel() + srm.numel() * 2),
        "base3_to_t2": (lambda: lowbit.lowbit_base3_to_t2(b3, srm, n, k, codes, scales),
                        b3.numel() + srm.numel() * 2 + cb + sb),
    }
    out = {"base3_bits_per_weight": round(8 * b3.numel() / (n * k) + 16 / 128, 4)}
    for name, (fn, moved) in jobs.items():
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        out[name] = {"us": round(ms * 1e3, 1), "gbs": round(moved / (ms * 1e-3) / 1e9, 1)}
    del w, codes, scales, b3, srm
    torch.cuda.empty_cache()
    return out


def time_quantize(n, k, seed, steps, warmup):
    import torch

    from bit_matmul_lowbit_amd import lowbit, synth

    w = synth.dev_fp16_normal((n, k), 0.02, seed)
    codes = torch.empty(lowbit.lowbit_codes_bytes("q1", n, k), dtype=torch.uint8, device="cuda")
    scales = torch.empty(lowbit.lowbit_scales_bytes("q1", n, k) // 2, dtype=torch.float16, device="cuda")
    for _ in range(warmup):
        lowbit.lowbit_quantize_q1(w, codes, scales)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        lowbit.lowbit_quantize_q1(w, codes, scales)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    moved = n * k * 2 + codes.numel() + scales.numel() * 2
    del w, codes, scales
    torch.cuda.empty_cache()
    return {"bytes_moved": moved, "ms": ms, "gbs": moved / (ms * 1e-3) / 1e9}


def time_gemm(fmt, m, n, k, seed, steps, warmup):
    """pp512 GEMM: per-GEMM device time of a replayed HIP graph of launches,
    (a) cold: one launch per distinct set of (codes, scales, X, Y), the sets
    totalling >= 1 GiB, so weights and activations come from HBM as for
    successive layers; (b) hot: `steps` launches on one set (cache-resident,
    context).  Each graph is replayed 10 times: min / median / p90 per GEMM."""
    import torch

    from bit_matmul_lowbit_amd import lowbit, synth

    codes, scales = make_weights(fmt, n, k, seed)
    x = synth.dev_bf16_normal((m, k), 1.0, seed + 2)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    set_bytes = codes.numel() + scales.numel() * 2 + x.numel() * 2 + y.numel() * 2
    r = max(1, math.ceil(ROTATE_BYTES / set_bytes))
    sets = [(codes.clone(), scales.clone(), x.clone(), torch.empty_like(y)) for _ in range(r)]
    for _ in range(warmup):
        lowbit.lowbit_gemm(fmt, codes, scales, n, k, x, out=y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        lowbit.lowbit_gemm(fmt, codes, scales, n, k, x, out=y)
    b.record()
    torch.cuda.synchronize()
    eager_ms = a.elapsed_time(b) / steps

    def graph_stats(launch_list):
        # the launches captured once and replayed; the kernel writes only its
        # Y, so replays are independent
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for c, sc, xx, yy in launch_list:
                    lowbit.lowbit_gemm(fmt, c, sc, n, k, xx, out=yy, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / len(launch_list) * 1e3)
        del g
        return stats(ts)

    cold = graph_stats(sets)
    hot = graph_stats([(codes, scales, x, y)] * steps)
    del sets
    torch.cuda.empty_cache()
    flops = 2.0 * m * n * k
    us = cold["median"]
    return {"us": us, "tflops": flops / (us * 1e-6) / 1e12,
            "frac_bf16_peak": flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
            "cold_us": rounded(cold, 2), "rotated_sets": r,
            "hot_us": rounded(hot, 2),
            "hot_tflops": round(flops / (hot["median"] * 1e-6) / 1e12, 1),
            "eager_us": eager_ms * 1e3}


# ---------------------------------------------------------------------------
# measured ceilings (context for the roofline): a streaming read over 4 GiB
# and a matrix-core loop, each doing nothing but the one thing it measures

def ceilings():
    import numpy as np
    import torch

    from bit_matmul_lowbit_amd import lowbit

    cus = lowbit.lowbit_probe_cu_count()
    out = {"compute_units": cus}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)  # touch every page before timing
    sink = torch.zeros(64 * cus, dtype=torch.int32, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def read_gbs(bpc, order, reps):
        lowbit.lowbit_probe_stream_read(buf, bpc, sink, order)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a.record()
            lowbit.lowbit_probe_stream_read(buf, bpc, sink, order)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return [nbytes / (t * 1e-3) / 1e9 for t in ts]

    # launch shapes: work-groups per CU x (0: grid-stride, 1: a contiguous
    # share per work-group); the best is timed 10 more times
    sweep = {(bpc, order): max(read_gbs(bpc, order, 3))
             for order in (0, 1) for bpc in (1, 2, 4, 8, 16, 32)}
    best = max(sweep, key=sweep.get)
    rates = read_gbs(best[0], best[1], 10)
    out["stream_read"] = {"bytes": nbytes, "blocks_per_cu": best[0],
                          "order": "grid-stride" if best[1] == 0 else "contiguous share per work-group",
                          "gbs": rounded(stats(rates), 1),
                          "sweep_gbs": {f"{k[0]}/cu,{'stride' if k[1] == 0 else 'share'}": round(v, 1)
                                        for k, v in sweep.items()},
                          "frac_of_hbm_peak": round(float(np.median(rates)) / HBM_PEAK_GBS, 4)}
    del buf, sink
    torch.cuda.empty_cache()

    lsink = torch.zeros(4 * cus * 256, dtype=torch.int32, device="cuda")
    lres = {}
    for bpc in (1, 2, 4):
        lowbit.lowbit_probe_lds_read(100, bpc, lsink)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a.record()
            nb = lowbit.lowbit_probe_lds_read(4000, bpc, lsink)
            b.record()
            torch.cuda.synchronize()
            ts.append(nb / (a.elapsed_time(b) * 1e-3))
        lres[bpc] = ts
    best = max(lres, key=lambda k: float(np.median(lres[k])))
    med = float(np.median(lres[best]))
    out["lds_read"] = {"blocks_per_cu": best, "tb_per_s": round(med / 1e12, 2),
                       "bytes_per_clk_per_cu_at_2p4ghz": round(med / cus / 2.4e9, 1),
                       "sweep_tb_per_s": {str(k): round(float(np.median(v)) / 1e12, 2)
                                          for k, v in lres.items()}}
    del lsink

    msink = torch.zeros(8 * cus * 256, dtype=torch.float32, device="cuda")
    iters = 20000
    res = {}
    for bpc in (1, 2):
        lowbit.lowbit_probe_mfma_bf16(100, bpc, msink)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a.record()
            flops = lowbit.lowbit_probe_mfma_bf16(iters, bpc, msink)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        res[bpc] = [flops / (t * 1e-3) / 1e12 for t in ts]
    best = max(res, key=lambda k: max(res[k]))
    out["mfma_bf16_32x32x16"] = {"blocks_per_cu": best, "waves_per_simd": best,
                                 "tflops": rounded(stats(res[best]), 1),
                                 "frac_of_bf16_peak": round(float(sorted(res[best])[2]) / BF16_PEAK_TFLOPS, 4)}
    del msink

    # the matrix-core GEMV's per-row work (512 weights: byte expansion +
    # one 16x16x32 MFMA) on register data, per SIMD, at one and two waves
    # per SIMD (the kernel runs two); its floor for the 27B matrices, which
    # the 1-bit persistent kernel runs with the LDS-lookup expansion
    esink = torch.zeros(2 * cus * 256, dtype=torch.float32, device="cuda")
    eres = {}
    for mode, name in ((0, "expansion+mfma"), (1, "mfma"), (2, "lut+mfma")):
        for bpc in (1, 2):
            lowbit.lowbit_probe_expand_mfma(mode, 100, bpc, esink)
            torch.cuda.synchronize()
            ts = []
            for _ in range(5):
                a.record()
                steps = lowbit.lowbit_probe_expand_mfma(mode, 4000, bpc, esink)
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e6 / steps)
            eres[f"{name},{bpc}/simd"] = round(float(np.median(ts)), 2)
    step_ns = eres["lut+mfma,2/simd"]
    out["gemv_mfma_row_step"] = {
        "ns_per_row_step_per_simd": eres, "weights_per_row_step": 512,
        "floor_us_at_2_waves_per_simd": {
            f"q1_{n}x{k}": round(n * k / 512 / (4 * cus) * step_ns / 1e3, 2)
            for n, k in ((34816, 5120), (5120, 17408))}}
    del esink
    torch.cuda.empty_cache()
    return out


def dense_gemm_context(m, n, k, seed, reps=50):
    """torch.matmul (hipBLASLt) on dense BF16 operands of the same pp512
    shape: what a tuned library reaches at M = 512 on this GPU (context)."""
    import torch

    from bit_matmul_lowbit_amd import synth

    x = synth.dev_bf16_normal((m, k), 1.0, seed)
    w_nk = synth.dev_bf16_normal((n, k), 0.1, seed + 1)  # W as stored: [n][k]
    w_kn = w_nk.t().contiguous()
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for name, wt in (("x_wT", w_nk.t()), ("x_w", w_kn)):
        for _ in range(10):
            torch.matmul(x, wt, out=y)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a.record()
            for _ in range(reps):
                torch.matmul(x, wt, out=y)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / reps)
        ms = min(ts)
        out[name] = {"us": round(ms * 1e3, 2), "tflops": round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 1)}
    del x, w_nk, w_kn, y
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample, on one thread
# and on all host threads (ctypes releases the GIL during each oracle call)

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rows_rate(call, total_rows, threads, budget_s, chunk):
    """Run call(r0, r) over successive row ranges of `chunk` rows (wrapping
    at total_rows) on `threads` threads until about budget_s of wall time
    has passed; returns (rows done, seconds)."""
    from concurrent.futures import ThreadPoolExecutor

    done = 0
    t0 = time.perf_counter()
    nxt = 0
    with ThreadPoolExecutor(threads) as ex:
        while time.perf_counter() - t0 < budget_s:
            starts = []
            for _ in range(threads):
                r0 = nxt % total_rows
                r = min(chunk, total_rows - r0)
                starts.append((r0, r))
                nxt += r
            list(ex.map(lambda a: call(*a), starts))
            done += sum(r for _, r in starts)
    return done, time.perf_counter() - t0


def cpu_baseline(fmt, n, k, seed, budget_s=6.0):
    import numpy as np
    import torch

    import oracle
    from bit_matmul_lowbit_amd import synth
    from bit_matmul_lowbit_amd.lowbit import lowbit_codes_bytes, lowbit_scales_bytes

    codes, scales = make_weights(fmt, n, k, seed)
    x = synth.dev_fp16_normal((1, k), 1.0, seed + 2)
    hc = codes.cpu().numpy()
    hs = scales.view(torch.int16).cpu().numpy().view(np.uint16)
    hx = x.view(torch.int16).cpu().numpy().view(np.uint16)
    del codes, scales
    f = oracle.Q1 if fmt == "q1" else oracle.T2
    per_row = (lowbit_codes_bytes(fmt, n, k) + lowbit_scales_bytes(fmt, n, k)) / ((n + 15) // 16 * 16)
    threads = max(1, min(16, os.cpu_count() or 1))

    def gemv_rows(r0, r):
        oracle.gemv(f, hc, hs, n, k, hx, row0=r0, nrows=r)

    rows1, t1 = _oracle_rows_rate(gemv_rows, n, 1, budget_s, 2048)
    rowsn, tn = _oracle_rows_rate(gemv_rows, n, threads, budget_s, 2048)
    gbs1 = rows1 * per_row / t1 / 1e9
    gbsn = rowsn * per_row / tn / 1e9

    # oracle GEMM (one X row per call) on the ternary pp512 shape, and the
    # CPU Q1 quantiser on rows of the quantiser workload, all threads
    gm, gn, gk = 512, 6144, 2048
    gc, gs = make_weights("t2", gn, gk, 1004 + gn)
    gx = synth.dev_bf16_normal((gm, gk), 1.0, 1004 + gn + 2)
    hgc = gc.cpu().numpy()
    hgs = gs.view(torch.int16).cpu().numpy().view(np.uint16)
    hgx = gx.view(torch.int16).cpu().numpy().view(np.uint16)
    del gc, gs, gx

    def gemm_rows(m0, mr):
        oracle.gemm(oracle.T2, hgc, hgs, gn, gk, hgx, m0=m0, mrows=mr)

    mrows, tg = _oracle_rows_rate(gemm_rows, gm, threads, budget_s / 2, 1)
    gemm_gflops = 2.0 * mrows * gn * gk / tg / 1e9

    # the whole FP16 -> Q1 quantisation of the 151936 x 5120 matrix, in
    # 1024-row blocks on all threads
    qn, qk = 151936, 5120
    w = synth.dev_fp16_normal((qn, qk), 0.02, 1003)
    hw = w.view(torch.int16).cpu().numpy().view(np.uint16)
    del w
    blocks = [hw[i:i + 1024] for i in range(0, qn, 1024)]
    from concurrent.futures import ThreadPoolExecutor

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda blk: oracle.q1_quantize(np.ascontiguousarray(blk)), blocks))
    q_full_s = time.perf_counter() - t0
    del hw, blocks

    return {"value": round(gbsn, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle GEMV (scalar C, double precision) over row ranges of the same {fmt} "
                      f"{n}x{k} matrix and x, b=1, on {threads} threads ({rowsn} rows in {tn:.1f} s); "
                      f"host: {os.cpu_count()} logical CPUs, {cpu_model()}",
            "single_thread": {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{rows1} rows in {t1:.1f} s"},
            "gemm_pp512_t2_gflops": {"value": round(gemm_gflops, 3), "cores": threads,
                                     "sample": f"{mrows} X rows (the 512 rows of the 512x6144x2048 "
                                               f"ternary GEMM, repeated) in {tg:.1f} s"},
            "q1_quantize_151936x5120_s": {"value": round(q_full_s, 2), "cores": threads,
                                          "sample": "the whole 151936x5120 FP16 matrix"},
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count()}


# ---------------------------------------------------------------------------

def traffic_record(kernel_src):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    r = rec.get(MAIN_KERNEL)
    if not r or r.get("source_sha") != source_sha(kernel_src):
        return None
    return r.get("hbm_bytes_per_launch")


WORKLOADS = {
    "t2_lmhead_152k": ("t2", 151936, 5120, 1, 1003),
    "q1_2048x2048": ("q1", 2048, 2048, 1, 1000),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="t2_lmhead_152k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the streaming-read and matrix-core ceiling probes")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default="all",
                    help="comma-separated secondary groups to run: gemv, quantize, ffn, "
                         "ternary, ends, gemm (default: all)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    groups = {"gemv", "quantize", "ffn", "ternary", "ends", "gemm"}
    chosen = groups if args.secondary == "all" else set(args.secondary.split(","))
    if not chosen <= groups:
        ap.error(f"--secondary: unknown group(s) {sorted(chosen - groups)}")

    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from bit_matmul_lowbit_amd import lowbit

    lowbit.load()  # fail loudly if the HIP library is missing

    fmt, n, k, b, seed = WORKLOADS[args.workload]
    log(f"[bench] {args.workload}: {fmt} {n}x{k} b={b}, {args.steps} steps, {args.warmup} warmup")
    r = time_gemv(fmt, n, k, b, seed, args.steps, args.warmup, with_hash=True)
    achieved = r["weight_bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
    log(f"[bench] step {r['ms_per_step'] * 1e3:.2f} us, {r['gbs']:.1f} GB/s; "
        f"accumulate kernel {r['kernel_ms'] * 1e3:.2f} us, {achieved:.1f} GB/s")

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 1 GiB device copies done")
        del src, dst

    kernel_src = os.path.join(ROOT, "bit_matmul_lowbit_amd", "csrc", "gemv.hip")
    result = {
        "metric": METRIC,
        "value": round(r["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "format": "ternary g128, 2 bits + FP16 scale per 128 (2.125 bpw)" if fmt == "t2"
            else "Q1_0_g128, 1 bit + FP16 scale per 128 (1.125 bpw)",
            "n": n, "k": k, "batch": b,
            "weight_bytes_per_step": r["weight_bytes"],
            "rotated_weight_copies": r["copies"],
            "frac_of_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": MAIN_KERNEL,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_record(kernel_src),
            "kernel_us": round(r["kernel_ms"] * 1e3, 3),
            "kernel_us_stats": rounded(r["kernel_us_stats"], 3),
        },
        "step_us_stats": rounded(r["step_us_stats"], 3) if r["step_us_stats"] else None,
        "provenance": provenance(r["sha256"], {"weights": seed, "x": seed + 2}),
    }

    if not args.no_ceilings:
        log("[bench] ceiling probes ...")
        ceil = ceilings()
        result["ceilings"] = ceil
        med = ceil["stream_read"]["gbs"]["median"]
        result["roofline"]["frac_of_measured_stream_read"] = round(achieved / med, 4)
        log(f"[bench] ceilings: {ceil}")

    if not args.no_secondary:
        sec = {}
        for name, (f2, n2, k2, seeds) in {
            "q1_2048x2048_b1": ("q1", 2048, 2048, 1000),
            "t2_ffn_1p7b_up_6144x2048_b1": ("t2", 6144, 2048, 1001),
            "t2_ffn_1p7b_down_2048x6144_b1": ("t2", 2048, 6144, 1001),
            "q1_ffn_27b_gateup_34816x5120": ("q1", 34816, 5120, 1002),
            "q1_ffn_27b_down_5120x17408": ("q1", 5120, 17408, 1002),
        }.items() if "gemv" in chosen else ():
            for b2 in ([1, 2, 5, 8] if "27b" in name else [1]):
                key = name if "27b" not in name else f"{name}_b{b2}"
                rr = time_gemv(f2, n2, k2, b2, seeds, 50, 10, with_graph=True)
                sec[key] = {"gbs": round(rr["gbs"], 1), "us_per_step": round(rr["ms_per_step"] * 1e3, 2),
                            "kernel_gbs": round(rr["weight_bytes"] / (rr["kernel_ms"] * 1e-3) / 1e9, 1),
                            "kernel_us": rounded(rr["kernel_us_stats"], 2),
                            "graph_us_per_step": round(rr["graph_ms_per_step"] * 1e3, 2),
                            "graph_gbs": round(rr["weight_bytes"] / (rr["graph_ms_per_step"] * 1e-3) / 1e9, 1)}
                log(f"[bench] {key}: {sec[key]}")
        if "quantize" in chosen:
            q = time_quantize(151936, 5120, 1003, 20, 3)
            sec["q1_quantize_151936x5120"] = {"gbs": round(q["gbs"], 1), "us": round(q["ms"] * 1e3, 1),
                                              "bytes_moved": q["bytes_moved"]}
            log(f"[bench] quantize: {sec['q1_quantize_151936x5120']}")
        for key, (ff, kf, fff, bf) in {
                "ffn_q1_27b_k5120_f17408_b1": ("q1", 5120, 17408, 1),
                "ffn_q1_27b_k5120_f17408_b5": ("q1", 5120, 17408, 5),
                "ffn_t2_1p7b_k2048_f6144_b1": ("t2", 2048, 6144, 1)}.items() if "ffn" in chosen else ():
            sec[key] = time_ffn(ff, kf, fff, bf, 1100 + fff + bf, 30, 5)
            log(f"[bench] {key}: {sec[key]}")
        if "ternary" in chosen:
            sec["ternary_151936x5120"] = time_ternary(151936, 5120, 1950)
            log(f"[bench] ternary_151936x5120: {sec['ternary_151936x5120']}")
        if "ends" in chosen:
            sec["ends_t2_151936x5120_b1"] = time_ends(151936, 5120, 1900)
            log(f"[bench] ends_t2_151936x5120_b1: {sec['ends_t2_151936x5120_b1']}")
        for key, (f2, m2, n2, k2) in {"gemm_pp512_t2_512x6144x2048": ("t2", 512, 6144, 2048),
                                       "gemm_pp512_q1_512x2048x6144": ("q1", 512, 2048, 6144)}.items() \
                if "gemm" in chosen else ():
            g = time_gemm(f2, m2, n2, k2, 1004 + n2, 50, 10)
            sec[key] = {"tflops": round(g["tflops"], 2), "us": round(g["us"], 2),
                        "frac_bf16_peak": round(g["frac_bf16_peak"], 4),
                        "timing": "cold: median over 10 replays of a graph with one GEMM per "
                                  f"rotated set of codes, scales, X and Y ({g['rotated_sets']} sets "
                                  ">= 1 GiB)",
                        "cold_us": g["cold_us"], "hot_us": g["hot_us"], "hot_tflops": g["hot_tflops"],
                        "eager_us": round(g["eager_us"], 2),
                        "dense_bf16_torch_matmul": dense_gemm_context(m2, n2, k2, 77 + n2)}
            log(f"[bench] {key}: {sec[key]}")
        result["secondary"] = sec

    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(fmt, n, k, seed)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
