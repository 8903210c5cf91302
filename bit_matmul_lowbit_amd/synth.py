"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and rounds them to the storage formats
(FP16 / BF16 / int8); it holds none of the method's arithmetic (no scale rule,
no sign rule, no packing, no products).  Both the HIP path and the CPU oracle
consume the same arrays it returns.

Host generator: numpy ``Generator(PCG64(seed))``; FP16 values are the
round-to-nearest-even images of float64 normal samples (numpy ``astype``),
BF16 values those of float64 samples rounded by torch's nearest-even cast.
Device generator (for the full-size workloads, to avoid multi-GB host
arrays): torch's seeded CUDA generator, FP16/BF16 rounded from float32 samples.

Workloads (the names say what they are; sizes as stated):
  q1_2048x2048      1-bit W 2048x2048 from FP16 N(0, 0.1); x FP16 N(0,1), b=1
  t2_ffn_1p7b       ternary gate/up 6144x2048 and down 2048x6144; t with
                    P(-1,0,+1) = (.25,.5,.25); scales FP16 U[0.01, 0.2]; b=1
  q1_ffn_27b        1-bit fused gate+up 34816x5120 and down 5120x17408 from
                    FP16 N(0, 0.1); b in {1,2,5,8}
  t2_lmhead_152k    ternary LM head 151936x5120 (codes as t2_ffn_1p7b), b=1;
                    plus quantisation of an FP16 N(0, 0.02) 151936x5120 matrix
  gemm_pp512        X BF16 N(0,1) 512x2048 by ternary W 6144x2048, and X BF16
                    N(0,1) 512x6144 by 1-bit W 2048x6144 (from FP16 N(0,0.1))
"""
from __future__ import annotations

import numpy as np

TERNARY_PROBS = (0.25, 0.5, 0.25)  # P(t = -1), P(t = 0), P(t = +1)
SCALE_RANGE = (0.01, 0.2)


def rng(seed: int, stream: int = 0) -> np.random.Generator:
    """Independent PCG64 stream `stream` of master seed `seed`."""
    ss = np.random.SeedSequence(seed)
    child = ss.spawn(stream + 1)[stream]
    return np.random.Generator(np.random.PCG64(child))


def fp16_normal(g: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """FP16 patterns (uint16) of N(0, sigma^2) samples, nearest-even rounded."""
    return (g.standard_normal(shape) * sigma).astype(np.float16).view(np.uint16)


def fp16_uniform(g: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return g.uniform(lo, hi, shape).astype(np.float16).view(np.uint16)


def bf16_normal(g: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """BF16 patterns (uint16) of N(0, sigma^2) samples, nearest-even rounded."""
    import torch

    v = torch.from_numpy(g.standard_normal(shape) * sigma).to(torch.bfloat16)
    return v.view(torch.int16).numpy().view(np.uint16).copy()


def ternary(g: np.random.Generator, shape, probs=TERNARY_PROBS) -> np.ndarray:
    """int8 values in {-1, 0, +1} with probabilities `probs`."""
    u = g.random(shape)
    out = np.zeros(shape, dtype=np.int8)
    out[u < probs[0]] = -1
    out[u >= probs[0] + probs[1]] = 1
    return out


# ---------------------------------------------------------------------------
# device-side generators (torch, seeded CUDA generator)

def _dev_gen(seed: int, device):
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def dev_fp16_normal(shape, sigma: float, seed: int, device="cuda"):
    import torch

    gen = _dev_gen(seed, device)
    return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * sigma).to(torch.float16)


def dev_bf16_normal(shape, sigma: float, seed: int, device="cuda"):
    import torch

    gen = _dev_gen(seed, device)
    return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * sigma).to(torch.bfloat16)


def dev_ternary(shape, seed: int, device="cuda", probs=TERNARY_PROBS):
    import torch

    gen = _dev_gen(seed, device)
    u = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    t = torch.zeros(shape, dtype=torch.int8, device=device)
    t[u < probs[0]] = -1
    t[u >= probs[0] + probs[1]] = 1
    return t


def dev_fp16_uniform(shape, lo: float, hi: float, seed: int, device="cuda"):
    import torch

    gen = _dev_gen(seed, device)
    return (torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * (hi - lo) + lo).to(torch.float16)


# ---------------------------------------------------------------------------
# workload table

WORKLOADS = {
    "q1_2048x2048": {
        "seed": 1000,
        "gemv": [("q1", 2048, 2048)],
        "weight_sigma": 0.1,
        "batches": [1],
    },
    "t2_ffn_1p7b": {
        "seed": 1001,
        "gemv": [("t2", 6144, 2048), ("t2", 6144, 2048), ("t2", 2048, 6144)],
        "batches": [1],
    },
    "q1_ffn_27b": {
        "seed": 1002,
        "gemv": [("q1", 34816, 5120), ("q1", 5120, 17408)],
        "weight_sigma": 0.1,
        "batches": [1, 2, 5, 8],
    },
    "t2_lmhead_152k": {
        "seed": 1003,
        "gemv": [("t2", 151936, 5120)],
        "batches": [1],
        "quantize": (151936, 5120, 0.02),
    },
    "gemm_pp512": {
        "seed": 1004,
        "gemm": [("t2", 6144, 2048, 512), ("q1", 2048, 6144, 512)],
        "weight_sigma": 0.1,
    },
}
