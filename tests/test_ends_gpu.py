"""GPU parity of the two ends of a decode step: the embedding-row gather and
the LM head's top-1 token.

[P2 "Como funciona la compresion", P4: embeddings and the LM head are
low-bit; P5 "Detalles tecnicos": decode checked by top-1 token match.]

* lowbit_embed must equal the oracle's unpacked rows bit for bit (zeros for
  ids outside the vocabulary);
* lowbit_argmax, on a given y, must give numpy's argmax (first maximum,
  NaN largest) exactly;
* lowbit_lm_head's logits follow the GEMV bound (floored 1e-3); its top-1 is
  unique only when the oracle's best logit leads the runner-up by more
  than the two sides' error, so the test checks that the returned index is
  the GPU's own maximum, that its oracle logit is within the error bound of
  the oracle's maximum, and that it is the oracle's argmax whenever that
  lead is clear.
"""
import numpy as np
import pytest

import oracle
from bit_matmul_lowbit_amd import lowbit, synth
from tests.helpers import TOL, assert_close, dev_u16, full_weights, host_u16, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["q1", "t2"])
@pytest.mark.parametrize("n,k", [(37, 384), (1000, 128), (16, 1280)])
def test_embed_matches_oracle_rows(fmt, n, k):
    import torch

    say(f"embed {fmt} n={n} k={k}")
    g = synth.rng(500 + n + k)
    if fmt == "q1":
        codes, scales = oracle.q1_quantize(synth.fp16_normal(g, (n, k), 0.1))
    else:
        codes, scales = oracle.t2_pack(synth.ternary(g, (n, k)), synth.fp16_uniform(g, (n, k // 128), 0.01, 0.2))
    of = oracle.Q1 if fmt == "q1" else oracle.T2
    dense = oracle.unpack(of, codes, scales, n, k)
    ids = np.concatenate([[0, n - 1, n // 2, n - 1, -1, n, 1 << 30], g.integers(0, n, 40)]).astype(np.int32)
    out = lowbit.lowbit_embed(fmt, torch.from_numpy(codes).cuda(), dev_u16(scales), n, k,
                              torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    got = host_u16(out)
    valid = (ids >= 0) & (ids < n)
    assert np.array_equal(got[valid], dense[ids[valid]])
    assert not got[~valid].any()


def _tile_rows(of, hc, hs, k, t):
    """The 16 dequantised rows of tile t: the oracle unpacks that tile's
    slice of the planes (both are tile-major), not all 151936 rows."""
    cb = (k // 8) * 16 * (1 if of == oracle.Q1 else 2)
    sb = (k // 128) * 16
    return oracle.unpack(of, hc[t * cb:(t + 1) * cb], hs[t * sb:(t + 1) * sb], 16, k)


def test_embed_full_vocabulary():
    import torch

    n, k = 151936, 5120
    say(f"embed t2 full n={n} k={k}")
    codes, scales, hc, hs = full_weights("t2", n, k, 1700)
    ids = np.array([0, 1, 15, 16, 75968, n - 17, n - 1, 12345], np.int32)
    out = host_u16(lowbit.lowbit_embed("t2", codes, scales, n, k, torch.from_numpy(ids).cuda()))
    torch.cuda.synchronize()
    for j, r in enumerate(ids):
        assert np.array_equal(out[j], _tile_rows(oracle.T2, hc, hs, k, int(r) // 16)[int(r) % 16]), r


def test_argmax_exact_semantics():
    import torch

    say("argmax semantics")
    g = np.random.default_rng(81)
    n = 5000
    rows = []
    rows.append(g.standard_normal(n).astype(np.float32))
    r = g.standard_normal(n).astype(np.float32); r[[7, 4000]] = r.max() + 1; rows.append(r)  # tie: first
    rows.append(np.full(n, -np.inf, np.float32))                                             # all -inf
    r = -np.abs(g.standard_normal(n)).astype(np.float32); r[50] = -0.0; r[100] = 0.0; rows.append(r)  # -0 == +0
    r = g.standard_normal(n).astype(np.float32); r[[300, 2000]] = np.nan; rows.append(r)      # NaN wins
    r = g.standard_normal(n).astype(np.float32); r[n - 1] = 1e30; rows.append(r)              # last element
    y = np.stack(rows)
    idx, val = lowbit.lowbit_argmax(torch.from_numpy(y).cuda())
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    want = np.argmax(y, axis=1)
    assert want[3] == 50  # -0 (first) and +0 compare equal: the first zero wins
    assert np.array_equal(idx, want), (idx, want)
    for i in range(y.shape[0]):
        a, b = val[i], y[i, idx[i]]
        assert (np.isnan(a) and np.isnan(b)) or a == b
    # sizes around the part boundaries (1024 per part, up to 256 parts)
    for n2 in (1, 1023, 1025, 262144, 262145, 300000):
        v = g.standard_normal((2, n2)).astype(np.float32)
        i2, _ = lowbit.lowbit_argmax(torch.from_numpy(v).cuda())
        assert np.array_equal(i2.cpu().numpy(), np.argmax(v, axis=1)), n2


@pytest.mark.parametrize("fmt,n,k,b", [("t2", 151936, 5120, 1), ("t2", 151936, 5120, 2),
                                       ("q1", 4096, 1024, 5)])
def test_lm_head_top1(fmt, n, k, b):
    import torch

    say(f"lm head {fmt} n={n} k={k} b={b}")
    codes, scales, hc, hs = full_weights(fmt, n, k, 1800 + b)
    x = synth.dev_fp16_normal((b, k), 1.0, 1810 + b)
    y, idx, val = lowbit.lowbit_lm_head(fmt, codes, scales, n, k, x)
    torch.cuda.synchronize()
    y, idx, val = y.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
    of = oracle.Q1 if fmt == "q1" else oracle.T2
    ref = oracle.gemv(of, hc, hs, n, k, host_u16(x))
    assert_close(y, ref, f"lm head logits {fmt}")
    for i in range(b):
        assert idx[i] == np.argmax(y[i]) and val[i] == y[i, idx[i]]
        rms = np.sqrt(np.mean(ref[i] ** 2))
        err = 2 * TOL * max(abs(ref[i]).max(), 0.01 * rms)  # both sides' error, generously
        top = np.sort(ref[i])[-2:]
        assert ref[i, idx[i]] >= top[1] - err
        if top[1] - top[0] > err:
            assert idx[i] == np.argmax(ref[i])


@pytest.mark.parametrize("fmt,n,k,b", [("t2", 37, 256, 1), ("q1", 5000, 384, 2), ("q1", 1500, 128, 3),
                                       ("t2", 5000, 256, 8), ("q1", 262160, 128, 1)])
def test_lm_head_reused_workspace(fmt, n, k, b):
    """The workspace's contents are ignored on entry: with a workspace full
    of 0xFF, and again on a second call that finds the first call's
    leftovers, the logits follow the GEMV bound and the index is the argmax
    of the logits the call returned.  Shapes cover one argmax part, several,
    the 256-part cap, and both GEMV kernels (b <= 2 and b >= 3)."""
    import torch

    say(f"lm head reused workspace {fmt} n={n} k={k} b={b}")
    codes, scales, hc, hs = full_weights(fmt, n, k, 1900 + b)
    ws = torch.full((lowbit.lowbit_lm_head_workspace_bytes(fmt, n, k, b),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    of = oracle.Q1 if fmt == "q1" else oracle.T2
    for call in range(2):
        x = synth.dev_fp16_normal((b, k), 1.0, 1910 + 10 * b + call)
        y, idx, val = lowbit.lowbit_lm_head(fmt, codes, scales, n, k, x, workspace=ws)
        torch.cuda.synchronize()
        y, idx, val = y.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
        assert_close(y, oracle.gemv(of, hc, hs, n, k, host_u16(x)), f"lm head logits call {call}")
        assert np.array_equal(idx, np.argmax(y, axis=1)), (call, idx)
        assert np.array_equal(val, y[np.arange(b), idx]), call
