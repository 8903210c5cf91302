"""Thin ctypes binding of liblowbit.so (include/lowbit.h), same names.

Argument marshalling only: every function checks tensor dtype / device /
contiguity, allocates outputs when none are given (torch is the allocator),
passes raw device pointers and torch's current HIP stream, and raises
``LowbitError`` on a non-zero status.  All computation happens in the HIP
kernels of the library.  If the library is missing this module raises on
first use; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblowbit.so")

LOWBIT_FMT_Q1_G128 = 1
LOWBIT_FMT_T2_G128 = 2
FORMATS = {"q1": LOWBIT_FMT_Q1_G128, "t2": LOWBIT_FMT_T2_G128}

# exported symbols, in the order include/lowbit.h declares them
SYMBOLS = [
    "lowbit_version", "lowbit_status_str", "lowbit_codes_bytes", "lowbit_scales_bytes",
    "lowbit_quantize_q1", "lowbit_pack_t2", "lowbit_pack", "lowbit_unpack",
    "lowbit_quantize_t2", "lowbit_base3_bytes", "lowbit_t2_to_base3", "lowbit_base3_to_t2",
    "lowbit_gemv_workspace_bytes", "lowbit_gemv_prepare", "lowbit_gemv_accumulate",
    "lowbit_gemv", "lowbit_gemv_noalloc", "lowbit_gemm", "lowbit_gemm_f32", "lowbit_silu_mul",
    "lowbit_ffn_workspace_bytes", "lowbit_ffn", "lowbit_embed", "lowbit_argmax_workspace_bytes",
    "lowbit_argmax", "lowbit_lm_head_workspace_bytes", "lowbit_lm_head",
]


# ceiling probes (include/lowbit_probes.h): context for the roofline only
PROBE_SYMBOLS = ["lowbit_probe_stream_read", "lowbit_probe_mfma_bf16", "lowbit_probe_lds_read",
                 "lowbit_probe_expand_mfma", "lowbit_probe_cu_count"]


class LowbitError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


_lib = None


def load() -> ctypes.CDLL:
    """Load liblowbit.so (built in-tree); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m bit_matmul_lowbit_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    # torch first: it ships its own HIP runtime under the same soname as the
    # system one the library links against, and whichever is loaded first
    # serves both.  Loaded the other way round, torch's tensors and the
    # library's launches end up in different runtimes and every launch fails.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    p, i64, sz, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "lowbit_version": ([], i),
        "lowbit_status_str": ([i], ctypes.c_char_p),
        "lowbit_codes_bytes": ([i, i64, i64], sz),
        "lowbit_scales_bytes": ([i, i64, i64], sz),
        "lowbit_quantize_q1": ([p, i64, i64, p, p, p], i),
        "lowbit_pack_t2": ([p, p, i64, i64, p, p, p], i),
        "lowbit_pack": ([i, p, p, i64, i64, p, p, p], i),
        "lowbit_unpack": ([i, p, p, i64, i64, p, p], i),
        "lowbit_gemv_workspace_bytes": ([i, i64, i64, i64], sz),
        "lowbit_gemv_prepare": ([i64, i64, p, i64, p, p, sz, p], i),
        "lowbit_gemv_accumulate": ([i, p, p, i64, i64, i64, p, p, sz, p], i),
        "lowbit_gemv": ([i, p, p, i64, i64, p, i64, p, p, sz, p], i),
        "lowbit_gemv_noalloc": ([i, p, p, i64, i64, p, i64, p, p], i),
        "lowbit_gemm": ([i, p, p, i64, i64, p, i64, p, p], i),
        "lowbit_gemm_f32": ([i, p, p, i64, i64, p, i64, p, p], i),
        "lowbit_silu_mul": ([p, i64, i64, p, p], i),
        "lowbit_ffn_workspace_bytes": ([i, i64, i64, i64], sz),
        "lowbit_ffn": ([i, p, p, p, p, i64, i64, p, i64, p, p, sz, p], i),
        "lowbit_embed": ([i, p, p, i64, i64, p, i64, p, p], i),
        "lowbit_argmax_workspace_bytes": ([i64, i64], sz),
        "lowbit_argmax": ([p, i64, i64, p, p, p, sz, p], i),
        "lowbit_lm_head_workspace_bytes": ([i, i64, i64, i64], sz),
        "lowbit_lm_head": ([i, p, p, i64, i64, p, i64, p, p, p, p, sz, p], i),
        "lowbit_quantize_t2": ([p, i64, i64, p, p, p], i),
        "lowbit_base3_bytes": ([i64, i64], sz),
        "lowbit_t2_to_base3": ([p, p, i64, i64, p, p, p], i),
        "lowbit_base3_to_t2": ([p, p, i64, i64, p, p, p], i),
        "lowbit_probe_stream_read": ([p, sz, i, i, p, p], i),
        "lowbit_probe_mfma_bf16": ([i, i, p, p], i),
        "lowbit_probe_lds_read": ([i, i, p, p], i),
        "lowbit_probe_expand_mfma": ([i, i, i, p, p], i),
        "lowbit_probe_cu_count": ([], i),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().lowbit_status_str(int(status)).decode()


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LowbitError(status, where)


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtypes, name):
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need_numel(t, count, name):
    """t must hold at least `count` elements (the C interface takes no buffer
    lengths, so a short buffer would be read or written past its end)."""
    if t.numel() < count:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {count}")


def _need_shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _need_planes(fmt, n, k, codes, scales, what=""):
    """codes / scales large enough for an n x k matrix in `fmt` (layout v1).
    An invalid shape is left to the library, which rejects it."""
    cb = lowbit_codes_bytes(fmt, n, k)
    sb = lowbit_scales_bytes(fmt, n, k)
    if cb:
        _need_numel(codes, cb, what + "codes")
    if sb:
        _need_numel(scales, sb // 2, what + "scales")


# ---------------------------------------------------------------------------
# host-only queries

def lowbit_version() -> int:
    return load().lowbit_version()


def lowbit_codes_bytes(fmt, n: int, k: int) -> int:
    return load().lowbit_codes_bytes(_fmt(fmt), n, k)


def lowbit_scales_bytes(fmt, n: int, k: int) -> int:
    return load().lowbit_scales_bytes(_fmt(fmt), n, k)


def lowbit_gemv_workspace_bytes(fmt, n: int, k: int, b: int) -> int:
    return load().lowbit_gemv_workspace_bytes(_fmt(fmt), n, k, b)


# ---------------------------------------------------------------------------
# device entry points

def _planes(fmt, n, k, device, codes, scales):
    import torch

    if codes is None:
        codes = torch.empty(lowbit_codes_bytes(fmt, n, k), dtype=torch.uint8, device=device)
    if scales is None:
        scales = torch.empty(lowbit_scales_bytes(fmt, n, k) // 2, dtype=torch.float16, device=device)
    return codes, scales


def lowbit_quantize_q1(w, codes=None, scales=None, stream=None):
    """FP16 [n][k] -> (codes uint8, scales fp16) in the Q1 layout."""
    import torch

    n, k = w.shape
    wp = _dev(w, (torch.float16,), "w")
    codes, scales = _planes(LOWBIT_FMT_Q1_G128, n, k, w.device, codes, scales)
    _need_planes(LOWBIT_FMT_Q1_G128, n, k, codes, scales)
    _check(load().lowbit_quantize_q1(wp, n, k, _dev(codes, (torch.uint8,), "codes"),
                                     _dev(scales, (torch.float16, torch.int16), "scales"),
                                     _stream(stream)), "lowbit_quantize_q1")
    return codes, scales


def lowbit_pack_t2(t, s, codes=None, scales=None, stream=None):
    """int8 t [n][k] + FP16 group scales [n][k/128] -> (codes, scales)."""
    import torch

    n, k = t.shape
    tp = _dev(t, (torch.int8,), "t")
    sp = _dev(s, (torch.float16, torch.int16), "s")
    if tuple(s.shape) != (n, k // 128):
        raise ValueError("s must be [n][k/128]")
    codes, scales = _planes(LOWBIT_FMT_T2_G128, n, k, t.device, codes, scales)
    _need_planes(LOWBIT_FMT_T2_G128, n, k, codes, scales)
    _check(load().lowbit_pack_t2(tp, sp, n, k, _dev(codes, (torch.uint8,), "codes"),
                                 _dev(scales, (torch.float16, torch.int16), "scales"),
                                 _stream(stream)), "lowbit_pack_t2")
    return codes, scales


def lowbit_pack(fmt, src, src_scales=None, codes=None, scales=None, stream=None):
    if _fmt(fmt) == LOWBIT_FMT_Q1_G128:
        if src_scales is not None:
            raise ValueError("Q1 packing computes its scales; src_scales must be None")
        return lowbit_quantize_q1(src, codes, scales, stream)
    return lowbit_pack_t2(src, src_scales, codes, scales, stream)


def lowbit_unpack(fmt, codes, scales, n: int, k: int, out=None, stream=None):
    """codes + scales -> dense FP16 [n][k]."""
    import torch

    _need_planes(fmt, n, k, codes, scales)
    if out is None:
        out = torch.empty((n, k), dtype=torch.float16, device=codes.device)
    _need_shape(out, (n, k), "out")
    _check(load().lowbit_unpack(_fmt(fmt), _dev(codes, (torch.uint8,), "codes"),
                                _dev(scales, (torch.float16, torch.int16), "scales"), n, k,
                                _dev(out, (torch.float16, torch.int16), "out"), _stream(stream)),
           "lowbit_unpack")
    return out


def lowbit_gemv(fmt, codes, scales, n: int, k: int, x, out=None, workspace=None, stream=None):
    """x FP16 [b][k] (or [k]) -> y FP32 [b][n]."""
    import torch

    x2 = x if x.dim() == 2 else x.view(1, -1)
    b = x2.shape[0]
    if x2.shape[1] != k:
        raise ValueError("x must have k columns")
    _need_planes(fmt, n, k, codes, scales)
    if out is None:
        out = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _need_numel(out, b * n, "out")
    need = lowbit_gemv_workspace_bytes(fmt, n, k, b)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(load().lowbit_gemv(_fmt(fmt), _dev(codes, (torch.uint8,), "codes"),
                              _dev(scales, (torch.float16, torch.int16), "scales"), n, k,
                              _dev(x2, (torch.float16,), "x"), b,
                              _dev(out, (torch.float32,), "out"),
                              _dev(workspace, (torch.uint8,), "workspace"),
                              workspace.numel(), _stream(stream)), "lowbit_gemv")
    return out


def lowbit_gemv_noalloc(fmt, codes, scales, n: int, k: int, x, out=None, stream=None):
    """x FP16 [b][k] (or [k]) -> y FP32 [b][n], with the library's static
    scratch instead of a workspace (the library allocates nothing; pass
    `out` to allocate nothing here either)."""
    import torch

    x2 = x if x.dim() == 2 else x.view(1, -1)
    b = x2.shape[0]
    if x2.shape[1] != k:
        raise ValueError("x must have k columns")
    _need_planes(fmt, n, k, codes, scales)
    if out is None:
        out = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _need_numel(out, b * n, "out")
    _check(load().lowbit_gemv_noalloc(_fmt(fmt), _dev(codes, (torch.uint8,), "codes"),
                                      _dev(scales, (torch.float16, torch.int16), "scales"), n, k,
                                      _dev(x2, (torch.float16,), "x"), b,
                                      _dev(out, (torch.float32,), "out"), _stream(stream)),
           "lowbit_gemv_noalloc")
    return out


def lowbit_gemv_prepare(n: int, k: int, x, out, workspace, stream=None):
    """x FP16 [b][k] prepared into `workspace`; out FP32 [b][n] := 0."""
    import torch

    x2 = x if x.dim() == 2 else x.view(1, -1)
    b = x2.shape[0]
    if x2.shape[1] != k:
        raise ValueError("x must have k columns")
    _need_numel(out, b * n, "out")
    _check(load().lowbit_gemv_prepare(n, k, _dev(x2, (torch.float16,), "x"), b,
                                      _dev(out, (torch.float32,), "out"),
                                      _dev(workspace, (torch.uint8,), "workspace"),
                                      workspace.numel(), _stream(stream)), "lowbit_gemv_prepare")
    return out


def lowbit_gemv_accumulate(fmt, codes, scales, n: int, k: int, b: int, out, workspace,
                           stream=None):
    """out FP32 [b][n] += W.x with the tables left by lowbit_gemv_prepare."""
    import torch

    _need_planes(fmt, n, k, codes, scales)
    _need_numel(out, b * n, "out")
    _check(load().lowbit_gemv_accumulate(_fmt(fmt), _dev(codes, (torch.uint8,), "codes"),
                                         _dev(scales, (torch.float16, torch.int16), "scales"),
                                         n, k, b, _dev(out, (torch.float32,), "out"),
                                         _dev(workspace, (torch.uint8,), "workspace"),
                                         workspace.numel(), _stream(stream)),
           "lowbit_gemv_accumulate")
    return out


def lowbit_gemm(fmt, codes, scales, n: int, k: int, x, out=None, stream=None):
    """X BF16 [m][k] -> Y BF16 [m][n]."""
    import torch

    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [m][k]")
    m = x.shape[0]
    _need_planes(fmt, n, k, codes, scales)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _need_numel(out, m * n, "out")
    _check(load().lowbit_gemm(_fmt(fmt), _dev(codes, (torch.uint8,), "codes"),
                              _dev(scales, (torch.float16, torch.int16), "scales"), n, k,
                              _dev(x, (torch.bfloat16,), "x"), m,
                              _dev(out, (torch.bfloat16,), "out"), _stream(stream)), "lowbit_gemm")
    return out


def lowbit_gemm_f32(fmt, codes, scales, n: int, k: int, x, out=None, stream=None):
    """X BF16 [m][k] -> Y FP32 [m][n] (same contraction, unrounded store)."""
    import torch

    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [m][k]")
    m = x.shape[0]
    _need_planes(fmt, n, k, codes, scales)
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _need_numel(out, m * n, "out")
    _check(load().lowbit_gemm_f32(_fmt(fmt), _dev(codes, (torch.uint8,), "codes"),
                                  _dev(scales, (torch.float16, torch.int16), "scales"), n, k,
                                  _dev(x, (torch.bfloat16,), "x"), m,
                                  _dev(out, (torch.float32,), "out"), _stream(stream)),
           "lowbit_gemm_f32")
    return out


def lowbit_silu_mul(h, out=None, stream=None):
    """h FP32 [b][2f] (gate | up) -> z FP16 [b][f] = SiLU(gate) * up."""
    import torch

    h2 = h if h.dim() == 2 else h.view(1, -1)
    b, f2 = h2.shape
    if f2 % 2:
        raise ValueError("h must have 2f columns")
    f = f2 // 2
    if out is None:
        out = torch.empty((b, f), dtype=torch.float16, device=h.device)
    _need_numel(out, b * f, "out")
    _check(load().lowbit_silu_mul(_dev(h2, (torch.float32,), "h"), f, b,
                                  _dev(out, (torch.float16,), "out"), _stream(stream)),
           "lowbit_silu_mul")
    return out


def lowbit_ffn_workspace_bytes(fmt, k: int, f: int, b: int) -> int:
    return int(load().lowbit_ffn_workspace_bytes(_fmt(fmt), k, f, b))


def lowbit_ffn(fmt, gu_codes, gu_scales, dn_codes, dn_scales, k: int, f: int, x, out=None,
               workspace=None, stream=None):
    """Decode FFN: x FP16 [b][k] -> y FP32 [b][k] = W_dn (SiLU(W_gate x) * (W_up x)),
    W_gu = [gate; up] stacked as [2f][k], W_dn [k][f]."""
    import torch

    x2 = x if x.dim() == 2 else x.view(1, -1)
    b = x2.shape[0]
    if x2.shape[1] != k:
        raise ValueError("x must have k columns")
    _need_planes(fmt, 2 * f, k, gu_codes, gu_scales, "gu_")
    _need_planes(fmt, k, f, dn_codes, dn_scales, "dn_")
    if out is None:
        out = torch.empty((b, k), dtype=torch.float32, device=x.device)
    _need_numel(out, b * k, "out")
    need = lowbit_ffn_workspace_bytes(fmt, k, f, b)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(load().lowbit_ffn(_fmt(fmt), _dev(gu_codes, (torch.uint8,), "gu_codes"),
                             _dev(gu_scales, (torch.float16, torch.int16), "gu_scales"),
                             _dev(dn_codes, (torch.uint8,), "dn_codes"),
                             _dev(dn_scales, (torch.float16, torch.int16), "dn_scales"),
                             k, f, _dev(x2, (torch.float16,), "x"), b,
                             _dev(out, (torch.float32,), "out"),
                             _dev(workspace, (torch.uint8,), "workspace"),
                             workspace.numel(), _stream(stream)), "lowbit_ffn")
    return out


def lowbit_embed(fmt, codes, scales, n: int, k: int, ids, out=None, stream=None):
    """Rows ids (int32 [count]) of W [n][k], dequantised to FP16 [count][k]."""
    import torch

    count = ids.numel()
    _need_planes(fmt, n, k, codes, scales)
    if out is None:
        out = torch.empty((count, k), dtype=torch.float16, device=ids.device)
    _need_numel(out, count * k, "out")
    _check(load().lowbit_embed(_fmt(fmt), _dev(codes, (torch.uint8,), "codes"),
                               _dev(scales, (torch.float16, torch.int16), "scales"), n, k,
                               _dev(ids, (torch.int32,), "ids"), count,
                               _dev(out, (torch.float16,), "out"), _stream(stream)),
           "lowbit_embed")
    return out


def lowbit_argmax(y, idx=None, val=None, workspace=None, stream=None):
    """Top-1 of each row of y FP32 [b][n] -> (idx int32 [b], val FP32 [b])."""
    import torch

    y2 = y if y.dim() == 2 else y.view(1, -1)
    b, n = y2.shape
    if idx is None:
        idx = torch.empty(b, dtype=torch.int32, device=y.device)
    if val is None:
        val = torch.empty(b, dtype=torch.float32, device=y.device)
    _need_numel(idx, b, "idx")
    _need_numel(val, b, "val")
    need = int(load().lowbit_argmax_workspace_bytes(n, b))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=y.device)
    _check(load().lowbit_argmax(_dev(y2, (torch.float32,), "y"), n, b,
                                _dev(idx, (torch.int32,), "idx"), _dev(val, (torch.float32,), "val"),
                                _dev(workspace, (torch.uint8,), "workspace"), workspace.numel(),
                                _stream(stream)), "lowbit_argmax")
    return idx, val


def lowbit_lm_head_workspace_bytes(fmt, n: int, k: int, b: int) -> int:
    return int(load().lowbit_lm_head_workspace_bytes(_fmt(fmt), n, k, b))


def lowbit_lm_head(fmt, codes, scales, n: int, k: int, x, out=None, idx=None, val=None,
                   workspace=None, stream=None):
    """Logits y FP32 [b][n] = W.x and their top-1 (idx int32 [b], val FP32 [b])."""
    import torch

    x2 = x if x.dim() == 2 else x.view(1, -1)
    b = x2.shape[0]
    if x2.shape[1] != k:
        raise ValueError("x must have k columns")
    _need_planes(fmt, n, k, codes, scales)
    if out is None:
        out = torch.empty((b, n), dtype=torch.float32, device=x.device)
    if idx is None:
        idx = torch.empty(b, dtype=torch.int32, device=x.device)
    if val is None:
        val = torch.empty(b, dtype=torch.float32, device=x.device)
    _need_numel(out, b * n, "out")
    _need_numel(idx, b, "idx")
    _need_numel(val, b, "val")
    need = lowbit_lm_head_workspace_bytes(fmt, n, k, b)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(load().lowbit_lm_head(_fmt(fmt), _dev(codes, (torch.uint8,), "codes"),
                                 _dev(scales, (torch.float16, torch.int16), "scales"), n, k,
                                 _dev(x2, (torch.float16,), "x"), b,
                                 _dev(out, (torch.float32,), "out"),
                                 _dev(idx, (torch.int32,), "idx"), _dev(val, (torch.float32,), "val"),
                                 _dev(workspace, (torch.uint8,), "workspace"), workspace.numel(),
                                 _stream(stream)), "lowbit_lm_head")
    return out, idx, val


def lowbit_quantize_t2(w, codes=None, scales=None, stream=None):
    """FP16 [n][k] -> ternary g128 codes and scales (layout v1)."""
    import torch

    n, k = w.shape
    codes, scales = _planes("t2", n, k, w.device, codes, scales)
    _need_planes("t2", n, k, codes, scales)
    _check(load().lowbit_quantize_t2(_dev(w, (torch.float16,), "w"), n, k,
                                     _dev(codes, (torch.uint8,), "codes"),
                                     _dev(scales, (torch.float16, torch.int16), "scales"),
                                     _stream(stream)), "lowbit_quantize_t2")
    return codes, scales


def lowbit_t2_to_base3(codes, scales, n: int, k: int, out=None, out_scales=None, stream=None):
    """Ternary codes -> (base-3 bytes [n][ceil(k/5)], scales FP16 [n][k/128])."""
    import torch

    if out is None:
        out = torch.empty((n, (k + 4) // 5), dtype=torch.uint8, device=codes.device)
    if out_scales is None:
        out_scales = torch.empty((n, k // 128), dtype=torch.float16, device=codes.device)
    _need_planes("t2", n, k, codes, scales)
    _need_numel(out, n * ((k + 4) // 5), "out")
    _need_numel(out_scales, n * (k // 128), "out_scales")
    _check(load().lowbit_t2_to_base3(_dev(codes, (torch.uint8,), "codes"),
                                     _dev(scales, (torch.float16, torch.int16), "scales"), n, k,
                                     _dev(out, (torch.uint8,), "out"),
                                     _dev(out_scales, (torch.float16, torch.int16), "out_scales"),
                                     _stream(stream)), "lowbit_t2_to_base3")
    return out, out_scales


def lowbit_base3_to_t2(b3, scales_rm, n: int, k: int, codes=None, scales=None, stream=None):
    """Base-3 bytes + row-major scales -> ternary codes and scales (layout v1)."""
    import torch

    codes, scales = _planes("t2", n, k, b3.device, codes, scales)
    _need_planes("t2", n, k, codes, scales)
    _need_numel(b3, n * ((k + 4) // 5), "b3")
    _need_numel(scales_rm, n * (k // 128), "scales_rm")
    _check(load().lowbit_base3_to_t2(_dev(b3, (torch.uint8,), "b3"),
                                     _dev(scales_rm, (torch.float16, torch.int16), "scales_rm"),
                                     n, k, _dev(codes, (torch.uint8,), "codes"),
                                     _dev(scales, (torch.float16, torch.int16), "scales"),
                                     _stream(stream)), "lowbit_base3_to_t2")
    return codes, scales


# ---------------------------------------------------------------------------
# ceiling probes (context for the roofline, not part of the path)

def lowbit_probe_cu_count() -> int:
    return int(load().lowbit_probe_cu_count())


def lowbit_probe_stream_read(buf, blocks_per_cu: int, sink, order: int = 0, stream=None):
    """Read every byte of the device tensor `buf` once (streaming-read probe;
    order 0 grid-stride, 1 one contiguous share per work-group)."""
    import torch

    nbytes = buf.numel() * buf.element_size()
    _need_numel(sink, blocks_per_cu * lowbit_probe_cu_count(), "sink")
    _check(load().lowbit_probe_stream_read(_dev(buf, (buf.dtype,), "buf"), nbytes, blocks_per_cu,
                                           order, _dev(sink, (torch.int32, torch.uint32), "sink"),
                                           _stream(stream)), "lowbit_probe_stream_read")


def lowbit_probe_mfma_bf16(iters: int, blocks_per_cu: int, sink, stream=None):
    """Matrix-core loop probe; returns the flops it executes."""
    import torch

    blocks = blocks_per_cu * lowbit_probe_cu_count()
    _need_numel(sink, blocks * 256, "sink")
    _check(load().lowbit_probe_mfma_bf16(iters, blocks_per_cu, _dev(sink, (torch.float32,), "sink"),
                                         _stream(stream)), "lowbit_probe_mfma_bf16")
    return blocks * 4 * iters * 4 * 2 * 32 * 32 * 16


def lowbit_probe_lds_read(iters: int, blocks_per_cu: int, sink, stream=None):
    """LDS read-bandwidth probe; returns the bytes it reads from LDS."""
    import torch

    blocks = blocks_per_cu * lowbit_probe_cu_count()
    _need_numel(sink, blocks * 256, "sink")
    _check(load().lowbit_probe_lds_read(iters, blocks_per_cu,
                                        _dev(sink, (torch.int32, torch.uint32), "sink"),
                                        _stream(stream)), "lowbit_probe_lds_read")
    return blocks * 256 * iters * 8 * 16


def lowbit_probe_expand_mfma(mode: int, iters: int, blocks_per_cu: int, sink, stream=None):
    """Probe of the matrix-core GEMV's per-row work (mode 0: expansion +
    MFMA, 1: the MFMA alone, 2: LDS-lookup expansion + MFMA + per-group
    scale, iters a multiple of 4); returns the row steps each SIMD runs."""
    import torch

    blocks = blocks_per_cu * lowbit_probe_cu_count()
    _need_numel(sink, blocks * 256, "sink")
    _check(load().lowbit_probe_expand_mfma(mode, iters, blocks_per_cu,
                                           _dev(sink, (torch.float32,), "sink"), _stream(stream)),
           "lowbit_probe_expand_mfma")
    return blocks_per_cu * iters * 16
