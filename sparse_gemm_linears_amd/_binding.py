"""ctypes binding of ``libfp8lin.so`` (argument marshalling only).

The functions carry the C names.  Each takes torch device tensors, checks
dtype / device / contiguity, allocates outputs unless ``out=`` tensors are
given, and calls the C entry point on torch's current HIP stream.  Every step
of the computation runs in the library's HIP kernels; there is no other code
path, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8lin.so")
GROUP = 128

# status codes of include/fp8lin.h
FP8L_OK = 0
FP8L_ERR_NULL = 1
FP8L_ERR_SHAPE = 2
FP8L_ERR_ALIGN = 3
FP8L_ERR_ALIAS = 4
FP8L_ERR_DEVICE = 5
FP8L_ERR_LAUNCH = 6
FP8L_ERR_MEMORY = 7
FP8L_ERR_SCRATCH = 8

EXPORTS = ("fp8_quant_act", "fp8_quant_weight_block", "prune24_compress", "fp8_block_gemm",
           "fp8_sparse24_gemm", "fp8_quant_act_ue8m0", "fp8_quant_weight_block_ue8m0", "fp8_block_gemm_ue8m0",
           "fp8_grouped_gemm", "fp8_block_gemm_swiglu", "fp8_block_linear", "fp8_sparse24_linear",
           "fp8_quant_act_tensor", "fp8_quant_act_static", "fp8_quant_weight_tensor", "prune24_compress_tensor",
           "fp8_block_gemm_noalloc",
           "fp8lin_release_graph_scratch", "fp8lin_status_str")
MAX_LINEAR_M = 64  # the fused-quantization calls take decode-sized batches

_lock = threading.Lock()
_lib = None


class Fp8LinError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


def load_library():
    """Load ``libfp8lin.so``; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python sparse_gemm_linears_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int64
        sig = {
            "fp8_quant_act": [P, I, I, P, P, P],
            "fp8_quant_weight_block": [P, I, I, P, P, P],
            "fp8_quant_act_tensor": [P, I, I, P, P, P],
            "fp8_quant_act_static": [P, P, I, I, P, P, P],
            "fp8_quant_weight_tensor": [P, I, I, P, P, P],
            "prune24_compress": [P, P, I, I, P, P, P, P],
            "prune24_compress_tensor": [P, P, I, I, P, P, P, P],
            "fp8_block_gemm": [P, P, P, P, I, I, I, P, P],
            "fp8_block_gemm_noalloc": [P, P, P, P, I, I, I, P, P],
            "fp8lin_release_graph_scratch": [],
            "fp8_sparse24_gemm": [P, P, P, P, P, I, I, I, P, P],
            "fp8_quant_act_ue8m0": [P, I, I, P, P, P],
            "fp8_quant_weight_block_ue8m0": [P, I, I, P, P, P],
            "fp8_block_gemm_ue8m0": [P, P, P, P, I, I, I, P, P],
            "fp8_block_gemm_swiglu": [P, P, P, P, I, I, I, P, P, P, P],
            "fp8_grouped_gemm": [P, P, P, P, P, I, I, I, I, P, P],
            "fp8_block_linear": [P, P, P, I, I, I, P, P],
            "fp8_sparse24_linear": [P, P, P, P, I, I, I, P, P],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        lib.fp8lin_status_str.argtypes = [ctypes.c_int]
        lib.fp8lin_status_str.restype = ctypes.c_char_p
        _lib = lib
        return lib


def status_str(status: int) -> str:
    return load_library().fp8lin_status_str(int(status)).decode()


def _check(fn: str, status: int):
    if status != FP8L_OK:
        raise Fp8LinError(fn, status, status_str(status))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _want(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _codes(t: torch.Tensor) -> torch.Tensor:
    """Accept e4m3 codes as uint8 or float8_e4m3fn; returns a uint8 view."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    return t


def _out(out, name, shape, dtype, like):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _want(out, name, dtype, shape)
    return out


def fp8_quant_act(x: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None):
    """x [M,K] bf16 -> (q [M,K] uint8 e4m3 codes, s [M,K/128] fp32)."""
    _want(x, "x", torch.bfloat16)
    M, K = x.shape
    q = _out(q, "q", (M, K), torch.uint8, x)
    s = _out(s, "s", (M, K // GROUP), torch.float32, x)
    _check("fp8_quant_act", load_library().fp8_quant_act(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(x)))
    return q, s


def fp8_quant_act_tensor(x: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None):
    """x [M,K] bf16 -> (q [M,K] codes, s [M,K/128] fp32, every entry the per-tensor amax / 448)."""
    _want(x, "x", torch.bfloat16)
    M, K = x.shape
    q = _out(q, "q", (M, K), torch.uint8, x)
    s = _out(s, "s", (M, K // GROUP), torch.float32, x)
    _check("fp8_quant_act_tensor", load_library().fp8_quant_act_tensor(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(x)))
    return q, s


def fp8_quant_act_static(x: torch.Tensor, scale: torch.Tensor, q: torch.Tensor | None = None,
                         s: torch.Tensor | None = None):
    """x [M,K] bf16, scale: one fp32 on the device -> (q [M,K] codes, s [M,K/128] fp32 = scale)."""
    _want(x, "x", torch.bfloat16)
    _want(scale, "scale", torch.float32)
    if scale.numel() != 1 or scale.device != x.device:
        raise ValueError("scale must be one fp32 value on the device of x")
    M, K = x.shape
    q = _out(q, "q", (M, K), torch.uint8, x)
    s = _out(s, "s", (M, K // GROUP), torch.float32, x)
    _check("fp8_quant_act_static",
           load_library().fp8_quant_act_static(_ptr(x), _ptr(scale), M, K, _ptr(q), _ptr(s), _stream(x)))
    return q, s


def fp8_quant_weight_tensor(w: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None):
    """w [N,K] bf16 -> (q [N,K] codes, s [N/128,K/128] fp32, every entry the per-tensor amax / 448)."""
    _want(w, "w", torch.bfloat16)
    N, K = w.shape
    q = _out(q, "q", (N, K), torch.uint8, w)
    s = _out(s, "s", (N // GROUP, K // GROUP), torch.float32, w)
    _check("fp8_quant_weight_tensor",
           load_library().fp8_quant_weight_tensor(_ptr(w), N, K, _ptr(q), _ptr(s), _stream(w)))
    return q, s


def fp8_quant_weight_block(w: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None):
    """w [N,K] bf16 -> (q [N,K] uint8 codes, s [N/128,K/128] fp32)."""
    _want(w, "w", torch.bfloat16)
    N, K = w.shape
    q = _out(q, "q", (N, K), torch.uint8, w)
    s = _out(s, "s", (N // GROUP, K // GROUP), torch.float32, w)
    _check("fp8_quant_weight_block",
           load_library().fp8_quant_weight_block(_ptr(w), N, K, _ptr(q), _ptr(s), _stream(w)))
    return q, s


def prune24_compress(w: torch.Tensor, col_norm: torch.Tensor | None = None, vals=None, meta=None, s=None):
    """w [N,K] bf16 (+ col_norm [K] fp32) -> (vals [N,K/2], meta [N,K/8] uint8, s [N/128,K/128] fp32)."""
    _want(w, "w", torch.bfloat16)
    N, K = w.shape
    if col_norm is not None:
        _want(col_norm, "col_norm", torch.float32, (K,))
    vals = _out(vals, "vals", (N, K // 2), torch.uint8, w)
    meta = _out(meta, "meta", (N, K // 8), torch.uint8, w)
    s = _out(s, "s", (N // GROUP, K // GROUP), torch.float32, w)
    _check("prune24_compress", load_library().prune24_compress(
        _ptr(w), _ptr(col_norm), N, K, _ptr(vals), _ptr(meta), _ptr(s), _stream(w)))
    return vals, meta, s


def prune24_compress_tensor(w: torch.Tensor, col_norm: torch.Tensor | None = None, vals=None, meta=None, s=None):
    """prune24_compress with one per-tensor scale (broadcast into s [N/128,K/128])."""
    _want(w, "w", torch.bfloat16)
    N, K = w.shape
    if col_norm is not None:
        _want(col_norm, "col_norm", torch.float32, (K,))
    vals = _out(vals, "vals", (N, K // 2), torch.uint8, w)
    meta = _out(meta, "meta", (N, K // 8), torch.uint8, w)
    s = _out(s, "s", (N // GROUP, K // GROUP), torch.float32, w)
    _check("prune24_compress_tensor", load_library().prune24_compress_tensor(
        _ptr(w), _ptr(col_norm), N, K, _ptr(vals), _ptr(meta), _ptr(s), _stream(w)))
    return vals, meta, s


def fp8_block_gemm(xq, xs, wq, ws, y: torch.Tensor | None = None):
    """(xq [M,K], xs [M,K/128], wq [N,K], ws [N/128,K/128]) -> y [M,N] bf16."""
    xq, wq = _codes(xq), _codes(wq)
    _want(xq, "xq", torch.uint8)
    _want(wq, "wq", torch.uint8)
    M, K = xq.shape
    N = wq.shape[0]
    _want(wq, "wq", torch.uint8, (N, K))
    _want(xs, "xs", torch.float32, (M, K // GROUP))
    _want(ws, "ws", torch.float32, (N // GROUP, K // GROUP))
    y = _out(y, "y", (M, N), torch.bfloat16, xq)
    _check("fp8_block_gemm", load_library().fp8_block_gemm(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _stream(xq)))
    return y


def fp8_block_gemm_noalloc(xq, xs, wq, ws, y: torch.Tensor):
    """fp8_block_gemm with its split-K partials in the library's fixed device array
    (no allocation by the library; the caller passes the output y [M,N] bf16)."""
    xq, wq = _codes(xq), _codes(wq)
    _want(xq, "xq", torch.uint8)
    _want(wq, "wq", torch.uint8)
    M, K = xq.shape
    N = wq.shape[0]
    _want(wq, "wq", torch.uint8, (N, K))
    _want(xs, "xs", torch.float32, (M, K // GROUP))
    _want(ws, "ws", torch.float32, (N // GROUP, K // GROUP))
    _want(y, "y", torch.bfloat16, (M, N))
    _check("fp8_block_gemm_noalloc", load_library().fp8_block_gemm_noalloc(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _stream(xq)))
    return y


def fp8lin_release_graph_scratch():
    """Free the scratch memory kept for captured calls (no graph holding it may remain)."""
    _check("fp8lin_release_graph_scratch", load_library().fp8lin_release_graph_scratch())


def fp8_sparse24_gemm(xq, xs, wvals, wmeta, ws, y: torch.Tensor | None = None):
    """(xq [M,K], xs, wvals [N,K/2], wmeta [N,K/8], ws) -> y [M,N] bf16."""
    xq, wvals = _codes(xq), _codes(wvals)
    _want(xq, "xq", torch.uint8)
    M, K = xq.shape
    N = wvals.shape[0]
    _want(wvals, "wvals", torch.uint8, (N, K // 2))
    _want(wmeta, "wmeta", torch.uint8, (N, K // 8))
    _want(xs, "xs", torch.float32, (M, K // GROUP))
    _want(ws, "ws", torch.float32, (N // GROUP, K // GROUP))
    y = _out(y, "y", (M, N), torch.bfloat16, xq)
    _check("fp8_sparse24_gemm", load_library().fp8_sparse24_gemm(
        _ptr(xq), _ptr(xs), _ptr(wvals), _ptr(wmeta), _ptr(ws), M, N, K, _ptr(y), _stream(xq)))
    return y


def fp8_block_linear(x, wq, ws, y: torch.Tensor | None = None):
    """(x [M,K] bf16 with M <= 64, wq [N,K], ws [N/128,K/128]) -> y [M,N] bf16, bit-identical to fp8_quant_act
    followed by fp8_block_gemm (one or two tokens are quantized inside the GEMM kernel)."""
    wq = _codes(wq)
    _want(x, "x", torch.bfloat16)
    _want(wq, "wq", torch.uint8)
    M, K = x.shape
    N = wq.shape[0]
    _want(wq, "wq", torch.uint8, (N, K))
    _want(ws, "ws", torch.float32, (N // GROUP, K // GROUP))
    y = _out(y, "y", (M, N), torch.bfloat16, x)
    _check("fp8_block_linear", load_library().fp8_block_linear(
        _ptr(x), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _stream(x)))
    return y


def fp8_sparse24_linear(x, wvals, wmeta, ws, y: torch.Tensor | None = None):
    """(x [M,K] bf16 with M <= 64, wvals [N,K/2], wmeta [N,K/8], ws) -> y [M,N] bf16 (fused quantization)."""
    wvals = _codes(wvals)
    _want(x, "x", torch.bfloat16)
    M, K = x.shape
    N = wvals.shape[0]
    _want(wvals, "wvals", torch.uint8, (N, K // 2))
    _want(wmeta, "wmeta", torch.uint8, (N, K // 8))
    _want(ws, "ws", torch.float32, (N // GROUP, K // GROUP))
    y = _out(y, "y", (M, N), torch.bfloat16, x)
    _check("fp8_sparse24_linear", load_library().fp8_sparse24_linear(
        _ptr(x), _ptr(wvals), _ptr(wmeta), _ptr(ws), M, N, K, _ptr(y), _stream(x)))
    return y


def fp8_block_gemm_swiglu(xq, xs, wq, ws, h: torch.Tensor | None = None, quantize: bool = True,
                          hq: torch.Tensor | None = None, hs: torch.Tensor | None = None, keep_h: bool = True):
    """(xq [M,K], xs, wq [2I,K] = [gate; up], ws [2I/128,K/128]) -> h [M,I] bf16 = silu(gate) * up, and, when
    ``quantize``, (hq [M,I] e4m3 codes, hs [M,I/128]) = fp8_quant_act(h).  Returns (h, hq, hs); with
    ``keep_h=False`` (only with ``quantize``) h is not stored and None is returned in its place."""
    if not keep_h and not quantize:
        raise ValueError("fp8_block_gemm_swiglu: keep_h=False needs quantize=True")
    xq, wq = _codes(xq), _codes(wq)
    _want(xq, "xq", torch.uint8)
    _want(wq, "wq", torch.uint8)
    M, K = xq.shape
    I = wq.shape[0] // 2
    _want(wq, "wq", torch.uint8, (2 * I, K))
    _want(xs, "xs", torch.float32, (M, K // GROUP))
    _want(ws, "ws", torch.float32, (2 * I // GROUP, K // GROUP))
    h = _out(h, "h", (M, I), torch.bfloat16, xq) if keep_h else None
    if quantize:
        hq = _out(hq, "hq", (M, I), torch.uint8, xq)
        hs = _out(hs, "hs", (M, I // GROUP), torch.float32, xq)
    else:
        hq = hs = None
    _check("fp8_block_gemm_swiglu", load_library().fp8_block_gemm_swiglu(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, I, K, _ptr(h), _ptr(hq), _ptr(hs), _stream(xq)))
    return h, hq, hs


def _exps(t: torch.Tensor) -> torch.Tensor:
    """Accept UE8M0 scales as uint8 or float8_e8m0fnu; returns a uint8 view."""
    if t.dtype == getattr(torch, "float8_e8m0fnu", None):
        return t.view(torch.uint8)
    return t


def fp8_quant_act_ue8m0(x: torch.Tensor, q: torch.Tensor | None = None, e: torch.Tensor | None = None):
    """x [M,K] bf16 -> (q [M,K] e4m3 codes, e [M,K/128] UE8M0 exponent bytes; scale 2^(e-127))."""
    _want(x, "x", torch.bfloat16)
    M, K = x.shape
    q = _out(q, "q", (M, K), torch.uint8, x)
    e = _out(e, "e", (M, K // GROUP), torch.uint8, x)
    _check("fp8_quant_act_ue8m0", load_library().fp8_quant_act_ue8m0(_ptr(x), M, K, _ptr(q), _ptr(e), _stream(x)))
    return q, e


def fp8_quant_weight_block_ue8m0(w: torch.Tensor, q: torch.Tensor | None = None, e: torch.Tensor | None = None):
    """w [N,K] bf16 -> (q [N,K] e4m3 codes, e [N/128,K/128] UE8M0 exponent bytes)."""
    _want(w, "w", torch.bfloat16)
    N, K = w.shape
    q = _out(q, "q", (N, K), torch.uint8, w)
    e = _out(e, "e", (N // GROUP, K // GROUP), torch.uint8, w)
    _check("fp8_quant_weight_block_ue8m0",
           load_library().fp8_quant_weight_block_ue8m0(_ptr(w), N, K, _ptr(q), _ptr(e), _stream(w)))
    return q, e


def fp8_block_gemm_ue8m0(xq, xe, wq, we, y: torch.Tensor | None = None):
    """(xq [M,K], xe [M,K/128], wq [N,K], we [N/128,K/128], UE8M0 exponents) -> y [M,N] bf16."""
    xq, wq, xe, we = _codes(xq), _codes(wq), _exps(xe), _exps(we)
    _want(xq, "xq", torch.uint8)
    _want(wq, "wq", torch.uint8)
    M, K = xq.shape
    N = wq.shape[0]
    _want(wq, "wq", torch.uint8, (N, K))
    _want(xe, "xe", torch.uint8, (M, K // GROUP))
    _want(we, "we", torch.uint8, (N // GROUP, K // GROUP))
    y = _out(y, "y", (M, N), torch.bfloat16, xq)
    _check("fp8_block_gemm_ue8m0", load_library().fp8_block_gemm_ue8m0(
        _ptr(xq), _ptr(xe), _ptr(wq), _ptr(we), M, N, K, _ptr(y), _stream(xq)))
    return y


def fp8_grouped_gemm(xq, xs, wq, ws, offsets: torch.Tensor, y: torch.Tensor | None = None):
    """Grouped (MoE) GEMM: rows offsets[g] .. offsets[g+1]-1 of (xq [M,K], xs) times expert g of
    (wq [G,N,K], ws [G,N/128,K/128]); offsets is a device int32 tensor [G+1].  -> y [M,N] bf16."""
    xq, wq = _codes(xq), _codes(wq)
    _want(xq, "xq", torch.uint8)
    _want(wq, "wq", torch.uint8)
    M, K = xq.shape
    G, N = wq.shape[0], wq.shape[1]
    _want(wq, "wq", torch.uint8, (G, N, K))
    _want(xs, "xs", torch.float32, (M, K // GROUP))
    _want(ws, "ws", torch.float32, (G, N // GROUP, K // GROUP))
    _want(offsets, "offsets", torch.int32, (G + 1,))
    y = _out(y, "y", (M, N), torch.bfloat16, xq)
    _check("fp8_grouped_gemm", load_library().fp8_grouped_gemm(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(offsets), G, M, N, K, _ptr(y), _stream(xq)))
    return y
