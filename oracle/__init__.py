"""CPU oracle for the FP8 quantized linear layer (dense block-scaled and 2:4 sparse).

TEST INFRASTRUCTURE ONLY.  Tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the library and its
Python binding never do.  It shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, compiled with gcc into
``liboracle.so``); this module only marshals numpy arrays.  The definitions it
follows are cited in ``oracle.c``:

* "FP8 a granularite fine" (transformers docs), intro bullets and section
  "Chemin rapide de DeepGEMM": 128x128 weight blocks, dynamic per-token
  1x128 activation groups;
* "Deployer la parcimonie 2:4 avec FP8 sur Hopper", pipeline steps 2, 4, 6, 7
  and practical example 1: groups of 4 along K, keep the top two scores,
  recalibrate scales after pruning, export values + masks;
* "Combiner elagage et quantification", section "La cle": keep the two
  largest of every four;
* "FP8 Quantization" (TensorRT-LLM docs), section "GEMM + SwiGLU Fusion in
  Gated-MLP": the gate and up GEMMs of a gated MLP combined by SwiGLU
  (``swiglu`` / ``gemm_swiglu`` below, in numpy fp64).

Every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, brute force and exact rational arithmetic; none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GROUP = 128


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (no fast-math, no FTZ)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int64
            lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
            lib.oracle_e4m3_decode.restype = ctypes.c_double
            lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
            lib.oracle_e4m3_encode.restype = ctypes.c_uint8
            lib.oracle_quant_act.argtypes = [P, I, I, P, P]
            lib.oracle_quant_wblock.argtypes = [P, I, I, P, P]
            lib.oracle_quant_act_ue8m0.argtypes = [P, I, I, P, P]
            lib.oracle_quant_act_static.argtypes = [P, I, I, ctypes.c_float, P, P]
            lib.oracle_quant_act_tensor.argtypes = [P, I, I, P, P]
            lib.oracle_quant_wblock_ue8m0.argtypes = [P, I, I, P, P]
            lib.oracle_prune24_mask.argtypes = [P, P, I, I, P]
            lib.oracle_prune24_compress.argtypes = [P, P, I, I, P, P, P]
            lib.oracle_prune24_compress_tensor.argtypes = [P, P, I, I, P, P, P]
            lib.oracle_decompress24.argtypes = [P, P, I, I, P]
            lib.oracle_gemm.argtypes = [P, P, P, P, I, I, I, P]
            lib.oracle_gemm_rows.argtypes = [P, P, P, P, I, I, I, P, I, P]
            lib.oracle_num_threads.restype = ctypes.c_int
            for f in ("oracle_quant_act", "oracle_quant_wblock", "oracle_quant_act_ue8m0",
                      "oracle_quant_act_static", "oracle_quant_act_tensor",
                      "oracle_quant_wblock_ue8m0", "oracle_prune24_mask",
                      "oracle_prune24_compress", "oracle_prune24_compress_tensor", "oracle_decompress24",
                      "oracle_gemm",
                      "oracle_gemm_rows"):
                getattr(lib, f).restype = None
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_bf16(x: np.ndarray, name: str):
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError(f"{name}: expected a 2-D uint16 array of bf16 bits")


# ----------------------------------------------------------------- codec ----

def e4m3_decode(code: int) -> float:
    """Value of one E4M3FN code (NaN for 0x7F / 0xFF)."""
    return _load().oracle_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    """Round a real value to the nearest E4M3FN code, ties to even, saturating at +-448."""
    return int(_load().oracle_e4m3_encode(float(v)))


def e4m3_decode_table() -> np.ndarray:
    """fp64 value of each of the 256 codes."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    """Element-wise encode of a float array (slow: one C call per element)."""
    lib = _load()
    flat = np.asarray(v, dtype=np.float64).ravel()
    out = np.fromiter((lib.oracle_e4m3_encode(float(t)) for t in flat), dtype=np.uint8, count=flat.size)
    return out.reshape(np.shape(v))


# ------------------------------------------------------------ quantizers ----

def quant_act(x_bf16: np.ndarray):
    """Per-token 1x128 quantization: returns (codes [M,K] u8, scales [M,K/128] f32)."""
    _check_bf16(x_bf16, "x")
    x = np.ascontiguousarray(x_bf16)
    M, K = x.shape
    assert K % GROUP == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // GROUP), np.float32)
    if M:
        _load().oracle_quant_act(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def quant_wblock(w_bf16: np.ndarray):
    """128x128 block quantization: returns (codes [N,K] u8, scales [N/128,K/128] f32)."""
    _check_bf16(w_bf16, "w")
    w = np.ascontiguousarray(w_bf16)
    N, K = w.shape
    assert N % GROUP == 0 and K % GROUP == 0
    q = np.empty((N, K), np.uint8)
    s = np.empty((N // GROUP, K // GROUP), np.float32)
    _load().oracle_quant_wblock(_ptr(w), N, K, _ptr(q), _ptr(s))
    return q, s


# ------------------------------------------------------------------ 2:4 -----

def prune24_mask(w_bf16: np.ndarray, col_norm: np.ndarray | None = None) -> np.ndarray:
    """Boolean keep-mask [N,K]: exactly two per group of 4 along K."""
    _check_bf16(w_bf16, "w")
    w = np.ascontiguousarray(w_bf16)
    N, K = w.shape
    assert K % 4 == 0
    keep = np.empty((N, K), np.uint8)
    c = None if col_norm is None else np.ascontiguousarray(col_norm, dtype=np.float32)
    if c is not None:
        assert c.shape == (K,)
    _load().oracle_prune24_mask(_ptr(w), None if c is None else _ptr(c), N, K, _ptr(keep))
    return keep.astype(bool)


def prune24_compress(w_bf16: np.ndarray, col_norm: np.ndarray | None = None):
    """Prune 2:4, block scales over kept values, quantize, pack.

    Returns (vals [N,K/2] u8, meta [N,K/8] u8, scales [N/128,K/128] f32).
    """
    _check_bf16(w_bf16, "w")
    w = np.ascontiguousarray(w_bf16)
    N, K = w.shape
    assert N % GROUP == 0 and K % GROUP == 0
    c = None if col_norm is None else np.ascontiguousarray(col_norm, dtype=np.float32)
    vals = np.empty((N, K // 2), np.uint8)
    meta = np.empty((N, K // 8), np.uint8)
    s = np.empty((N // GROUP, K // GROUP), np.float32)
    _load().oracle_prune24_compress(_ptr(w), None if c is None else _ptr(c), N, K,
                                    _ptr(vals), _ptr(meta), _ptr(s))
    return vals, meta, s


def prune24_compress_tensor(w_bf16: np.ndarray, col_norm: np.ndarray | None = None):
    """Prune 2:4 and compress as ``prune24_compress``, with one scale for the whole tensor:
    amax over all kept values / 448, written to every entry of the [N/128,K/128] scale array.

    Returns (vals [N,K/2] u8, meta [N,K/8] u8, scales [N/128,K/128] f32, all equal).
    """
    _check_bf16(w_bf16, "w")
    w = np.ascontiguousarray(w_bf16)
    N, K = w.shape
    assert N % GROUP == 0 and K % GROUP == 0
    c = None if col_norm is None else np.ascontiguousarray(col_norm, dtype=np.float32)
    vals = np.empty((N, K // 2), np.uint8)
    meta = np.empty((N, K // 8), np.uint8)
    s = np.empty((N // GROUP, K // GROUP), np.float32)
    _load().oracle_prune24_compress_tensor(_ptr(w), None if c is None else _ptr(c), N, K,
                                           _ptr(vals), _ptr(meta), _ptr(s))
    return vals, meta, s


def decompress24(vals: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """Dense codes [N,K] from the packed 2:4 form (0x00 at pruned places)."""
    vals = np.ascontiguousarray(vals, dtype=np.uint8)
    meta = np.ascontiguousarray(meta, dtype=np.uint8)
    N, K2 = vals.shape
    K = 2 * K2
    assert meta.shape == (N, K // 8)
    q = np.empty((N, K), np.uint8)
    _load().oracle_decompress24(_ptr(vals), _ptr(meta), N, K, _ptr(q))
    return q


# ------------------------------------------------------------------ GEMM ----

def gemm(xq, xs, wq, ws, rows: np.ndarray | None = None) -> np.ndarray:
    """fp64 Y = sum over K blocks of (sx * sw) * (exact fp64 block dot product).

    ``rows`` (optional int64 indices) restricts the output to those rows of Y.
    """
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    ws = np.ascontiguousarray(ws, dtype=np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape == (N, K) and xs.shape == (M, K // GROUP) and ws.shape == (N // GROUP, K // GROUP)
    lib = _load()
    if rows is None:
        y = np.empty((M, N), np.float64)
        if M:
            lib.oracle_gemm(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y))
        return y
    r = np.ascontiguousarray(rows, dtype=np.int64)
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < M))
    y = np.empty((r.size, N), np.float64)
    if r.size:
        lib.oracle_gemm_rows(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(r), r.size, _ptr(y))
    return y


def sparse24_gemm(xq, xs, vals, meta, ws, rows: np.ndarray | None = None) -> np.ndarray:
    """The GEMM on the decompressed 2:4 weight (pruned places contribute zero)."""
    return gemm(xq, xs, decompress24(vals, meta), ws, rows=rows)


def quant_act_static(x_bf16: np.ndarray, s: float):
    """x [M,K] bf16 bits with one given fp32 scale s -> (codes enc(fp32(x/s)) saturating, s broadcast
    to [M,K/128])."""
    _check_bf16(x_bf16, "x")
    M, K = x_bf16.shape
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    q = np.empty((M, K), np.uint8)
    sa = np.empty((M, K // GROUP), np.float32)
    _load().oracle_quant_act_static(_ptr(x), M, K, ctypes.c_float(float(np.float32(s))), _ptr(q), _ptr(sa))
    return q, sa


def quant_act_tensor(x_bf16: np.ndarray):
    """Per-tensor dynamic scaling: s = fp32(amax over all of x / 448); codes and s broadcast as in
    ``quant_act_static``."""
    _check_bf16(x_bf16, "x")
    M, K = x_bf16.shape
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    q = np.empty((M, K), np.uint8)
    sa = np.empty((M, K // GROUP), np.float32)
    _load().oracle_quant_act_tensor(_ptr(x), M, K, _ptr(q), _ptr(sa))
    return q, sa


def quant_weight_tensor(w_bf16: np.ndarray):
    """Per-tensor dynamic weight scaling: the amax / 448 of all of W [N,K] and the codes of every
    element with it (the element-wise formula of ``quant_act_tensor`` on the flattened tensor),
    the scale broadcast to the [N/128,K/128] block-scale layout."""
    N, K = w_bf16.shape
    if N % GROUP:
        raise ValueError("N must be a multiple of 128")
    q, s = quant_act_tensor(w_bf16)
    return q, np.full((N // GROUP, K // GROUP), s.flat[0], np.float32)


def quant_act_ue8m0(x_bf16: np.ndarray):
    """x [M,K] bf16 bits -> (codes [M,K] uint8, UE8M0 exponents [M,K/128] uint8); scale = 2^(e-127)."""
    _check_bf16(x_bf16, "x")
    M, K = x_bf16.shape
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    q = np.empty((M, K), np.uint8)
    e = np.empty((M, K // GROUP), np.uint8)
    _load().oracle_quant_act_ue8m0(_ptr(x), M, K, _ptr(q), _ptr(e))
    return q, e


def quant_wblock_ue8m0(w_bf16: np.ndarray):
    """w [N,K] bf16 bits -> (codes [N,K] uint8, UE8M0 exponents [N/128,K/128] uint8)."""
    _check_bf16(w_bf16, "w")
    N, K = w_bf16.shape
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    q = np.empty((N, K), np.uint8)
    e = np.empty((N // GROUP, K // GROUP), np.uint8)
    _load().oracle_quant_wblock_ue8m0(_ptr(w), N, K, _ptr(q), _ptr(e))
    return q, e


def ue8m0_to_f32(e: np.ndarray) -> np.ndarray:
    """UE8M0 bytes -> their values 2^(e-127) as fp32 (exact: 2^-127 is an fp32 subnormal)."""
    return np.ldexp(np.float32(1.0), np.asarray(e, dtype=np.int32) - 127).astype(np.float32)


def gemm_ue8m0(xq, xe, wq, we, rows: np.ndarray | None = None) -> np.ndarray:
    """Block-scaled GEMM with UE8M0 scales: ``gemm`` with scales 2^(e-127)."""
    return gemm(xq, ue8m0_to_f32(xe), wq, ue8m0_to_f32(we), rows=rows)


def grouped_gemm(xq, xs, wq, ws, offsets, rows: np.ndarray | None = None) -> np.ndarray:
    """Grouped GEMM: row m of the result is ``gemm`` of row m with expert g's weight
    wq[g], ws[g], where offsets[g] <= m < offsets[g+1]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    M = xq.shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, wq.shape[1]), np.float64)
    group = np.searchsorted(offsets, rows, side="right") - 1
    for g in np.unique(group):
        sel = np.nonzero(group == g)[0]
        out[sel] = gemm(xq, xs, wq[g], ws[g], rows=rows[sel])
    return out


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """SwiGLU of gate and up values in fp64: silu(g) * u with silu(g) = g / (1 + exp(-g))."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * np.asarray(u, dtype=np.float64)


def gemm_swiglu(xq, xs, wq, ws, rows: np.ndarray | None = None) -> np.ndarray:
    """Gated-MLP up projection: wq [2I,K] stacks the gate (rows 0..I-1) and up
    (rows I..2I-1) projections; returns swiglu(gate GEMM, up GEMM) [M or rows, I]
    in fp64, each GEMM as in ``gemm``."""
    I = wq.shape[0] // 2
    nb = I // GROUP
    g = gemm(xq, xs, wq[:I], ws[:nb], rows=rows)
    u = gemm(xq, xs, wq[I:], ws[nb:], rows=rows)
    return swiglu(g, u)


def num_threads() -> int:
    """OpenMP threads the oracle GEMM runs on."""
    return int(_load().oracle_num_threads())
