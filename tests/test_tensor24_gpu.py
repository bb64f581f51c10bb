"""2:4 with one per-tensor scale, and the 2:4 GEMM on scales that are the same
in every K block.

* prune24_compress_tensor: values, index words and the (broadcast) scale are
  bit-exact against the oracle, magnitude and activation-aware, on the
  Llama-3-8B shapes and ragged ones, an all-zero weight and a reused dirty
  scale array.
* fp8_sparse24_gemm on per-tensor operands (fp8_quant_act_tensor codes and
  prune24_compress_tensor weights), on per-token activation scales that are
  constant along K, and on mixed cases (per-tensor activations with block
  weight scales and the reverse), within the GEMM tolerance of the oracle.
  Where every scale a wave uses is the same in every K block the tile kernel
  sums unscaled block products and scales once; these cases cover that form,
  its neighbours and the row-sampled full-size shapes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, bf16_dev, dev, host, sample_tile_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("aware", [False, True])
@pytest.mark.parametrize("N,K", [(128, 128), (384, 640), (4096, 4096), (4096, 14336), (28672, 4096)])
def test_prune24_tensor_bit_exact(gpu_lib, N, K, aware):
    print(f"prune24_compress_tensor N={N} K={K} aware={aware}", flush=True)
    w = si.weights(N, K)
    c = si.column_norms(si.calibration_batch(K)) if aware else None
    vals, meta, s = gpu_lib.prune24_compress_tensor(bf16_dev(w), None if c is None else dev(c))
    vr, mr, sr = oracle.prune24_compress_tensor(w, c)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(host(meta), mr)
    assert np.array_equal(host(vals), vr)


def test_prune24_tensor_zero_weight_and_dirty_scales(gpu_lib):
    w = np.zeros((256, 384), np.uint16)
    s = torch.full((2, 3), 7.0, dtype=torch.float32, device="cuda")
    vals, meta, s = gpu_lib.prune24_compress_tensor(bf16_dev(w), None, s=s)
    vr, mr, sr = oracle.prune24_compress_tensor(w)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32)) and sr.flat[0] == 0.0
    assert np.array_equal(host(meta), mr) and np.array_equal(host(vals), vr)
    w = si.weights(256, 384)                           # the same scale array again, now dirty
    vals, meta, s = gpu_lib.prune24_compress_tensor(bf16_dev(w), None, s=s)
    vr, mr, sr = oracle.prune24_compress_tensor(w)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(host(vals), vr)


def _row_constant_acts(x):
    """Per-token scales constant along K: each row quantized with its own single scale."""
    qs, ss = [], []
    for r in range(x.shape[0]):
        amax = np.abs(si.bf16_bits_to_f32(x[r])).max()
        q, s = oracle.quant_act_static(x[r:r + 1], float(np.float32(amax) / np.float32(448)))
        qs.append(q)
        ss.append(s)
    return np.concatenate(qs), np.concatenate(ss)


@pytest.mark.parametrize("M,name", [(4096, "gate_up"), (4096, "down"), (300, "qkv"), (1000, "o_proj")])
@pytest.mark.parametrize("acts,weights", [("tensor", "tensor"), ("row", "tensor"), ("tensor", "block"),
                                          ("group", "tensor")])
def test_sparse_gemm_scale_forms(gpu_lib, M, name, acts, weights):
    _, K, N = next(s for s in si.LLAMA3_8B if s[0] == name)
    print(f"fp8_sparse24_gemm M={M} {name} acts={acts} weights={weights}", flush=True)
    x = si.activations(M, K)
    if acts == "tensor":
        xq, xs = oracle.quant_act_tensor(x)
    elif acts == "row":
        xq, xs = _row_constant_acts(x)
    else:
        xq, xs = oracle.quant_act(x)
    w = si.weights(N, K)
    c = si.column_norms(si.calibration_batch(K))
    vals, meta, ws = (oracle.prune24_compress_tensor if weights == "tensor" else oracle.prune24_compress)(w, c)
    y = gpu_lib.fp8_sparse24_gemm(dev(xq), dev(xs), dev(vals), dev(meta), dev(ws))
    rows = sample_tile_rows(M, 8)
    ref = oracle.sparse24_gemm(xq, xs, vals, meta, ws, rows=rows)
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], ref, f"{name} M={M} {acts}/{weights}")


def test_sparse_gemm_constant_scales_with_zero_rows(gpu_lib):
    """Zero token rows (scale 0, zero codes) inside tiles whose other tokens keep one
    scale along K: the summed form scales them by zero."""
    M, K, N = 512, 4096, 4096
    x = si.activations(M, K).copy()
    x[::7] = 0
    xq, xs = _row_constant_acts(x)
    w = si.weights(N, K)
    vals, meta, ws = oracle.prune24_compress_tensor(w)
    y = gpu_lib.fp8_sparse24_gemm(dev(xq), dev(xs), dev(vals), dev(meta), dev(ws))
    assert_gemm_close(y, oracle.sparse24_gemm(xq, xs, vals, meta, ws), "zero rows")
    assert torch.count_nonzero(y[::7].float()) == 0


def test_gpu_tensor_path_end_to_end(gpu_lib):
    """GPU per-tensor quantizers feeding the 2:4 GEMM, against the oracle doing every step."""
    M, K, N = 4096, 4096, 6144
    x = si.activations(M, K)
    w = si.weights(N, K)
    c = si.column_norms(si.calibration_batch(K))
    xq, xs = gpu_lib.fp8_quant_act_tensor(bf16_dev(x))
    v, m, s = gpu_lib.prune24_compress_tensor(bf16_dev(w), dev(c))
    y = gpu_lib.fp8_sparse24_gemm(xq, xs, v, m, s)
    rxq, rxs = oracle.quant_act_tensor(x)
    rv, rm, rs = oracle.prune24_compress_tensor(w, c)
    rows = sample_tile_rows(M, 4)
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.sparse24_gemm(rxq, rxs, rv, rm, rs, rows=rows),
                      "per-tensor 2:4 path")
