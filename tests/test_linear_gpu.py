"""Parity of the fused decode-sized linear calls (bf16 activations quantized
inside the GEMM kernel) through the C ABI.

Each call must give bit-identical outputs to the two-call path it fuses
(fp8_quant_act, then fp8_block_gemm / fp8_sparse24_gemm), and, like the GEMMs,
stay within the stated tolerance of the CPU oracle run on the oracle's own
activation codes:  ||Y - Y_ref||_F / ||Y_ref||_F <= 5e-3  and
|Y - Y_ref| <= 2^-7 |Y_ref| + 1e-3 max|Y_ref| element-wise.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, bf16_dev, dev, sample_tile_rows

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def dense_weight(K: int, N: int):
    return oracle.quant_wblock(si.weights(N, K))


@functools.lru_cache(maxsize=None)
def sparse_weight(K: int, N: int):
    c = si.column_norms(si.calibration_batch(K))
    return oracle.prune24_compress(si.weights(N, K), c)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("M", [1, 2, 5, 8, 16, 32, 37, 64])
@pytest.mark.parametrize("name,K,N", si.LLAMA3_8B)
def test_block_linear_llama(gpu_lib, name, K, N, M):
    x = si.activations(M, K)
    wq, ws = dense_weight(K, N)
    xd, wqd, wsd = bf16_dev(x), dev(wq), dev(ws)
    y = gpu_lib.fp8_block_linear(xd, wqd, wsd)
    xq, xs = gpu_lib.fp8_quant_act(xd)
    assert same_bits(y, gpu_lib.fp8_block_gemm(xq, xs, wqd, wsd)), f"{name} M={M}: fused != two-step"
    rxq, rxs = oracle.quant_act(x)
    rows = np.unique(np.array([0, M // 2, M - 1]))
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.gemm(rxq, rxs, wq, ws, rows=rows),
                      f"{name} M={M}")


@pytest.mark.parametrize("M", [1, 2, 16, 40, 64])
@pytest.mark.parametrize("name,K,N", si.LLAMA3_8B)
def test_sparse24_linear_llama(gpu_lib, name, K, N, M):
    x = si.activations(M, K)
    vals, meta, ws = sparse_weight(K, N)
    xd, vd, md, wsd = bf16_dev(x), dev(vals), dev(meta), dev(ws)
    y = gpu_lib.fp8_sparse24_linear(xd, vd, md, wsd)
    xq, xs = gpu_lib.fp8_quant_act(xd)
    assert same_bits(y, gpu_lib.fp8_sparse24_gemm(xq, xs, vd, md, wsd)), f"{name} M={M}: fused != two-step"
    rxq, rxs = oracle.quant_act(x)
    rows = np.unique(np.array([0, M // 2, M - 1]))
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.sparse24_gemm(rxq, rxs, vals, meta, ws, rows=rows),
                      f"{name} M={M}")


def edge_activations() -> np.ndarray:
    """Groups that take every branch of the in-kernel quantizer: zero groups,
    bf16 subnormals (subnormal fp32 scale), e4m3 rounding midpoints (exact
    division fallback), +-448-scaled ramps and heavy tails."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((12, 1024)).astype(np.float32)
    x[0, :128] = 0.0
    x[0, 128:256] = -0.0
    x[1, :128] = rng.standard_normal(128) * 1e-39
    x[1, 128:256] = rng.standard_normal(128) * 1e38
    x[2, :128] = np.float32(2.0 ** -133)
    x[3, :] = np.tile(np.linspace(-448, 448, 128, dtype=np.float32), 8)
    x[4, :] = np.tile(np.float32(432.0) * np.arange(1, 129, dtype=np.float32) / 128, 8)
    x[5, :] = -x[4, :]
    z = rng.standard_normal((4, 6, 1024))
    x[6:12] = (z[0] / np.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3)).astype(np.float32)
    return si.to_bf16_bits(torch.from_numpy(x))


def test_linear_edge_groups(gpu_lib):
    x = edge_activations()
    M, K = x.shape
    N = 256
    w = si.weights(N, K)
    wq, ws = oracle.quant_wblock(w)
    vals, meta, ws2 = oracle.prune24_compress(w)
    xd = bf16_dev(x)
    xq, xs = gpu_lib.fp8_quant_act(xd)
    y = gpu_lib.fp8_block_linear(xd, dev(wq), dev(ws))
    y2 = gpu_lib.fp8_sparse24_linear(xd, dev(vals), dev(meta), dev(ws2))
    assert same_bits(y, gpu_lib.fp8_block_gemm(xq, xs, dev(wq), dev(ws)))
    assert same_bits(y2, gpu_lib.fp8_sparse24_gemm(xq, xs, dev(vals), dev(meta), dev(ws2)))
    rxq, rxs = oracle.quant_act(x)
    # rows with finite, non-overflowing products only (row 1 mixes 1e-39 and 1e38 groups)
    rows = np.array([0, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11])
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.gemm(rxq, rxs, wq, ws, rows=rows), "dense")
    assert_gemm_close(y2[torch.from_numpy(rows).to("cuda")],
                      oracle.sparse24_gemm(rxq, rxs, vals, meta, ws2, rows=rows), "sparse")


def test_linear_empty_and_too_large(gpu_lib):
    wq, ws = dense_weight(4096, 4096)
    y = gpu_lib.fp8_block_linear(torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda"), dev(wq), dev(ws))
    assert tuple(y.shape) == (0, 4096)
    with pytest.raises(gpu_lib.Fp8LinError) as err:
        gpu_lib.fp8_block_linear(torch.zeros((65, 4096), dtype=torch.bfloat16, device="cuda"), dev(wq), dev(ws))
    assert err.value.status == gpu_lib.FP8L_ERR_SHAPE


def test_linear_deterministic(gpu_lib):
    x = bf16_dev(si.activations(16, 14336))
    wq, ws = dense_weight(14336, 4096)
    a = gpu_lib.fp8_block_linear(x, dev(wq), dev(ws))
    b = gpu_lib.fp8_block_linear(x, dev(wq), dev(ws))
    assert same_bits(a, b)


# ------------------------------------------------- GEMM + SwiGLU epilogue ---

@functools.lru_cache(maxsize=None)
def gate_up_weight(K: int, I: int):
    """[gate; up] stacked weight (the Llama-3-8B gate/up shape when I = 14336)."""
    return oracle.quant_wblock(si.weights(2 * I, K))


@pytest.mark.parametrize("M,I,K", [(4096, 14336, 4096), (300, 256, 640), (16, 128, 128), (513, 384, 1152),
                                   (1, 14336, 4096), (64, 14336, 4096), (200, 14336, 4096), (97, 384, 1152)])
def test_gemm_swiglu(gpu_lib, M, I, K):
    x = si.activations(M, K, outliers=(K == 4096))
    xq, xs = oracle.quant_act(x)
    wq, ws = gate_up_weight(K, I)
    h, hq, hs = gpu_lib.fp8_block_gemm_swiglu(dev(xq), dev(xs), dev(wq), dev(ws))
    rows = sample_tile_rows(M, 8, seed=9)  # every 128-token tile: first, last and a seeded row
    assert_gemm_close(h[torch.from_numpy(rows).to("cuda")], oracle.gemm_swiglu(xq, xs, wq, ws, rows=rows),
                      f"h {M}x{I}x{K}")
    # the fused quantization equals fp8_quant_act of the stored h, bit for bit (oracle and library quantizer)
    h_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)
    rq, rs = oracle.quant_act(h_bits[rows])
    assert np.array_equal(hq.cpu().numpy()[rows], rq)
    assert np.array_equal(hs.cpu().numpy()[rows].view(np.uint32), rs.view(np.uint32))
    lq, ls = gpu_lib.fp8_quant_act(h)
    assert torch.equal(lq, hq) and torch.equal(ls.view(torch.int32), hs.view(torch.int32))


@pytest.mark.parametrize("M,I,K", [(4096, 14336, 4096), (300, 256, 640), (16, 128, 128), (64, 14336, 4096)])
def test_gemm_swiglu_quantized_only(gpu_lib, M, I, K):
    """h not stored (NULL): the codes and scales equal, bit for bit, those of the call that stores h, on the
    fused kernel (prefill M) and on the partials path (few tokens)."""
    xq, xs = oracle.quant_act(si.activations(M, K, outliers=(K == 4096)))
    wq, ws = gate_up_weight(K, I)
    h, hq, hs = gpu_lib.fp8_block_gemm_swiglu(dev(xq), dev(xs), dev(wq), dev(ws))
    h2, hq2, hs2 = gpu_lib.fp8_block_gemm_swiglu(dev(xq), dev(xs), dev(wq), dev(ws), keep_h=False)
    assert h2 is None
    assert torch.equal(hq, hq2) and torch.equal(hs.view(torch.int32), hs2.view(torch.int32))


def test_gemm_swiglu_without_quantization(gpu_lib):
    M, I, K = 256, 256, 512
    xq, xs = oracle.quant_act(si.activations(M, K, outliers=False))
    wq, ws = gate_up_weight(K, I)
    h, hq, hs = gpu_lib.fp8_block_gemm_swiglu(dev(xq), dev(xs), dev(wq), dev(ws), quantize=False)
    assert hq is None and hs is None
    h2, _, _ = gpu_lib.fp8_block_gemm_swiglu(dev(xq), dev(xs), dev(wq), dev(ws))
    assert same_bits(h, h2)
    assert_gemm_close(h, oracle.gemm_swiglu(xq, xs, wq, ws), "h")
