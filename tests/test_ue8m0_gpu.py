"""Parity of the UE8M0 (power-of-two scale) calls through the C ABI with the CPU
oracle: codes and exponent bytes bit-exact; the GEMM within the stated tolerance
(||Y - Y_ref||_F / ||Y_ref||_F <= 5e-3 and |Y - Y_ref| <= 2^-7 |Y_ref| +
1e-3 max|Y_ref| element-wise) of the oracle fed the oracle's own codes."""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, bf16_dev, dev, host, sample_tile_rows
from test_linear_gpu import edge_activations

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,dist", [(16, 512, "normal"), (37, 4096, "normal"), (300, 640, "normal"),
                                      (4096, 14336, "normal"), (1024, 18432, "student_t3")])
def test_quant_act_ue8m0_bit_exact(gpu_lib, M, K, dist):
    x = si.activations(M, K, dist=dist, outliers=(dist == "normal"))
    q, e = gpu_lib.fp8_quant_act_ue8m0(bf16_dev(x))
    rq, re = oracle.quant_act_ue8m0(x)
    assert np.array_equal(host(e), re)
    assert np.array_equal(host(q), rq)


def test_quant_act_ue8m0_edge_groups(gpu_lib):
    x = edge_activations()
    q, e = gpu_lib.fp8_quant_act_ue8m0(bf16_dev(x))
    rq, re = oracle.quant_act_ue8m0(x)
    assert np.array_equal(host(e), re) and np.array_equal(host(q), rq)
    # every bf16 value once, in groups that mix magnitudes
    bits = np.arange(65536, dtype=np.uint32)
    finite = bits[np.isfinite((bits << 16).view(np.float32))].astype(np.uint16)
    xa = np.concatenate([finite, finite[:(-finite.size) % 128]]).reshape(-1, 256)
    q, e = gpu_lib.fp8_quant_act_ue8m0(bf16_dev(xa))
    rq, re = oracle.quant_act_ue8m0(xa)
    assert np.array_equal(host(e), re) and np.array_equal(host(q), rq)


@pytest.mark.parametrize("N,K,std", [(512, 512, 0.02), (384, 640, 0.02), (28672, 4096, 0.02), (7168, 18432, 0.01)])
def test_quant_wblock_ue8m0_bit_exact(gpu_lib, N, K, std):
    w = si.weights(N, K, std=std)
    q, e = gpu_lib.fp8_quant_weight_block_ue8m0(bf16_dev(w))
    rq, re = oracle.quant_wblock_ue8m0(w)
    assert np.array_equal(host(e), re)
    assert np.array_equal(host(q), rq)


@functools.lru_cache(maxsize=None)
def weight_ue8m0(K: int, N: int, std: float = 0.02):
    return oracle.quant_wblock_ue8m0(si.weights(N, K, std=std))


@pytest.mark.parametrize("M", [1, 8, 64, 4096])
@pytest.mark.parametrize("name,K,N", si.LLAMA3_8B)
def test_gemm_ue8m0_llama(gpu_lib, name, K, N, M):
    xq, xe = oracle.quant_act_ue8m0(si.activations(M, K))
    wq, we = weight_ue8m0(K, N)
    y = gpu_lib.fp8_block_gemm_ue8m0(dev(xq), dev(xe), dev(wq), dev(we))
    rows = sample_tile_rows(M, 10) if M > 8 else np.arange(M)
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.gemm_ue8m0(xq, xe, wq, we, rows=rows),
                      f"{name} M={M}")


@pytest.mark.parametrize("name,K,N", si.DSV3_FFN)
def test_gemm_ue8m0_dsv3_sampled(gpu_lib, name, K, N):
    x = si.activations(si.DSV3_M, K, dist="student_t3", outliers=False)
    xq, xe = oracle.quant_act_ue8m0(x)
    wq, we = weight_ue8m0(K, N, 0.01)
    y = gpu_lib.fp8_block_gemm_ue8m0(dev(xq), dev(xe), dev(wq), dev(we))
    rows = sample_tile_rows(si.DSV3_M, 6)
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.gemm_ue8m0(xq, xe, wq, we, rows=rows), name)


@pytest.mark.parametrize("M,N,K", [(65, 384, 640), (300, 256, 1152), (3, 128, 256), (512, 512, 384), (40, 384, 256)])
def test_gemm_ue8m0_ragged(gpu_lib, M, N, K):
    xq, xe = oracle.quant_act_ue8m0(si.activations(M, K, outliers=False))
    wq, we = oracle.quant_wblock_ue8m0(si.weights(N, K))
    y = gpu_lib.fp8_block_gemm_ue8m0(dev(xq), dev(xe), dev(wq), dev(we))
    assert_gemm_close(y, oracle.gemm_ue8m0(xq, xe, wq, we), f"{M}x{N}x{K}")


def test_gemm_ue8m0_equals_fp32_scale_gemm_on_power_of_two_scales(gpu_lib):
    """With scales that are powers of two, the two GEMMs compute the same sums."""
    M, K, N = 512, 4096, 1024
    xq, xe = oracle.quant_act_ue8m0(si.activations(M, K))
    wq, we = weight_ue8m0(K, N)
    y8 = gpu_lib.fp8_block_gemm_ue8m0(dev(xq), dev(xe), dev(wq), dev(we))
    y32 = gpu_lib.fp8_block_gemm(dev(xq), dev(oracle.ue8m0_to_f32(xe)), dev(wq), dev(oracle.ue8m0_to_f32(we)))
    ref = oracle.gemm_ue8m0(xq, xe, wq, we)
    assert_gemm_close(y8, ref, "ue8m0")
    assert_gemm_close(y32, ref, "fp32 scales")
    d = (y8.float() - y32.float()).abs().max().item()
    assert d <= 2.0 ** -7 * y32.float().abs().max().item()


def test_ue8m0_end_to_end(gpu_lib):
    M, K, N = 64, 4096, 6144
    x, w = si.activations(M, K), si.weights(N, K)
    xq, xe = gpu_lib.fp8_quant_act_ue8m0(bf16_dev(x))
    wq, we = gpu_lib.fp8_quant_weight_block_ue8m0(bf16_dev(w))
    y = gpu_lib.fp8_block_gemm_ue8m0(xq, xe, wq, we)
    rxq, rxe = oracle.quant_act_ue8m0(x)
    rwq, rwe = oracle.quant_wblock_ue8m0(w)
    assert_gemm_close(y, oracle.gemm_ue8m0(rxq, rxe, rwq, rwe), "ue8m0 path")
