"""Block-scaled dense, 2:4 and UE8M0 GEMMs at mid-size M (21 .. ~1000 tokens:
past 20 tokens on the large weights, past 64 on all), where the tile kernel
runs with 256 x 128 tiles and, when the tiles cover at most half of the
compute units, splits K over several workgroups whose fp32 partials are summed
in a second kernel.  Parity with the oracle within the GEMM tolerance, on the
Llama-3-8B and DeepSeek-V3 shapes and ragged ones, and bit-identical repeats."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import (DEV, assert_gemm_close, dev, llama_acts, llama_sparse_weight, llama_weight, run_dense,
                             run_sparse, sample_tile_rows)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [20, 21, 24, 33, 48, 65, 128, 256, 512, 1000])
@pytest.mark.parametrize("name,K,N", si.LLAMA3_8B)
def test_dense_gemm_mid_m(gpu_lib, name, K, N, M):
    _, (xq, xs) = llama_acts(M, K)
    _, (wq, ws) = llama_weight(K, N)
    y = run_dense(gpu_lib, xq, xs, wq, ws)
    rows = sample_tile_rows(M, 10)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], oracle.gemm(xq, xs, wq, ws, rows=rows), f"{name} M={M}")


@pytest.mark.parametrize("M,K,N", [(200, 18432, 7168), (96, 7168, 18432)])
def test_dense_gemm_mid_m_dsv3(gpu_lib, M, K, N):
    x = si.activations(M, K, dist="student_t3", outliers=False)
    w = si.weights(N, K, std=0.01)
    xq, xs = oracle.quant_act(x)
    wq, ws = oracle.quant_wblock(w)
    y = run_dense(gpu_lib, xq, xs, wq, ws)
    rows = sample_tile_rows(M, 8)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], oracle.gemm(xq, xs, wq, ws, rows=rows), f"M={M} K={K}")


@pytest.mark.parametrize("M,N,K", [(130, 384, 2048), (65, 128, 1024), (700, 640, 1152), (97, 256, 4224)])
def test_dense_gemm_mid_m_ragged(gpu_lib, M, N, K):
    """Ragged M and N tails with a split K, including K/128 not a multiple of 4."""
    x = si.activations(M, K, outliers=False)
    w = si.weights(N, K)
    xq, xs = oracle.quant_act(x)
    wq, ws = oracle.quant_wblock(w)
    assert_gemm_close(run_dense(gpu_lib, xq, xs, wq, ws), oracle.gemm(xq, xs, wq, ws), f"{M}x{N}x{K}")


def test_dense_gemm_mid_m_deterministic(gpu_lib):
    _, (xq, xs) = llama_acts(128, 14336)
    _, (wq, ws) = llama_weight(14336, 4096)
    a = run_dense(gpu_lib, xq, xs, wq, ws)
    b = run_dense(gpu_lib, xq, xs, wq, ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("M", [20, 21, 48, 65, 256, 1000])
@pytest.mark.parametrize("name,K,N", si.LLAMA3_8B)
def test_sparse_gemm_mid_m(gpu_lib, name, K, N, M):
    _, (xq, xs) = llama_acts(M, K)
    _, (vals, meta, ws) = llama_sparse_weight(K, N, True)
    y = run_sparse(gpu_lib, xq, xs, vals, meta, ws)
    rows = sample_tile_rows(M, 8)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], oracle.sparse24_gemm(xq, xs, vals, meta, ws, rows=rows),
                      f"2:4 {name} M={M}")


@pytest.mark.parametrize("M,N,K", [(130, 384, 2048), (97, 256, 1152), (700, 640, 4096)])
def test_sparse_gemm_mid_m_ragged(gpu_lib, M, N, K):
    x = si.activations(M, K, outliers=False)
    vals, meta, ws = oracle.prune24_compress(si.weights(N, K))
    xq, xs = oracle.quant_act(x)
    assert_gemm_close(run_sparse(gpu_lib, xq, xs, vals, meta, ws), oracle.sparse24_gemm(xq, xs, vals, meta, ws),
                      f"2:4 {M}x{N}x{K}")


def test_sparse_gemm_mid_m_deterministic(gpu_lib):
    _, (xq, xs) = llama_acts(128, 14336)
    _, (vals, meta, ws) = llama_sparse_weight(14336, 4096, True)
    a = run_sparse(gpu_lib, xq, xs, vals, meta, ws)
    b = run_sparse(gpu_lib, xq, xs, vals, meta, ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("M", [21, 48, 128, 512])
@pytest.mark.parametrize("name,K,N", si.LLAMA3_8B)
def test_ue8m0_gemm_mid_m(gpu_lib, name, K, N, M):
    xq, xe = oracle.quant_act_ue8m0(llama_acts(M, K)[0])
    wq, we = oracle.quant_wblock_ue8m0(llama_weight(K, N)[0])
    y = gpu_lib.fp8_block_gemm_ue8m0(dev(xq), dev(xe), dev(wq), dev(we))
    rows = sample_tile_rows(M, 8)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], oracle.gemm_ue8m0(xq, xe, wq, we, rows=rows),
                      f"ue8m0 {name} M={M}")
