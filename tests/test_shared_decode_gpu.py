"""The shared-token form of the decode GEMMs (decode_shared_kernel), against
the oracle on every output element.

fp8_block_gemm takes it for 3 to 16 tokens on K < 8192 when the weight has at
least 16384 rows (the waves split each band's units), fp8_sparse24_gemm for 3
to 16 tokens (split units at 3 and 4 tokens, whole bands per wave from 5).  The cases cover both grids (two
workgroups per compute unit up to 8 tokens, one above), bands per workgroup
fewer than its waves (2:4: 4 or 7 bands over 16 waves), token
counts that leave rows of the 16-row fragment past M (they re-read the last
token and are not stored), K
ranges of 1 to 4 units per wave and band (equal and unequal over the
waves), and the fused linear entry points, which
quantize the tokens first and then take the same kernel.  Tolerances as in
test_parity_gpu."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, dev

pytestmark = pytest.mark.gpu


def acts(M, K, seed):
    x = si.activations(M, K, seed=seed)
    return x, oracle.quant_act(x)


@pytest.mark.parametrize("M,N,K", [(3, 16384, 2048), (5, 16384, 2048), (7, 16384, 5120), (8, 28672, 4096),
                                   (11, 28672, 4096), (16, 28672, 4096), (16, 16384, 2048), (4, 32768, 4096),
                                   (13, 16384, 7168), (6, 16384, 7168)])
def test_dense_shared_decode(gpu_lib, M, N, K):
    """Weight tiles in whole rows from 12 tokens (or 5 on K >= 6144) where the LDS holds them: (16, 28672, 4096),
    (16, 16384, 2048), (13, 16384, 7168) and (6, 16384, 7168); fragments at 3-11 tokens on shorter K."""
    _, (xq, xs) = acts(M, K, 41 + M)
    wq, ws = oracle.quant_wblock(si.weights(N, K, seed=7 + N % 97))
    y = gpu_lib.fp8_block_gemm(dev(xq), dev(xs), dev(wq), dev(ws))
    assert_gemm_close(y, oracle.gemm(xq, xs, wq, ws), f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(3, 16384, 4096), (6, 16384, 5120), (8, 28672, 4096), (12, 16384, 2048),
                                   (16, 28672, 4096), (16, 16384, 7168), (5, 18432, 7168)])
def test_sparse_shared_decode(gpu_lib, M, N, K):
    """From 5 tokens the weight comes in whole-row tiles where they fit beside the staged tokens; (16, 16384, 7168)
    does not fit and keeps fragments."""
    _, (xq, xs) = acts(M, K, 43 + M)
    w = si.weights(N, K, seed=11 + N % 89)
    vals, meta, ws = oracle.prune24_compress(w)
    y = gpu_lib.fp8_sparse24_gemm(dev(xq), dev(xs), dev(vals), dev(meta), dev(ws))
    assert_gemm_close(y, oracle.sparse24_gemm(xq, xs, vals, meta, ws), f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(5, 16384, 2048), (12, 16384, 2048)])
def test_dense_linear_shared_decode(gpu_lib, M, N, K):
    x, (xq, xs) = acts(M, K, 47 + M)
    wq, ws = oracle.quant_wblock(si.weights(N, K, seed=13))
    xb = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda")
    y = gpu_lib.fp8_block_linear(xb, dev(wq), dev(ws))
    assert_gemm_close(y, oracle.gemm(xq, xs, wq, ws), f"linear {M}x{N}x{K}")


def test_shared_decode_repeatable(gpu_lib):
    """Fixed order of the waves' partial sums: two calls agree bit for bit."""
    _, (xq, xs) = acts(16, 4096, 3)
    wq, ws = oracle.quant_wblock(si.weights(28672, 4096, seed=5))
    a = gpu_lib.fp8_block_gemm(dev(xq), dev(xs), dev(wq), dev(ws))
    b = gpu_lib.fp8_block_gemm(dev(xq), dev(xs), dev(wq), dev(ws))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
