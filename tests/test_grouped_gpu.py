"""Parity of the grouped (mixture-of-experts) GEMM through the C ABI with the CPU
oracle, on DeepSeek-V3-like expert shapes with seeded, uneven routing (empty
experts, experts smaller and larger than a 256-token tile).  Tolerance as for
fp8_block_gemm: ||Y - Y_ref||_F / ||Y_ref||_F <= 5e-3 and |Y - Y_ref| <=
2^-7 |Y_ref| + 1e-3 max|Y_ref| element-wise."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, dev

pytestmark = pytest.mark.gpu


routed_offsets = si.routed_offsets  # seeded uneven routing (some experts empty), summing to M


def expert_weights(G: int, N: int, K: int, seed: int):
    wq, ws = [], []
    for g in range(G):
        q, s = oracle.quant_wblock(si.weights(N, K, std=0.01, seed=seed + g))
        wq.append(q)
        ws.append(s)
    return np.stack(wq), np.stack(ws)


@pytest.mark.parametrize("M,G,N,K", [(2048, 8, 4096, 7168), (1000, 16, 2048, 1024), (300, 3, 256, 640)])
def test_grouped_gemm(gpu_lib, M, G, N, K):
    x = si.activations(M, K, dist="student_t3", outliers=False)
    xq, xs = oracle.quant_act(x)
    wq, ws = expert_weights(G, N, K, seed=40)
    offsets = routed_offsets(M, G, seed=M + G)
    y = gpu_lib.fp8_grouped_gemm(dev(xq), dev(xs), dev(wq), dev(ws), dev(offsets))
    # rows at every group boundary and a seeded sample
    rows = np.unique(np.concatenate([np.clip(np.concatenate([offsets, offsets - 1]), 0, M - 1),
                                     si.sample_rows(M, 16, seed=13)]))
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.grouped_gemm(xq, xs, wq, ws, offsets, rows=rows),
                      f"grouped M={M} G={G}")
    # every row of every group against fp8_block_gemm of that group alone (the two
    # may add the fp32 K-block sums in different orders: compared to the tolerance)
    for g in range(G):
        o0, o1 = int(offsets[g]), int(offsets[g + 1])
        if o1 > o0:
            yg = gpu_lib.fp8_block_gemm(dev(xq[o0:o1]), dev(xs[o0:o1]), dev(wq[g]), dev(ws[g]))
            assert_gemm_close(y[o0:o1], yg.float().cpu().numpy().astype(np.float64), f"group {g}")


def test_grouped_gemm_single_group_and_empty(gpu_lib):
    M, K, N = 257, 512, 384
    xq, xs = oracle.quant_act(si.activations(M, K, outliers=False))
    wq, ws = expert_weights(2, N, K, seed=7)
    off = np.array([0, 0, M], np.int32)        # all tokens to expert 1
    y = gpu_lib.fp8_grouped_gemm(dev(xq), dev(xs), dev(wq), dev(ws), dev(off))
    assert_gemm_close(y, oracle.gemm(xq, xs, wq[1], ws[1]), "one non-empty group")


def test_grouped_gemm_few_tokens_and_empty_batch(gpu_lib):
    """Decode-sized routing (a handful of tokens over several experts, some empty)
    and an empty batch."""
    K, N = 1024, 512
    wq, ws = expert_weights(4, N, K, seed=11)
    M = 5
    xq, xs = oracle.quant_act(si.activations(M, K))
    off = np.array([0, 2, 2, 5, 5], np.int32)
    y = gpu_lib.fp8_grouped_gemm(dev(xq), dev(xs), dev(wq), dev(ws), dev(off))
    assert_gemm_close(y, oracle.grouped_gemm(xq, xs, wq, ws, off), "five tokens over four experts")
    xq0 = np.zeros((0, K), np.uint8)
    xs0 = np.zeros((0, K // 128), np.float32)
    y0 = gpu_lib.fp8_grouped_gemm(dev(xq0), dev(xs0), dev(wq), dev(ws), dev(np.zeros(5, np.int32)))
    assert tuple(y0.shape) == (0, N)
