"""Decode GEMMs on quantized tokens that go through LDS.

The decode kernel reads quantized tokens in one of three modes
(gemm_decode.hpp, QuantTokensT and launch_decode_kernel):
  * mode 2, from 17 tokens on where every wave of every K split has at least
    two one-block units and at most 16 fragments are in flight per wave: the
    scales of the K range are copied into LDS once per workgroup (linear
    loads, odd row stride), and each wave loads its token code tiles in whole
    128-byte rows, writes them to its own LDS tile and reads the MFMA
    fragments back;
  * mode 1, from 8 tokens on where mode 2 does not apply and the registers
    fit: the code tiles as in mode 2, the scales from global memory;
  * mode 0 otherwise: codes and scales as fragments from global memory.
Covered here:

  * against the oracle: the 6144- and 4096-row Llama weights at 17 to 64
    tokens (ragged token tiles, one and two K splits), the long-K down weight
    split four ways, a ragged K (33 K blocks), dense and 2:4;
  * the two paths give the same bits where the kernel configuration is the
    same: the first 16 rows of a 17-token call (through LDS) equal a 16-token
    call (from global memory);
  * graph replays of the LDS path with eager calls in between."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, dev, llama_sparse_weight, llama_weight

pytestmark = pytest.mark.gpu

# (M, N, K), with the mode each GEMM takes (dense / 2:4)
CASES = [(17, 6144, 4096), (23, 6144, 4096),   # 2 / 0 (2:4 four-block units, one per wave)
         (33, 6144, 4096), (64, 6144, 4096), (40, 6144, 4224), (48, 4096, 4096), (64, 4096, 4096),  # 2 / 2
         (17, 4096, 4096), (24, 4096, 4096),   # 2 / 1
         (20, 4096, 14336), (32, 4096, 14336),  # 2 / 2 (K split four ways)
         (8, 6144, 4096), (12, 4096, 4096), (16, 6144, 4096),  # 1 / 1
         (9, 4096, 14336),  # 1 / 0 (split K, 2:4 four-block units)
         (5, 6144, 4096)]  # 0 / 0


def operands(M, N, K, kind, seed_shift=0):
    x = si.activations(M, K, outliers=True, seed=11 + seed_shift)
    xq, xs = oracle.quant_act(x)
    if kind == "dense":
        _, (wq, ws) = llama_weight(K, N)
        return (xq, xs, wq, ws), oracle.gemm(xq, xs, wq, ws)
    _, (vals, meta, ws) = llama_sparse_weight(K, N, False)
    return (xq, xs, vals, meta, ws), oracle.sparse24_gemm(xq, xs, vals, meta, ws)


def call(gpu_lib, kind, ops, y=None):
    fn = gpu_lib.fp8_block_gemm if kind == "dense" else gpu_lib.fp8_sparse24_gemm
    return fn(*ops, y) if y is not None else fn(*ops)


@pytest.mark.parametrize("kind", ["dense", "sparse"])
@pytest.mark.parametrize("M,N,K", CASES)
def test_staged_scales_match_oracle(gpu_lib, M, N, K, kind):
    ops, ref = operands(M, N, K, kind)
    y = call(gpu_lib, kind, [dev(a) for a in ops])
    assert_gemm_close(y, ref, f"{kind} {M}x{N}x{K}")


@pytest.mark.parametrize("N", [6144, 4096])
def test_staged_scales_bit_identical_to_global_scales(gpu_lib, N):
    """At 16 and 17 tokens on these weights the decode kernel has the same row
    bands, waves and load depth, so each output row is summed in the same
    order; only how the tokens are read differs (modes 1 and 2)."""
    K = 4096
    ops17, _ = operands(17, N, K, "dense")
    xq17, xs17, wq, ws = ops17
    y17 = call(gpu_lib, "dense", [dev(a) for a in ops17])
    y16 = call(gpu_lib, "dense", [dev(xq17[:16]), dev(xs17[:16]), dev(wq), dev(ws)])
    torch.cuda.synchronize()
    assert torch.equal(y17[:16].view(torch.int16), y16.view(torch.int16))


def test_staged_scales_graph_replays(gpu_lib):
    cases = []
    for M, N, K, kind in ((64, 6144, 4096, "dense"), (32, 4096, 14336, "dense"), (48, 4096, 4096, "sparse")):
        ops, _ = operands(M, N, K, kind, seed_shift=1)
        d = [dev(a) for a in ops]
        cases.append((kind, d, call(gpu_lib, kind, d)))
    torch.cuda.synchronize()
    outs = [torch.zeros_like(ref) for _, _, ref in cases]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for (kind, d, _), y in zip(cases, outs):
                call(gpu_lib, kind, d, y)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in outs:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, ((kind, d, ref), y) in enumerate(zip(cases, outs)):
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {rep}, case {i}"
        for kind, d, ref in cases:
            assert torch.equal(call(gpu_lib, kind, d).view(torch.int16), ref.view(torch.int16))
