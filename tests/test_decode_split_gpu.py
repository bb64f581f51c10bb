"""Decode-sized GEMMs whose K is split over several workgroups per row band.

Long-K weights with few 16-row bands (N < 6144, K >= 8192) at 9 to 32 tokens
run 64-row bands with K split four ways: each split stores fp32 partial sums
in library scratch memory and a second kernel adds them in split order.
Covered here, against the oracle:

  * the Llama-3-8B down weight at 9, 16, 20, 21 and 32 tokens (from 21 on
    it would otherwise take the tile kernel), and at 8 (one split);
  * K < 8192 on few row bands at 33 to 64 tokens: 32-row bands with K split
    in two (the o_proj weight at 48 and 64 tokens; K = 640, five K blocks:
    splits of 3 and 2);
  * ragged splits: K = 8320 (65 K blocks: splits of 17, 17, 17 and 14), fewer
    row bands than splits (N = 128), two 16-token column tiles (M = 32), and
    M = 40, past the split configurations;
  * dense, 2:4 and UE8M0 weights (the three GEMMs share the decode kernel);
  * the 2:4 kernel's four-block units: exactly one unit per wave (3 tokens
    over 64 K blocks with 16 waves; 32 blocks over 8 waves) and ragged unit
    counts per split (K = 12800: 25 units split 7, 7, 7 and 4);
  * bit-identical results over repeated calls, and in a captured graph
    replayed several times with eager calls in between."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, dev, llama_sparse_weight, llama_weight, sample_tile_rows

pytestmark = pytest.mark.gpu

SHAPES = [(9, 4096, 14336), (16, 4096, 14336), (20, 4096, 14336), (21, 4096, 14336), (32, 4096, 14336),
          (8, 4096, 14336),
          (12, 512, 8320), (32, 128, 8192), (24, 256, 9216), (40, 512, 8192),
          (48, 4096, 4096), (64, 4096, 4096), (40, 256, 640),
          (3, 384, 8192), (16, 512, 4096), (12, 256, 12800)]


def operands(M, N, K, kind):
    """Device operands and the oracle's result on `rows` for one GEMM."""
    x = si.activations(M, K, outliers=K >= 4096)
    rows = sample_tile_rows(M, 8) if M > 8 else np.arange(M)
    if kind == "ue8m0":
        xq, xe = oracle.quant_act_ue8m0(x)
        wq, we = oracle.quant_wblock_ue8m0(si.weights(N, K))
        return (xq, xe, wq, we), rows, oracle.gemm_ue8m0(xq, xe, wq, we, rows=rows)
    xq, xs = oracle.quant_act(x)
    if kind == "dense":
        _, (wq, ws) = llama_weight(K, N)
        return (xq, xs, wq, ws), rows, oracle.gemm(xq, xs, wq, ws, rows=rows)
    _, (vals, meta, ws) = llama_sparse_weight(K, N, True)
    return (xq, xs, vals, meta, ws), rows, oracle.sparse24_gemm(xq, xs, vals, meta, ws, rows=rows)


def call(gpu_lib, kind, ops, y=None):
    fn = {"dense": gpu_lib.fp8_block_gemm, "sparse": gpu_lib.fp8_sparse24_gemm,
          "ue8m0": gpu_lib.fp8_block_gemm_ue8m0}[kind]
    return fn(*ops, y) if y is not None else fn(*ops)


@pytest.mark.parametrize("kind", ["dense", "sparse", "ue8m0"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_split_k_decode_matches_oracle(gpu_lib, M, N, K, kind):
    ops, rows, ref = operands(M, N, K, kind)
    y = call(gpu_lib, kind, [dev(a) for a in ops])
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], ref, f"{kind} {M}x{N}x{K}")


@pytest.mark.parametrize("kind", ["dense", "sparse"])
def test_split_k_decode_repeatable(gpu_lib, kind):
    ops, _, _ = operands(16, 4096, 14336, kind)
    d = [dev(a) for a in ops]
    first = call(gpu_lib, kind, d)
    for i in range(10):
        again = call(gpu_lib, kind, d)
        assert torch.equal(again.view(torch.int16), first.view(torch.int16)), f"call {i}"


def test_split_k_decode_graph_replays(gpu_lib):
    """Three split GEMMs with different row-band counts and K ranges,
    captured in one graph; replays alternate with eager calls of the same
    shapes on the graph's stream and on the default stream."""
    cases = []
    for M, N, K, kind in ((16, 4096, 14336, "dense"), (12, 512, 8320, "sparse"), (32, 128, 8192, "dense")):
        ops, _, _ = operands(M, N, K, kind)
        d = [dev(a) for a in ops]
        ref = call(gpu_lib, kind, d)
        cases.append((kind, d, ref))
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
    for rep in range(4):
        for y in outs:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, ((kind, d, ref), y) in enumerate(zip(cases, outs)):
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {rep}, case {i}"
        # eager calls in between, on the graph's stream and on the default stream
        with torch.cuda.stream(s):
            for kind, d, ref in cases[::-1]:
                assert torch.equal(call(gpu_lib, kind, d).view(torch.int16), ref.view(torch.int16))
        for kind, d, ref in cases:
            assert torch.equal(call(gpu_lib, kind, d).view(torch.int16), ref.view(torch.int16))
