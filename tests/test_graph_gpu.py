"""Calls captured in a HIP graph and replayed: every replay, with eager work and
synchronisations between replays, equals the eager result bit for bit.  Covers
the paths with more than one launch or with a stream-ordered workspace: the
split-K GEMMs (mid-size M), the fused linear through its quantize-then-GEMM
path, the per-tensor quantizer (three launches) and the decode GEMM."""
from __future__ import annotations

import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import bf16_dev, dev, llama_acts, llama_sparse_weight, llama_weight

pytestmark = pytest.mark.gpu


def replay_equals_eager(fn, outs):
    """fn() writes into the tensors in outs; capture it, then replay three times."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream (pool and module state)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {i}"
        fn()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M,name", [(128, "qkv"), (48, "down"), (1, "gate_up")])
def test_graph_dense_gemm(gpu_lib, M, name):
    _, K, N = next(s for s in si.LLAMA3_8B if s[0] == name)
    _, (xq, xs) = llama_acts(M, K)
    _, (wq, ws) = llama_weight(K, N)
    a, b, c, d = dev(xq), dev(xs), dev(wq), dev(ws)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    replay_equals_eager(lambda: gpu_lib.fp8_block_gemm(a, b, c, d, y), [y])


def test_graph_sparse_gemm(gpu_lib):
    M, K, N = 256, 14336, 4096
    _, (xq, xs) = llama_acts(M, K)
    _, (vals, meta, ws) = llama_sparse_weight(K, N, True)
    a, b, v, m, s = dev(xq), dev(xs), dev(vals), dev(meta), dev(ws)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    replay_equals_eager(lambda: gpu_lib.fp8_sparse24_gemm(a, b, v, m, s, y), [y])


def test_graph_linear_quantize_then_gemm(gpu_lib):
    M, K, N = 64, 4096, 28672
    x = bf16_dev(llama_acts(M, K)[0])
    _, (wq, ws) = llama_weight(K, N)
    c, d = dev(wq), dev(ws)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    replay_equals_eager(lambda: gpu_lib.fp8_block_linear(x, c, d, y), [y])


def test_graph_quant_act_tensor(gpu_lib):
    x = bf16_dev(si.activations(300, 4096))
    q = torch.empty((300, 4096), dtype=torch.uint8, device="cuda")
    s = torch.empty((300, 32), dtype=torch.float32, device="cuda")
    replay_equals_eager(lambda: gpu_lib.fp8_quant_act_tensor(x, q, s), [q, s])
    rq, rs = oracle.quant_act_tensor(si.activations(300, 4096))
    assert (q.cpu().numpy() == rq).all() and (s.cpu().numpy() == rs).all()
