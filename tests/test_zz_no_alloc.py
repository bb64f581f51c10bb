"""fp8_block_gemm_noalloc against fp8_block_gemm, through the C ABI.

The no-allocation entry point runs the same kernels as fp8_block_gemm, with the
split-K partials in the library's fixed device array instead of allocated
scratch, so its output must equal fp8_block_gemm's bit for bit (and both meet
the GEMM tolerance against the oracle).  Each case makes two calls in a row on
the shared array, the second with a smaller input, so the second call runs on
the first call's leftover partials.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, dev, sample_tile_rows

pytestmark = pytest.mark.gpu

# (M, N, K) pairs, the second smaller than the first:
#  * 512 x 8192 x 4096: 128 tiles of 128 x 256, K split in two: 32 MiB of
#    partials, the array's whole size;
#  * 128 and 64 tokens on the 4096 x 14336 weight: 16 tiles, 14 splits;
#  * 16 and 12 tokens on the same weight: the weight-streaming kernel, K split four ways;
#  * 4096 and 300 tokens on 1024 x 512: no split (no scratch), then a ragged split.
CASES = [((512, 8192, 4096), (200, 8192, 4096)),
         ((128, 4096, 14336), (64, 4096, 14336)),
         ((16, 4096, 14336), (12, 4096, 14336)),
         ((4096, 1024, 512), (300, 1024, 512))]


def _operands(M, N, K, seed):
    x = si.activations(M, K, outliers=K >= 4096, seed=seed)
    w = si.weights(N, K, seed=seed + 1)
    xq, xs = oracle.quant_act(x)
    wq, ws = oracle.quant_wblock(w)
    return xq, xs, wq, ws


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_equals_block_gemm(gpu_lib, first, second):
    for i, (M, N, K) in enumerate((first, second)):
        print(f"noalloc case M={M} N={N} K={K} (call {i + 1} of 2)", flush=True)
        xq, xs, wq, ws = _operands(M, N, K, seed=10 + i)
        dxq, dxs, dwq, dws = dev(xq), dev(xs), dev(wq), dev(ws)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        gpu_lib.fp8_block_gemm_noalloc(dxq, dxs, dwq, dws, y)
        ref = gpu_lib.fp8_block_gemm(dxq, dxs, dwq, dws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"M={M} N={N} K={K}"
        rows = sample_tile_rows(M, 4)
        assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.gemm(xq, xs, wq, ws, rows=rows),
                          f"noalloc {M}x{N}x{K}")


def test_noalloc_repeats_and_interleaves(gpu_lib):
    """Back-to-back calls of two shapes on one stream reuse the array in turn and
    stay equal to fp8_block_gemm."""
    a = _operands(128, 4096, 14336, seed=20)
    b = _operands(48, 4096, 14336, seed=22)
    da = [dev(t) for t in a]
    db = [dev(t) for t in b]
    ya = torch.empty((128, 4096), dtype=torch.bfloat16, device="cuda")
    yb = torch.empty((48, 4096), dtype=torch.bfloat16, device="cuda")
    ra = gpu_lib.fp8_block_gemm(*da)
    rb = gpu_lib.fp8_block_gemm(*db)
    for _ in range(3):
        gpu_lib.fp8_block_gemm_noalloc(*da, ya)
        gpu_lib.fp8_block_gemm_noalloc(*db, yb)
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int16), ra.view(torch.int16))
        assert torch.equal(yb.view(torch.int16), rb.view(torch.int16))
