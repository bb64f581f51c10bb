"""The 2:4 tile kernel's two forms of scale accumulation.

Each wave of the tile kernel keeps its running sums either in units of the
current K block's scale (the ratio form: the sparse MFMA accumulates straight
into them) or in absolute units with a scaled FMA per partial (the plain form).
It takes the ratio form only when every scale product it uses is a normal
number in [2^-100, 2^100] and all lie within 2^60 of each other, and no scale
is zero.  Realistic inputs (the other 2:4 tests) run the ratio form; these
cases must run the plain form, and would fail under the ratio form:

  * token groups with scales 2^60 apart (the rescaled sums would overflow);
  * a zero token scale, or a zero weight-block scale, over non-zero codes (the
    ratio form cannot leave out a K block);

plus tiles where only some tokens need the plain form, so that waves of one
workgroup run different forms, and a split-K case.  Every output is checked
against the oracle within the GEMM tolerance."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, dev

pytestmark = pytest.mark.gpu


def sparse_case(M, N, K, seed=0):
    x = si.activations(M, K, outliers=False)
    w = si.weights(N, K)
    vals, meta, ws = oracle.prune24_compress(w)
    return x, (vals, meta, ws)


def scaled_groups(x_bits: np.ndarray, rows, factors) -> np.ndarray:
    """bf16 activations with the 128-groups of `rows` multiplied by factors
    cycling over the groups (exact powers of two)."""
    x = si.bf16_bits_to_f32(x_bits).copy()
    K = x.shape[1]
    for m in rows:
        for g in range(K // 128):
            x[m, 128 * g:128 * g + 128] *= factors[g % len(factors)]
    return si.to_bf16_bits(torch.from_numpy(x.astype(np.float32)))


def run(gpu_lib, xq, xs, vals, meta, ws):
    return gpu_lib.fp8_sparse24_gemm(dev(xq), dev(xs), dev(vals), dev(meta), dev(ws))


@pytest.mark.parametrize("rows", ["all", "some"])
def test_scales_too_far_apart(gpu_lib, rows):
    M, N, K = 256, 512, 2048
    x, (vals, meta, ws) = sparse_case(M, N, K)
    chosen = range(M) if rows == "all" else [3, 70, 129, 200, 255]
    x = scaled_groups(x, chosen, [2.0 ** 60, 2.0 ** -60])
    xq, xs = oracle.quant_act(x)
    assert_gemm_close(run(gpu_lib, xq, xs, vals, meta, ws), oracle.sparse24_gemm(xq, xs, vals, meta, ws),
                      f"scales 2^120 apart, rows {rows}")


def test_zero_token_scale_over_nonzero_codes(gpu_lib):
    M, N, K = 130, 384, 1024
    x, (vals, meta, ws) = sparse_case(M, N, K)
    xq, xs = oracle.quant_act(x)
    xs = xs.copy()
    xs[5, 2] = 0.0     # codes of that group stay non-zero: its K block adds nothing
    xs[129, 0] = 0.0   # in the ragged last token tile
    assert np.any(xq[5, 256:384] != 0)
    assert_gemm_close(run(gpu_lib, xq, xs, vals, meta, ws), oracle.sparse24_gemm(xq, xs, vals, meta, ws),
                      "zero token scales")


def test_zero_weight_scale_over_nonzero_codes(gpu_lib):
    M, N, K = 256, 512, 1024
    x, (vals, meta, ws) = sparse_case(M, N, K)
    xq, xs = oracle.quant_act(x)
    ws = ws.copy()
    ws[1, 3] = 0.0
    assert_gemm_close(run(gpu_lib, xq, xs, vals, meta, ws), oracle.sparse24_gemm(xq, xs, vals, meta, ws),
                      "zero weight block scale")


def test_split_k_with_both_forms(gpu_lib):
    """256 tokens over a 4096 x 14336 weight split K into fp32 partials; a few
    tokens with scales far apart run the plain form in their waves."""
    M, N, K = 256, 4096, 14336
    x, (vals, meta, ws) = sparse_case(M, N, K)
    x = scaled_groups(x, [10, 100], [2.0 ** 50, 1.0, 2.0 ** -50])
    xq, xs = oracle.quant_act(x)
    rows = np.array([0, 10, 11, 100, 200, 255])
    y = run(gpu_lib, xq, xs, vals, meta, ws)
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.sparse24_gemm(xq, xs, vals, meta, ws, rows=rows),
                      "split K, both forms")
