"""The 2:4 tile kernel's two forms of scale accumulation.

Each wave of the tile kernel keeps its running sums either in units of the
current K block's scale (the ratio form: the sparse MFMA accumulates straight
into them) or in absolute units with a scaled FMA per partial (the plain form).
It takes the ratio form only when every scale product it uses is a normal
number in [2^-100, 2^100] and all lie within 2^60 of each other, and no scale
is zero.  Realistic inputs (the other 2:4 tests) run the ratio form; these
cases must run the plain form, and would fail under the ratio form:

  * token groups with scales 2^120 apart (the rescaled sums would overflow);
  * a zero token scale, or a zero weight-block scale, over non-zero codes (the
    ratio form cannot leave out a K block);

plus tiles where only some tokens need the plain form, so that waves of one
workgroup run different forms, a split-K launch with short K ranges (the plain
form throughout) and one whose ranges are long enough for the ratio form
(mixed waves again).  Every output is checked against the oracle within the
GEMM tolerance."""
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


# 2304 tokens over a 4096 x 4096 weight: 9 x 16 = 144 tiles of 256 x 256 (no
# split K, more than half the compute units busy) with 32 K blocks each, so
# every wave is eligible for the ratio form and the checks decide.
BIG = (2304, 4096, 4096)
SAMPLE = np.array([0, 3, 5, 70, 129, 200, 255, 256, 1000, 2047, 2303])


def check_sampled(gpu_lib, xq, xs, vals, meta, ws, what):
    y = run(gpu_lib, xq, xs, vals, meta, ws)
    assert_gemm_close(y[torch.from_numpy(SAMPLE).to("cuda")],
                      oracle.sparse24_gemm(xq, xs, vals, meta, ws, rows=SAMPLE), what)


@pytest.mark.parametrize("rows", ["all", "some"])
def test_scales_too_far_apart(gpu_lib, rows):
    """Groups scaled by 2^60 and 2^-60 in turn: the ratio form would rescale its
    sums by 2^120 and overflow."""
    M, N, K = BIG
    x, (vals, meta, ws) = sparse_case(M, N, K)
    chosen = range(M) if rows == "all" else [3, 70, 129, 1000, 2303]
    x = scaled_groups(x, chosen, [2.0 ** 60, 2.0 ** -60])
    xq, xs = oracle.quant_act(x)
    check_sampled(gpu_lib, xq, xs, vals, meta, ws, f"scales 2^120 apart, rows {rows}")


def test_zero_token_scale_over_nonzero_codes(gpu_lib):
    M, N, K = BIG
    x, (vals, meta, ws) = sparse_case(M, N, K)
    xq, xs = oracle.quant_act(x)
    xs = xs.copy()
    xs[5, 2] = 0.0      # codes of that group stay non-zero: its K block adds nothing
    xs[2303, 31] = 0.0  # the last token, the last K block
    assert np.any(xq[5, 256:384] != 0) and np.any(xq[2303, 31 * 128:] != 0)
    check_sampled(gpu_lib, xq, xs, vals, meta, ws, "zero token scales")


def test_zero_weight_scale_over_nonzero_codes(gpu_lib):
    M, N, K = BIG
    x, (vals, meta, ws) = sparse_case(M, N, K)
    xq, xs = oracle.quant_act(x)
    ws = ws.copy()
    ws[1, 3] = 0.0
    check_sampled(gpu_lib, xq, xs, vals, meta, ws, "zero weight block scale")


def test_split_k_short_ranges(gpu_lib):
    """256 tokens over a 4096 x 14336 weight split K into fp32 partials of 7 K
    blocks each: too short for the ratio form's scan, so every wave runs the
    plain form (including the tokens with scales far apart)."""
    M, N, K = 256, 4096, 14336
    x, (vals, meta, ws) = sparse_case(M, N, K)
    x = scaled_groups(x, [10, 100], [2.0 ** 50, 1.0, 2.0 ** -50])
    xq, xs = oracle.quant_act(x)
    rows = np.array([0, 10, 11, 100, 200, 255])
    y = run(gpu_lib, xq, xs, vals, meta, ws)
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.sparse24_gemm(xq, xs, vals, meta, ws, rows=rows),
                      "split K, short ranges")


def test_split_k_long_ranges_mixed_forms(gpu_lib):
    """512 tokens over an 8192 x 16384 weight: the split-K plan gives each
    workgroup at least 32 K blocks, so waves take the ratio form, except those
    holding the few tokens with scales 2^120 apart."""
    M, N, K = 512, 8192, 16384
    x, (vals, meta, ws) = sparse_case(M, N, K)
    x = scaled_groups(x, [7, 300], [2.0 ** 60, 2.0 ** -60])
    xq, xs = oracle.quant_act(x)
    rows = np.array([0, 7, 8, 64, 300, 301, 511])
    y = run(gpu_lib, xq, xs, vals, meta, ws)
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.sparse24_gemm(xq, xs, vals, meta, ws, rows=rows),
                      "split K, long ranges, mixed forms")
