"""Property tests of the oracle over random shapes and values (hypothesis, CPU).

Each property follows from the definitions alone, so a dropped term, a wrong
index or a transposed operand in the oracle breaks it on some draw:

* quantization is invariant under scaling a group by 2^j (codes unchanged,
  scale times 2^j) while the scaled values stay normal bf16 numbers;
* negating a group flips the sign bit of every code and keeps the scale;
* permuting the four values of a 2:4 group with distinct scores permutes the
  kept positions the same way;
* the GEMM is linear in each token's and each weight block's scales: scaling
  one token's scales by 2^j scales exactly that output row by 2^j, and scaling
  one weight block row's scales by 2^j exactly those 128 output columns;
* the sparse GEMM on (values, indices) equals the dense GEMM on the
  decompressed weight, on any shape.
"""
from __future__ import annotations

import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import synth_inputs as si

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


def _bf16(a: np.ndarray) -> np.ndarray:
    return si.to_bf16_bits(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)))


def _normal_values(rng, shape, lo_exp=-30, hi_exp=30):
    """Values whose magnitudes stay well inside the normal bf16 range."""
    mant = rng.uniform(1.0, 2.0, shape) * rng.choice([-1.0, 1.0], shape)
    return (mant * 2.0 ** rng.integers(lo_exp, hi_exp, shape)).astype(np.float32)


@SETTINGS
@given(M=st.integers(1, 9), kb=st.integers(1, 6), j=st.integers(-40, 40), seed=st.integers(0, 2 ** 31))
def test_quant_act_power_of_two_invariance(M, kb, j, seed):
    rng = np.random.default_rng(seed)
    x = _bf16(_normal_values(rng, (M, 128 * kb)))
    xj = _bf16(si.bf16_bits_to_f32(x) * np.float32(2.0 ** j))
    q, s = oracle.quant_act(x)
    qj, sj = oracle.quant_act(xj)
    assert np.array_equal(qj, q)
    assert np.array_equal(sj, (s.astype(np.float64) * 2.0 ** j).astype(np.float32))


@SETTINGS
@given(M=st.integers(1, 9), kb=st.integers(1, 6), seed=st.integers(0, 2 ** 31))
def test_quant_act_negation(M, kb, seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((M, 128 * kb)) * 2.0 ** rng.integers(-20, 20))
    q, s = oracle.quant_act(x)
    qn, sn = oracle.quant_act(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, q ^ np.uint8(0x80))
    assert np.array_equal(sn, s)


@SETTINGS
@given(N=st.integers(1, 4), groups=st.integers(1, 64), aware=st.booleans(), seed=st.integers(0, 2 ** 31))
def test_prune_permutation_within_groups(N, groups, aware, seed):
    rng = np.random.default_rng(seed)
    K = 128 * ((4 * groups + 127) // 128)
    w = _bf16(rng.standard_normal((128 * N, K)))
    c = rng.uniform(0.5, 2.0, K).astype(np.float32) if aware else None
    keep = oracle.prune24_mask(w, c).reshape(128 * N, K // 4, 4)
    perm = np.stack([rng.permutation(4) for _ in range(K // 4)])     # one permutation per group position
    idx = (np.arange(K // 4)[:, None] * 4 + perm).reshape(-1)
    wp = np.ascontiguousarray(w[:, idx])
    cp = None if c is None else np.ascontiguousarray(c[idx])
    keep_p = oracle.prune24_mask(wp, cp).reshape(128 * N, K // 4, 4)
    score = np.abs(si.bf16_bits_to_f32(w).astype(np.float64)) * (1.0 if c is None else c.astype(np.float64))
    srt = np.sort(score.reshape(128 * N, K // 4, 4), axis=-1)
    tie_free = srt[..., 2] != srt[..., 1]                           # the kept pair is unique
    # position p of the permuted group holds original position perm[g, p]
    back = np.take_along_axis(keep, np.broadcast_to(perm, keep.shape), axis=-1)
    assert np.array_equal(keep_p[tie_free], back[tie_free])


@SETTINGS
@given(M=st.integers(1, 40), nb=st.integers(1, 3), kb=st.integers(1, 4), j=st.integers(-12, 12),
       seed=st.integers(0, 2 ** 31))
def test_gemm_linear_in_scales(M, nb, kb, j, seed):
    rng = np.random.default_rng(seed)
    N, K = 128 * nb, 128 * kb
    xq, xs = oracle.quant_act(_bf16(rng.standard_normal((M, K))))
    wq, ws = oracle.quant_wblock(_bf16(rng.standard_normal((N, K)) * 0.02))
    y = oracle.gemm(xq, xs, wq, ws)
    m, b = int(rng.integers(M)), int(rng.integers(nb))
    xs2 = xs.copy()
    xs2[m] = (xs2[m].astype(np.float64) * 2.0 ** j).astype(np.float32)
    y2 = oracle.gemm(xq, xs2, wq, ws)
    want = y.copy()
    want[m] *= 2.0 ** j
    assert np.array_equal(y2, want)
    ws2 = ws.copy()
    ws2[b] = (ws2[b].astype(np.float64) * 2.0 ** j).astype(np.float32)
    y3 = oracle.gemm(xq, xs, wq, ws2)
    want = y.copy()
    want[:, 128 * b:128 * (b + 1)] *= 2.0 ** j
    assert np.array_equal(y3, want)


@SETTINGS
@given(M=st.integers(1, 40), nb=st.integers(1, 3), kb=st.integers(1, 4), aware=st.booleans(),
       seed=st.integers(0, 2 ** 31))
def test_sparse_gemm_is_dense_gemm_on_decompressed(M, nb, kb, aware, seed):
    rng = np.random.default_rng(seed)
    N, K = 128 * nb, 128 * kb
    xq, xs = oracle.quant_act(_bf16(rng.standard_normal((M, K))))
    w = _bf16(rng.standard_normal((N, K)) * 0.02)
    c = rng.uniform(0.5, 2.0, K).astype(np.float32) if aware else None
    vals, meta, s = oracle.prune24_compress(w, c)
    assert np.array_equal(oracle.sparse24_gemm(xq, xs, vals, meta, s),
                          oracle.gemm(xq, xs, oracle.decompress24(vals, meta), s))
