"""Property tests of the HIP kernels over random shapes (hypothesis, on the GPU).

Shapes are drawn with K and N multiples of 128 and any M (ragged token tails
included); values from normal, heavy-tailed and wide-exponent distributions.
Every draw is checked against the oracle (bit-exact for codes, scales, 2:4
values and index words; the GEMM tolerance for outputs), and the kernels must
keep the invariances the definitions give:

* activation quantization invariant under x -> 2^j x (codes equal, scales 2^j);
* 2:4 pruning equivariant under a permutation of the four values of each group
  (on groups with a unique kept pair);
* the GEMM output row of a token whose scales are multiplied by 2^j is 2^j
  times the original row, bit for bit (fp32 accumulation of exactly scaled
  terms, then bf16 rounding of an exactly scaled sum).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import synth_inputs as si
from test_parity_gpu import assert_gemm_close, bf16_dev, dev, host

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=25, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large,
                                           HealthCheck.function_scoped_fixture])


def _bf16(a: np.ndarray) -> np.ndarray:
    return si.to_bf16_bits(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)))


def _values(rng, shape, dist):
    if dist == "normal":
        return rng.standard_normal(shape)
    if dist == "t3":
        z = rng.standard_normal((4,) + shape)
        return z[0] / np.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3)
    mant = rng.uniform(1.0, 2.0, shape) * rng.choice([-1.0, 1.0], shape)   # wide exponents
    return mant * 2.0 ** rng.integers(-60, 60, shape)


DISTS = st.sampled_from(["normal", "t3", "wide"])


def _say(*args):
    print(*args, flush=True)


@SETTINGS
@given(M=st.integers(1, 300), kb=st.integers(1, 24), dist=DISTS, j=st.integers(-30, 30),
       seed=st.integers(0, 2 ** 31))
def test_quant_act_random_shapes(gpu_lib, M, kb, dist, j, seed):
    K = 128 * kb
    _say(f"fp8_quant_act M={M} K={K} {dist} j={j} seed={seed}")
    rng = np.random.default_rng(seed)
    x = _bf16(_values(rng, (M, K), dist) if dist != "wide" else _values(rng, (M, K), dist) * 2.0 ** -40)
    q, s = gpu_lib.fp8_quant_act(bf16_dev(x))
    qr, sr = oracle.quant_act(x)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    if dist != "wide":  # keep 2^j x inside the normal bf16 range
        xj = _bf16(si.bf16_bits_to_f32(x) * np.float32(2.0 ** j))
        qj, sj = gpu_lib.fp8_quant_act(bf16_dev(xj))
        assert np.array_equal(host(qj), qr)
        assert np.array_equal(host(sj), (sr.astype(np.float64) * 2.0 ** j).astype(np.float32))


@SETTINGS
@given(nb=st.integers(1, 4), kb=st.integers(1, 12), aware=st.booleans(), seed=st.integers(0, 2 ** 31))
def test_prune24_random_shapes_and_permutations(gpu_lib, nb, kb, aware, seed):
    N, K = 128 * nb, 128 * kb
    _say(f"prune24_compress N={N} K={K} aware={aware} seed={seed}")
    rng = np.random.default_rng(seed)
    w = _bf16(rng.standard_normal((N, K)) * 0.02)
    c = rng.uniform(0.1, 3.0, K).astype(np.float32) if aware else None
    v, m, s = gpu_lib.prune24_compress(bf16_dev(w), None if c is None else dev(c))
    vr, mr, sr = oracle.prune24_compress(w, c)
    assert np.array_equal(host(v), vr) and np.array_equal(host(m), mr)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    # permute the four values of every group; the kept values follow them
    perm = np.stack([rng.permutation(4) for _ in range(K // 4)])
    idx = (np.arange(K // 4)[:, None] * 4 + perm).reshape(-1)
    wp, cp = np.ascontiguousarray(w[:, idx]), None if c is None else np.ascontiguousarray(c[idx])
    vp, mp, sp = gpu_lib.prune24_compress(bf16_dev(wp), None if cp is None else dev(cp))
    keep = _kept(mr, N, K)
    keep_p = _kept(host(mp), N, K)
    score = np.abs(si.bf16_bits_to_f32(w).astype(np.float64)) * (1.0 if c is None else c.astype(np.float64))
    srt = np.sort(score.reshape(N, K // 4, 4), axis=-1)
    unique = srt[..., 2] != srt[..., 1]
    # position p of permuted group g holds original position perm[g, p]
    back = np.take_along_axis(keep, np.broadcast_to(perm, keep.shape), axis=-1)
    assert np.array_equal(keep_p[unique], back[unique])
    if unique.all():  # the same kept values, so the same block scales
        assert np.array_equal(host(sp).view(np.uint32), sr.view(np.uint32))


def _kept(meta: np.ndarray, N: int, K: int) -> np.ndarray:
    """[N, K/4, 4] kept positions from the 2-bit indices (nibble i0 | i1 << 2 per group)."""
    nib = np.stack([meta & 15, meta >> 4], axis=-1).reshape(N, K // 4)
    keep = np.zeros((N, K // 4, 4), bool)
    for pos in range(4):
        keep[..., pos] = ((nib & 3) == pos) | ((nib >> 2) == pos)
    return keep


@SETTINGS
@given(M=st.integers(1, 700), nb=st.integers(1, 12), kb=st.integers(1, 40), sparse=st.booleans(),
       dist=st.sampled_from(["normal", "t3"]), seed=st.integers(0, 2 ** 31))
def test_gemm_random_shapes(gpu_lib, M, nb, kb, sparse, dist, seed):
    N, K = 128 * nb, 128 * kb
    _say(f"{'fp8_sparse24_gemm' if sparse else 'fp8_block_gemm'} M={M} N={N} K={K} {dist} seed={seed}")
    rng = np.random.default_rng(seed)
    xq, xs = oracle.quant_act(_bf16(_values(rng, (M, K), dist)))
    w = _bf16(rng.standard_normal((N, K)) * 0.02)
    if sparse:
        vals, meta, ws = oracle.prune24_compress(w)
        y = gpu_lib.fp8_sparse24_gemm(dev(xq), dev(xs), dev(vals), dev(meta), dev(ws))
        ref = oracle.sparse24_gemm(xq, xs, vals, meta, ws)
    else:
        wq, ws = oracle.quant_wblock(w)
        y = gpu_lib.fp8_block_gemm(dev(xq), dev(xs), dev(wq), dev(ws))
        ref = oracle.gemm(xq, xs, wq, ws)
    assert_gemm_close(y, ref, f"M={M} N={N} K={K} sparse={sparse}")


@SETTINGS
@given(M=st.integers(1, 400), nb=st.integers(1, 6), kb=st.integers(1, 40), j=st.integers(-8, 8),
       seed=st.integers(0, 2 ** 31))
def test_gemm_row_scales_by_power_of_two(gpu_lib, M, nb, kb, j, seed):
    N, K = 128 * nb, 128 * kb
    _say(f"fp8_block_gemm scaled row M={M} N={N} K={K} j={j} seed={seed}")
    rng = np.random.default_rng(seed)
    xq, xs = oracle.quant_act(_bf16(rng.standard_normal((M, K))))
    wq, ws = oracle.quant_wblock(_bf16(rng.standard_normal((N, K)) * 0.02))
    m = int(rng.integers(M))
    xs2 = xs.copy()
    xs2[m] = (xs2[m].astype(np.float64) * 2.0 ** j).astype(np.float32)
    y = gpu_lib.fp8_block_gemm(dev(xq), dev(xs), dev(wq), dev(ws)).float().cpu().numpy()
    y2 = gpu_lib.fp8_block_gemm(dev(xq), dev(xs2), dev(wq), dev(ws)).float().cpu().numpy()
    assert np.array_equal(y2[m], (y[m].astype(np.float64) * 2.0 ** j).astype(np.float32))
    others = np.arange(M) != m
    assert np.array_equal(y2[others], y[others])
