"""Parity of the HIP library (through the C ABI) with the CPU oracle.

Quantization codes, scales, 2:4 values and index words must be bit-exact.
GEMM outputs must satisfy, against the oracle's fp64 result Y_ref:
    ||Y - Y_ref||_F / ||Y_ref||_F <= 5e-3   and
    |Y - Y_ref| <= 2^-7 |Y_ref| + 1e-3 max|Y_ref|   element-wise.
The GEMMs are fed the oracle's codes and scales, so GEMM and quantizer tests
are independent.  Large workloads are checked on seeded samples of rows (or
128-row weight block rows) that the oracle computes one by one.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

pytestmark = pytest.mark.gpu

DEV = "cuda"
REL_FRO = 5e-3
REL_ELEM = 2.0 ** -7
ABS_FRAC = 1e-3


# ------------------------------------------------------------------ helpers --

def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_gemm_close(y_dev: torch.Tensor, ref: np.ndarray, what: str = ""):
    y = y_dev.float().cpu().numpy().astype(np.float64)
    assert y.shape == ref.shape, what
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(y - ref) / max(nref, 1e-300)
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e}"
    bound = REL_ELEM * np.abs(ref) + ABS_FRAC * np.abs(ref).max()
    bad = np.abs(y - ref) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements out of bound, first at {np.argwhere(bad)[0]}"


TILE_ROWS = 128  # the smallest token tile of the tile kernels (they run 256- and 128-token tiles)


def sample_tile_rows(M: int, count: int = 12, seed: int = 5) -> np.ndarray:
    """Rows that reach every 128-token tile: its first and last row and one seeded row
    inside it, plus the 16-row MFMA tile edges at the top and a seeded sample of
    `count` rows over the whole matrix.  Compared across all N columns, these rows
    put at least three rows of every output tile of every launch under the oracle
    (48+ rows at M = 4096 per 256-token tile, 96+ per 128-token tile)."""
    fixed = {0, M - 1, min(15, M - 1), min(16, M - 1), M // 2}
    rng = np.random.default_rng(seed)
    for t0 in range(0, M, TILE_ROWS):
        t1 = min(M, t0 + TILE_ROWS) - 1
        fixed |= {t0, t1, int(rng.integers(t0, t1 + 1))}
    rest = si.sample_rows(M, count, seed=seed)
    return np.array(sorted(fixed | set(rest.tolist())), dtype=np.int64)


def test_sample_rows_reach_every_tile():
    """Every 128- and 256-token tile of a full-size launch has rows under comparison."""
    for M in (4096, 8192, 1000, 65):
        rows = sample_tile_rows(M)
        for bm in (128, 256):
            assert set(range((M + bm - 1) // bm)) == set((rows // bm).tolist()), (M, bm)
        assert len(rows) >= 3 * (M // TILE_ROWS)


@functools.lru_cache(maxsize=None)
def llama_weight(K: int, N: int):
    w = si.weights(N, K)
    return w, oracle.quant_wblock(w)


@functools.lru_cache(maxsize=None)
def llama_sparse_weight(K: int, N: int, aware: bool):
    w, _ = llama_weight(K, N)
    c = si.column_norms(si.calibration_batch(K)) if aware else None
    return c, oracle.prune24_compress(w, c)


@functools.lru_cache(maxsize=2)
def dsv3_acts(K: int):
    return si.activations(si.DSV3_M, K, dist="student_t3", outliers=False)


@functools.lru_cache(maxsize=None)
def llama_acts(M: int, K: int):
    x = si.activations(M, K)
    return x, oracle.quant_act(x)


# ------------------------------------------------- activation quantization --

# Each 16-lane set of the kernel takes two groups 16 apart (32 per workgroup):
# 300 x 640 (1500 groups) and 3 x 4224 (99) end in a partly filled workgroup,
# 5 x 384 (15) has no second group at all.
@pytest.mark.parametrize("M,K", [(16, 512), (1, 4096), (8, 4096), (37, 4096), (64, 14336), (300, 640), (3, 4224),
                                 (5, 384)])
def test_quant_act_bit_exact(gpu_lib, M, K):
    x = si.activations(M, K, outliers=K >= 4096)
    q, s = gpu_lib.fp8_quant_act(bf16_dev(x))
    qr, sr = oracle.quant_act(x)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))


def test_quant_act_every_bf16_value(gpu_lib):
    """All finite bf16 patterns, in sorted and in shuffled groups of 128."""
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    finite = bits[np.isfinite(vals)].astype(np.uint16)
    pad = (-finite.size) % 128
    ordered = np.concatenate([finite, finite[:pad]])
    rng = np.random.default_rng(1)
    x = np.concatenate([ordered, rng.permutation(ordered), rng.permutation(ordered)]).reshape(-1, 256)
    q, s = gpu_lib.fp8_quant_act(bf16_dev(x))
    qr, sr = oracle.quant_act(x)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(host(q), qr)


def test_quant_act_edge_groups(gpu_lib):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 1024)).astype(np.float32)
    x[0, :128] = 0.0                                       # all-zero group: s = 0, +0 codes
    x[0, 128:256] = -0.0                                   # all negative zeros: 0x80 codes
    x[1, :128] = rng.standard_normal(128) * 1e-39          # bf16 subnormals, fp32 subnormal scale
    x[1, 128:256] = rng.standard_normal(128) * 1e38        # near the top of the range
    x[2, :128] = np.float32(2.0 ** -133)                   # smallest bf16 subnormal everywhere
    x[3, :] = np.tile(np.linspace(-448, 448, 128, dtype=np.float32), 8)
    x[4, :] = np.tile(np.float32(432.0) * np.arange(1, 129, dtype=np.float32) / 128, 8)  # e4m3 midpoints
    z = rng.standard_normal((4, 3, 1024))
    x[5:8] = (z[0] / np.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3)).astype(np.float32)  # heavy tails
    xb = si.to_bf16_bits(torch.from_numpy(x))
    q, s = gpu_lib.fp8_quant_act(bf16_dev(xb))
    qr, sr = oracle.quant_act(xb)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(host(q), qr)
    assert sr[0, 0] == 0.0 and np.all(qr[0, :128] == 0x00) and np.all(qr[0, 128:256] == 0x80)
    assert 0.0 < sr[2, 0] < np.finfo(np.float32).tiny


@pytest.mark.parametrize("M,K,dist", [(4096, 14336, "normal"), (8192, 18432, "student_t3")])
def test_quant_act_full_size_sampled(gpu_lib, M, K, dist):
    x = si.activations(M, K) if dist == "normal" else dsv3_acts(K)
    q, s = gpu_lib.fp8_quant_act(bf16_dev(x))
    rows = sample_tile_rows(M, 32)
    qr, sr = oracle.quant_act(x[rows])
    qh, sh = host(q), host(s)
    assert np.array_equal(qh[rows], qr)
    assert np.array_equal(sh[rows].view(np.uint32), sr.view(np.uint32))


def test_quant_act_empty(gpu_lib):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    q, s = gpu_lib.fp8_quant_act(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)


# ---------------------------------------------------- weight quantization ---

@pytest.mark.parametrize("N,K", [(512, 512), (128, 128), (4096, 4096), (384, 640)])
def test_quant_wblock_bit_exact(gpu_lib, N, K):
    w = si.weights(N, K)
    q, s = gpu_lib.fp8_quant_weight_block(bf16_dev(w))
    qr, sr = oracle.quant_wblock(w)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(host(q), qr)


def test_quant_wblock_edge_blocks(gpu_lib):
    w = si.weights(256, 384).copy()
    w[:128, :128] = 0                                    # zero block
    w[128:, 128:256] = si.to_bf16_bits(torch.full((128, 128), 1e-39))  # subnormal block
    w[0:128, 256:384] = si.to_bf16_bits(torch.linspace(-500, 500, 128 * 128).reshape(128, 128))
    q, s = gpu_lib.fp8_quant_weight_block(bf16_dev(w))
    qr, sr = oracle.quant_wblock(w)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(host(q), qr)


@pytest.mark.parametrize("K,N,std", [(4096, 28672, 0.02), (18432, 7168, 0.01), (7168, 18432, 0.01)])
def test_quant_wblock_full_size_sampled(gpu_lib, K, N, std):
    w = si.weights(N, K, std=std)
    q, s = gpu_lib.fp8_quant_weight_block(bf16_dev(w))
    qh, sh = host(q), host(s)
    for nb in (0, N // 256, N // 128 - 1):
        rows = slice(nb * 128, (nb + 1) * 128)
        qr, sr = oracle.quant_wblock(w[rows])
        assert np.array_equal(qh[rows], qr)
        assert np.array_equal(sh[nb:nb + 1].view(np.uint32), sr.view(np.uint32))


# ------------------------------------------------------------------- 2:4 ----

@pytest.mark.parametrize("aware", [False, True])
@pytest.mark.parametrize("N,K", [(512, 512), (128, 256), (4096, 4096)])
def test_prune24_bit_exact(gpu_lib, N, K, aware):
    w = si.weights(N, K)
    c = si.column_norms(si.calibration_batch(K)) if aware else None
    vals, meta, s = gpu_lib.prune24_compress(bf16_dev(w), None if c is None else dev(c))
    vr, mr, sr = oracle.prune24_compress(w, c)
    assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(host(meta), mr)
    assert np.array_equal(host(vals), vr)


def test_prune24_ties_and_zeros(gpu_lib):
    rng = np.random.default_rng(4)
    w = rng.integers(-2, 3, (256, 512)).astype(np.float32)   # many equal magnitudes
    w[:128, :128] = 0.0                                        # all-zero block
    c = rng.integers(0, 3, 512).astype(np.float32)             # zero and equal column norms
    wb = si.to_bf16_bits(torch.from_numpy(w))
    for cn in (None, c):
        vals, meta, s = gpu_lib.prune24_compress(bf16_dev(wb), None if cn is None else dev(cn))
        vr, mr, sr = oracle.prune24_compress(wb, cn)
        assert np.array_equal(host(s).view(np.uint32), sr.view(np.uint32))
        assert np.array_equal(host(meta), mr)
        assert np.array_equal(host(vals), vr)


@pytest.mark.parametrize("K,N", [(4096, 28672), (14336, 4096)])
def test_prune24_full_size_sampled(gpu_lib, K, N):
    w = si.weights(N, K)
    c = si.column_norms(si.calibration_batch(K))
    vals, meta, s = gpu_lib.prune24_compress(bf16_dev(w), dev(c))
    vh, mh, sh = host(vals), host(meta), host(s)
    for nb in (0, N // 256, N // 128 - 1):
        rows = slice(nb * 128, (nb + 1) * 128)
        vr, mr, sr = oracle.prune24_compress(w[rows], c)
        assert np.array_equal(vh[rows], vr) and np.array_equal(mh[rows], mr)
        assert np.array_equal(sh[nb:nb + 1].view(np.uint32), sr.view(np.uint32))


# ------------------------------------------------------------ dense GEMM ----

def run_dense(gpu_lib, xq, xs, wq, ws):
    return gpu_lib.fp8_block_gemm(dev(xq), dev(xs), dev(wq), dev(ws))


def test_dense_gemm_single_linear(gpu_lib):
    x = si.activations(16, 512, outliers=False)
    w = si.weights(512, 512)
    xq, xs = oracle.quant_act(x)
    wq, ws = oracle.quant_wblock(w)
    assert_gemm_close(run_dense(gpu_lib, xq, xs, wq, ws), oracle.gemm(xq, xs, wq, ws), "16x512x512")


@pytest.mark.parametrize("M", [1, 8, 32, 64])
@pytest.mark.parametrize("name,K,N", si.LLAMA3_8B)
def test_dense_gemm_decode(gpu_lib, name, K, N, M):
    _, (xq, xs) = llama_acts(M, K)
    _, (wq, ws) = llama_weight(K, N)
    y = run_dense(gpu_lib, xq, xs, wq, ws)
    rows = sample_tile_rows(M, 8) if M > 8 else np.arange(M)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], oracle.gemm(xq, xs, wq, ws, rows=rows), f"{name} M={M}")


@pytest.mark.parametrize("name,K,N", si.LLAMA3_8B)
def test_dense_gemm_prefill_sampled(gpu_lib, name, K, N):
    _, (xq, xs) = llama_acts(si.PREFILL_M, K)
    _, (wq, ws) = llama_weight(K, N)
    y = run_dense(gpu_lib, xq, xs, wq, ws)
    rows = sample_tile_rows(si.PREFILL_M, 12)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], oracle.gemm(xq, xs, wq, ws, rows=rows), name)


@pytest.mark.parametrize("name,K,N", si.DSV3_FFN)
def test_dense_gemm_dsv3_sampled(gpu_lib, name, K, N):
    x = dsv3_acts(K)
    w = si.weights(N, K, std=0.01)
    xq, xs = oracle.quant_act(x)
    wq, ws = oracle.quant_wblock(w)
    y = run_dense(gpu_lib, xq, xs, wq, ws)
    rows = sample_tile_rows(si.DSV3_M, 6)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], oracle.gemm(xq, xs, wq, ws, rows=rows), name)


@pytest.mark.parametrize("M,N,K", [(65, 384, 640), (100, 128, 128), (257, 640, 256), (300, 256, 1152),
                                   (48, 384, 128), (3, 128, 256), (512, 512, 384)])
def test_dense_gemm_ragged(gpu_lib, M, N, K):
    x = si.activations(M, K, outliers=False)
    w = si.weights(N, K)
    xq, xs = oracle.quant_act(x)
    wq, ws = oracle.quant_wblock(w)
    assert_gemm_close(run_dense(gpu_lib, xq, xs, wq, ws), oracle.gemm(xq, xs, wq, ws), f"{M}x{N}x{K}")


def test_dense_gemm_deterministic(gpu_lib):
    _, (xq, xs) = llama_acts(si.PREFILL_M, 4096)
    _, (wq, ws) = llama_weight(4096, 4096)
    a = run_dense(gpu_lib, xq, xs, wq, ws)
    b = run_dense(gpu_lib, xq, xs, wq, ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ----------------------------------------------------------- sparse GEMM ----

def run_sparse(gpu_lib, xq, xs, vals, meta, ws):
    return gpu_lib.fp8_sparse24_gemm(dev(xq), dev(xs), dev(vals), dev(meta), dev(ws))


@pytest.mark.parametrize("M", [1, 2, 4, 16, 4096])
@pytest.mark.parametrize("name,K,N", si.LLAMA3_8B)
def test_sparse_gemm_llama(gpu_lib, name, K, N, M):
    _, (xq, xs) = llama_acts(M, K)
    _, (vals, meta, ws) = llama_sparse_weight(K, N, True)
    y = run_sparse(gpu_lib, xq, xs, vals, meta, ws)
    rows = sample_tile_rows(M, 12) if M > 16 else np.arange(M)
    ref = oracle.sparse24_gemm(xq, xs, vals, meta, ws, rows=rows)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], ref, f"{name} M={M}")


# 1-4 tokens with 8-15 four-block units per row (K of 4096-8064): whole-row
# tiles over 4 waves (N >= 16384), 32-row bands over 8 waves (6144 <= N <
# 16384) or 16-row bands over 8 waves.
@pytest.mark.parametrize("M,N,K", [(3, 6400, 5120), (1, 16384, 6144), (2, 640, 7680), (4, 384, 4608)])
def test_sparse_decode_few_tokens(gpu_lib, M, N, K):
    x = si.activations(M, K, outliers=True, seed=M + N % 101)
    xq, xs = oracle.quant_act(x)
    vals, meta, ws = oracle.prune24_compress(si.weights(N, K, seed=3 + K % 7))
    y = run_sparse(gpu_lib, xq, xs, vals, meta, ws)
    assert_gemm_close(y, oracle.sparse24_gemm(xq, xs, vals, meta, ws), f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(16, 512, 512), (1, 256, 384), (40, 384, 256), (65, 384, 640),
                                   (300, 256, 1152), (512, 512, 384)])
def test_sparse_gemm_ragged(gpu_lib, M, N, K):
    x = si.activations(M, K, outliers=False)
    w = si.weights(N, K)
    xq, xs = oracle.quant_act(x)
    vals, meta, ws = oracle.prune24_compress(w)
    y = run_sparse(gpu_lib, xq, xs, vals, meta, ws)
    assert_gemm_close(y, oracle.sparse24_gemm(xq, xs, vals, meta, ws), f"{M}x{N}x{K}")


def test_sparse_matches_dense_on_decompressed(gpu_lib):
    """Both GPU GEMMs on the same pruned weight agree closely (and with the oracle)."""
    _, (xq, xs) = llama_acts(64, 4096)
    _, (vals, meta, ws) = llama_sparse_weight(4096, 4096, True)
    dense_q = oracle.decompress24(vals, meta)
    ys = run_sparse(gpu_lib, xq, xs, vals, meta, ws)
    yd = run_dense(gpu_lib, xq, xs, dense_q, ws)
    ref = oracle.gemm(xq, xs, dense_q, ws)
    assert_gemm_close(ys, ref, "sparse")
    assert_gemm_close(yd, ref, "dense on decompressed")


# --------------------------------------------------------- whole path ------

def test_end_to_end_matches_oracle(gpu_lib):
    """GPU quantizers feeding GPU GEMMs, against the oracle doing every step."""
    M, K, N = 32, 4096, 6144
    x = si.activations(M, K)
    w = si.weights(N, K)
    c = si.column_norms(si.calibration_batch(K))
    xq, xs = gpu_lib.fp8_quant_act(bf16_dev(x))
    wq, ws = gpu_lib.fp8_quant_weight_block(bf16_dev(w))
    y = gpu_lib.fp8_block_gemm(xq, xs, wq, ws)
    v, m, s2 = gpu_lib.prune24_compress(bf16_dev(w), dev(c))
    y2 = gpu_lib.fp8_sparse24_gemm(xq, xs, v, m, s2)
    rxq, rxs = oracle.quant_act(x)
    rwq, rws = oracle.quant_wblock(w)
    rv, rm, rs2 = oracle.prune24_compress(w, c)
    assert_gemm_close(y, oracle.gemm(rxq, rxs, rwq, rws), "dense path")
    assert_gemm_close(y2, oracle.sparse24_gemm(rxq, rxs, rv, rm, rs2), "sparse path")
