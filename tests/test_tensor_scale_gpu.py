"""Parity of the one-scale-per-tensor quantizers (dynamic per-tensor and static)
through the C ABI with the CPU oracle: codes and scales bit-exact; the block-
scaled GEMM fed their output within the stated tolerance of the oracle GEMM."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from test_linear_gpu import edge_activations
from test_parity_gpu import assert_gemm_close, bf16_dev, dev, host, sample_tile_rows

pytestmark = pytest.mark.gpu


def every_bf16(width: int = 256) -> np.ndarray:
    """Every finite bf16 value once, padded to whole rows."""
    bits = np.arange(65536, dtype=np.uint32)
    finite = bits[np.isfinite((bits << 16).view(np.float32))].astype(np.uint16)
    return np.concatenate([finite, finite[:(-finite.size) % width]]).reshape(-1, width)


def check_tensor(gpu_lib, x):
    q, s = gpu_lib.fp8_quant_act_tensor(bf16_dev(x))
    rq, rs = oracle.quant_act_tensor(x)
    assert np.array_equal(host(s), rs), (host(s).ravel()[:4], rs.ravel()[:4])
    assert np.array_equal(host(q), rq)


@pytest.mark.parametrize("M,K,dist", [(1, 4096, "normal"), (16, 512, "normal"), (37, 4096, "normal"),
                                      (300, 640, "normal"), (4096, 14336, "normal"), (1024, 18432, "student_t3")])
def test_quant_act_tensor_bit_exact(gpu_lib, M, K, dist):
    check_tensor(gpu_lib, si.activations(M, K, dist=dist, outliers=(dist == "normal")))


def test_quant_act_tensor_edge_tensors(gpu_lib):
    check_tensor(gpu_lib, edge_activations())
    check_tensor(gpu_lib, every_bf16())
    check_tensor(gpu_lib, np.zeros((3, 384), np.uint16))                     # amax 0: s = 0, zero codes
    check_tensor(gpu_lib, np.full((2, 128), 0x8000, np.uint16))              # -0.0 everywhere
    x = np.zeros((5, 256), np.uint16)
    x[4, 255] = 0x0001                                                       # one bf16 subnormal
    check_tensor(gpu_lib, x)


def test_quant_act_tensor_reuses_a_dirty_scale_array(gpu_lib):
    """The scale array doubles as the partial-max buffer: a stale or garbage
    array, and a second call with a smaller tensor in the same buffers, give
    the same result as fresh buffers."""
    a = si.activations(64, 2048, dist="student_t3", outliers=False)
    b = si.activations(8, 1024)
    q = torch.empty((64 * 2048,), dtype=torch.uint8, device="cuda")
    s = torch.full((64 * 16,), float("nan"), dtype=torch.float32, device="cuda")
    for x in (a, b):
        M, K = x.shape
        qv, sv = q[:M * K].view(M, K), s[:M * K // 128].view(M, K // 128)
        gpu_lib.fp8_quant_act_tensor(bf16_dev(x), q=qv, s=sv)
        rq, rs = oracle.quant_act_tensor(x)
        assert np.array_equal(host(sv), rs) and np.array_equal(host(qv), rq)


@pytest.mark.parametrize("factor", [1.0, 0.25, 3.0, 2.0 ** -120, 2.0 ** 100])
def test_quant_act_static_bit_exact(gpu_lib, factor):
    """Static scales around the tensor's own amax / 448: equal, smaller (values
    saturate at +-448), larger, subnormal and huge."""
    x = si.activations(37, 4096)
    _, rs = oracle.quant_act_tensor(x)
    scale = float(np.float32(rs.flat[0] * np.float32(factor)))
    assert scale > 0.0
    q, s = gpu_lib.fp8_quant_act_static(bf16_dev(x), torch.tensor([scale], dtype=torch.float32, device="cuda"))
    rq, rs2 = oracle.quant_act_static(x, scale)
    assert np.array_equal(host(s), rs2) and np.all(rs2 == np.float32(scale))
    assert np.array_equal(host(q), rq)


def test_quant_act_static_edge_tensors(gpu_lib):
    for x, scale in ((edge_activations(), 0.5), (every_bf16(), 1.0), (every_bf16(), 2.0 ** -130),
                     (every_bf16(), 2.0 ** 120)):
        q, s = gpu_lib.fp8_quant_act_static(bf16_dev(x), torch.tensor([scale], dtype=torch.float32, device="cuda"))
        rq, rs = oracle.quant_act_static(x, scale)
        assert np.array_equal(host(s), rs) and np.array_equal(host(q), rq), scale


@pytest.mark.parametrize("N,K,std", [(128, 128, 0.02), (512, 512, 0.02), (384, 640, 0.02), (28672, 4096, 0.02),
                                     (7168, 18432, 0.01)])
def test_quant_weight_tensor_bit_exact(gpu_lib, N, K, std):
    w = si.weights(N, K, std=std)
    q, s = gpu_lib.fp8_quant_weight_tensor(bf16_dev(w))
    rq, rs = oracle.quant_weight_tensor(w)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)


@pytest.mark.parametrize("M", [1, 64, 4096])
def test_block_gemm_on_per_tensor_codes(gpu_lib, M):
    """The block-scaled GEMM takes per-tensor codes and broadcast scales as they
    come out of the quantizers."""
    name, K, N = si.LLAMA3_8B[0]
    x, w = si.activations(M, K), si.weights(N, K)
    xq, xs = gpu_lib.fp8_quant_act_tensor(bf16_dev(x))
    wq, ws = gpu_lib.fp8_quant_weight_tensor(bf16_dev(w))
    y = gpu_lib.fp8_block_gemm(xq, xs, wq, ws)
    rxq, rxs = oracle.quant_act_tensor(x)
    rwq, rws = oracle.quant_weight_tensor(w)
    rows = sample_tile_rows(M, 10) if M > 8 else np.arange(M)
    assert_gemm_close(y[torch.from_numpy(rows).to("cuda")], oracle.gemm(rxq, rxs, rwq, rws, rows=rows),
                      f"{name} M={M}")
