"""Seeded synthetic inputs for the FP8 linear-layer workloads.

Shared by the tests, the benchmark and the smoke check, and by both sides of
every parity comparison (the HIP library and the CPU oracle).  It holds the
workload shapes and the random draws only: no quantization, pruning or GEMM
arithmetic lives here.

Recipe (all tensors are drawn on the host in fp32 or fp64 with torch's CPU
generator and cast once to bf16 with round-to-nearest-even):

* activations X [M,K] ~ N(0,1), seed 0; for the Llama-3-8B shapes, 1 % of the K
  channels (``round(0.01 K)`` of them, picked by ``randperm(K)`` with seed 3)
  are multiplied by 20 before the cast (outlier channels);
* weights W [N,K] ~ N(0, 0.02), seed 1 (N(0, 0.01) for the DeepSeek-V3 FFN);
* calibration batch for the activation-aware 2:4 score: 512 tokens ~ N(0,1),
  seed 2, no outliers; its column norms are c[k] = fp32(sqrt(sum_t x[t,k]^2))
  with the sum in fp64 over the bf16 values in token order;
* DeepSeek-V3 activations: Student-t with 3 degrees of freedom, drawn as
  z0 / sqrt((z1^2 + z2^2 + z3^2) / 3) from four fp64 standard normals of the
  seed-0 generator, 512 rows at a time.

Shapes are (K, N) of nn.Linear-style weights W [N,K] (K contiguous).
"""
from __future__ import annotations

import numpy as np
import torch

SEED_X, SEED_W, SEED_CAL, SEED_OUTLIER = 0, 1, 2, 3

# Llama-3-8B linears, (name, K, N)
LLAMA3_8B = [("qkv", 4096, 6144), ("o_proj", 4096, 4096), ("gate_up", 4096, 28672), ("down", 14336, 4096)]
# DeepSeek-V3 dense FFN linears, (name, K, N)
DSV3_FFN = [("ffn_up", 7168, 18432), ("ffn_down", 18432, 7168)]

# DeepSeek-V3 routed-expert linears, (name, K, N): the gate and up projections of
# an expert stacked (7168 -> 2 x 2048) and its down projection (2048 -> 7168)
DSV3_EXPERTS = [("expert_gate_up", 7168, 4096), ("expert_down", 2048, 7168)]

DECODE_M = (1, 8, 32, 64)
PREFILL_M = 4096
SPARSE_M = (16, 4096)
DSV3_M = 8192

# The five workloads: the single small linear, Llama-3-8B decode, prefill and 2:4, DeepSeek-V3 FFN.
WORKLOADS = {
    "single_linear_16x512x512": dict(shapes=[("linear", 512, 512)], M=(16,), dist="normal", outliers=False,
                                     w_std=0.02, sparse=False),
    "llama3_8b_decode_dense": dict(shapes=LLAMA3_8B, M=DECODE_M, dist="normal", outliers=True, w_std=0.02,
                                   sparse=False),
    "llama3_8b_prefill_dense": dict(shapes=LLAMA3_8B, M=(PREFILL_M,), dist="normal", outliers=True,
                                    w_std=0.02, sparse=False),
    "llama3_8b_sparse24": dict(shapes=LLAMA3_8B, M=SPARSE_M, dist="normal", outliers=True, w_std=0.02,
                               sparse=True),
    "dsv3_ffn_dense": dict(shapes=DSV3_FFN, M=(DSV3_M,), dist="student_t3", outliers=False, w_std=0.01,
                           sparse=False),
}


def to_bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Round a float tensor to bf16 (RNE) and return the raw uint16 bit patterns."""
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed)


def outlier_channels(K: int) -> np.ndarray:
    """The 1 % of channels scaled by 20 in the Llama activations."""
    n = int(round(0.01 * K))
    return torch.randperm(K, generator=_gen(SEED_OUTLIER))[:n].numpy()


def activations(M: int, K: int, dist: str = "normal", outliers: bool = True, seed: int = SEED_X) -> np.ndarray:
    """X [M,K] as bf16 bits."""
    if dist == "normal":
        x = torch.randn((M, K), generator=_gen(seed), dtype=torch.float32)
        if outliers and K > 0:
            x[:, torch.from_numpy(outlier_channels(K))] *= 20.0
        return to_bf16_bits(x)
    if dist == "student_t3":
        g = _gen(seed)
        out = np.empty((M, K), np.uint16)
        for r0 in range(0, M, 512):
            r1 = min(M, r0 + 512)
            z = torch.randn((4, r1 - r0, K), generator=g, dtype=torch.float64)
            t = z[0] / torch.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0)
            out[r0:r1] = to_bf16_bits(t.to(torch.float32))
        return out
    raise ValueError(dist)


def weights(N: int, K: int, std: float = 0.02, seed: int = SEED_W) -> np.ndarray:
    """W [N,K] as bf16 bits."""
    w = torch.randn((N, K), generator=_gen(seed), dtype=torch.float32) * std
    return to_bf16_bits(w)


def calibration_batch(K: int, T: int = 512, seed: int = SEED_CAL) -> np.ndarray:
    """Calibration activations [T,K] as bf16 bits (no outlier channels)."""
    return to_bf16_bits(torch.randn((T, K), generator=_gen(seed), dtype=torch.float32))


def column_norms(xcal_bf16: np.ndarray) -> np.ndarray:
    """c[k] = fp32(sqrt(sum_t x[t,k]^2)), the sum in fp64 in token order."""
    x = bf16_bits_to_f32(xcal_bf16).astype(np.float64)
    acc = np.zeros(x.shape[1], np.float64)
    for t in range(x.shape[0]):
        acc += x[t] * x[t]
    return np.sqrt(acc).astype(np.float32)


def sample_rows(M: int, count: int = 256, seed: int = 5) -> np.ndarray:
    """Sorted seeded sample of row indices used for row-sampled oracle checks."""
    if M <= count:
        return np.arange(M, dtype=np.int64)
    idx = torch.randperm(M, generator=_gen(seed))[:count].numpy().astype(np.int64)
    return np.sort(idx)


def routed_offsets(M: int, G: int, seed: int) -> np.ndarray:
    """Seeded uneven token counts per expert (gamma-distributed, about one expert in
    eight empty), as G + 1 int32 row offsets of the contiguous grouped layout summing to M."""
    rng = np.random.default_rng(seed)
    w = rng.gamma(0.6, size=G)
    w[rng.choice(G, max(1, G // 8), replace=False)] = 0.0
    counts = np.floor(w / w.sum() * M).astype(np.int64)
    counts[np.argmax(counts)] += M - counts.sum()
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
