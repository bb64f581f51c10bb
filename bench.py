"""Benchmark of the FP8 quantized linear layer on one MI355X.

One step = one pass of the whole hot path over one batch, for each of the four
Llama-3-8B linears (QKV 4096->6144, o_proj 4096->4096, gate/up 4096->28672,
down 14336->4096) at M = 4096 tokens:
    fp8_quant_act(X) -> fp8_quant_weight_block(W) -> fp8_block_gemm
    prune24_compress(W, ||x_k||) -> fp8_sparse24_gemm
Inputs are seeded synthetic tensors, resident in HBM before timing starts.

`value` is the step's algorithmic GEMM work divided by the step time: 2*M*N*K
for each dense GEMM plus M*N*K for each 2:4 GEMM (the pruned half of the
multiply-adds is never done), in TFLOP/s.  The JSON line also carries the
roofline of the dominant kernel (the dense gate/up GEMM), per-kernel times
taken with HIP events on the launch stream, the decode-M GEMMs (HBM GB/s, with
the weights rotated through enough copies to defeat the caches) and the CPU
oracle timed on a bounded sample of the same step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu]
       python bench.py --profile-case NAME   (one kernel workload, for rocprofv3 counter runs)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s & % MFMA peak (dense, 2:4); decode-M HBM GB/s"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
CALIB_BYTES = 256 << 20    # size of the traffic-calibration copy

# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc runs
# of this script (FETCH_SIZE, then WRITE_SIZE; profiles/
# fp8_block_gemm_gate_up_m4096_traffic.md has the commands and the readings),
# each scaled by the same counter's reading for the calibration copy.  It is
# reported only while the kernel's sources hash to the value it was taken on.
TRAFFIC = {"bytes_per_launch": 941550383,
           "sources_sha256": "5c0c4ff81905ea0189a8f2f7f770bb9c045ab63e5f8700378fc74547b550bda2"}
TRAFFIC_SOURCES = ("sparse_gemm_linears_amd/csrc/gemm_dense.hip", "sparse_gemm_linears_amd/csrc/gemm_common.hpp",
                   "sparse_gemm_linears_amd/csrc/device_common.hpp")


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    if TRAFFIC is None or TRAFFIC["sources_sha256"] != kernel_sources_sha256():
        return None
    return TRAFFIC["bytes_per_launch"]


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-decode", action="store_true", help="skip the decode-M and mid-M GEMM measurements")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-rows", type=int, default=1024, help="token rows in the CPU oracle sample")
    p.add_argument("--profile-case", choices=sorted(PROFILE_CASES), default=None,
                   help="run only one kernel workload (for rocprofv3 counter runs) and exit")
    return p.parse_args()


# Single-kernel workloads for counter collection under rocprofv3 --pmc: each runs
# the named call `reps` times (after one warm-up call) on the inputs of the
# benchmark, plus the 256 MiB calibration copy, and prints one JSON line.
#   (kind, shape name, tokens, reps); decode kinds rotate the weight through
#   >= 1 GiB of copies so that every call reads it from HBM.
PROFILE_CASES = {
    "dense_gate_up_m4096": ("dense", "gate_up", 4096, 5),
    "sparse_gate_up_m4096": ("sparse", "gate_up", 4096, 5),
    "dense_down_m4096": ("dense", "down", 4096, 5),
    "sparse_down_m4096": ("sparse", "down", 4096, 5),
    "ue8m0_gate_up_m4096": ("ue8m0", "gate_up", 4096, 5),
    "decode_dense_gate_up_m1": ("dense", "gate_up", 1, 20),
    "decode_dense_down_m1": ("dense", "down", 1, 20),
    "decode_dense_gate_up_m8": ("dense", "gate_up", 8, 20),
    "decode_dense_gate_up_m16": ("dense", "gate_up", 16, 20),
    "decode_dense_down_m16": ("dense", "down", 16, 20),
    "decode_sparse_gate_up_m8": ("sparse", "gate_up", 8, 20),
    "decode_sparse_gate_up_m16": ("sparse", "gate_up", 16, 20),
    "decode_sparse_down_m16": ("sparse", "down", 16, 20),
    "decode_dense_qkv_m1": ("dense", "qkv", 1, 20),
    "decode_dense_qkv_m16": ("dense", "qkv", 16, 20),
    "decode_dense_qkv_m64": ("dense", "qkv", 64, 20),
    "decode_sparse_qkv_m16": ("sparse", "qkv", 16, 20),
    "decode_sparse_qkv_m64": ("sparse", "qkv", 64, 20),
}


def profile_case(name):
    import numpy as np
    import torch

    import sparse_gemm_linears_amd as sgl
    import synth_inputs as si

    kind, shape, M, reps = PROFILE_CASES[name]
    sgl.load_library()
    dev = torch.device("cuda:0")
    _, K, N = next(s for s in si.LLAMA3_8B if s[0] == shape)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    calib_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    torch.empty_like(calib_src).copy_(calib_src)
    x = bf16(si.activations(M, K))
    w = bf16(si.weights(N, K))
    xq, xs = sgl.fp8_quant_act(x)
    copies = 1 if M > 64 else max(2, math.ceil((1 << 30) / (N * K)))
    if kind == "ue8m0":
        xq, xs = sgl.fp8_quant_act_ue8m0(x)
        wq, ws = sgl.fp8_quant_weight_block_ue8m0(w)
        ops = [(wq, ws)]
        f = lambda i: sgl.fp8_block_gemm_ue8m0(xq, xs, wq, ws, y)
    elif kind == "dense":
        wq, ws = sgl.fp8_quant_weight_block(w)
        ops = [(wq.clone(), ws.clone()) for _ in range(copies)] if copies > 1 else [(wq, ws)]
        f = lambda i: sgl.fp8_block_gemm(xq, xs, *ops[i % len(ops)], y)
    else:
        c = torch.from_numpy(si.column_norms(si.calibration_batch(K))).to(dev)
        v, m, s2 = sgl.prune24_compress(w, c)
        ops = [(v.clone(), m.clone(), s2.clone()) for _ in range(copies)] if copies > 1 else [(v, m, s2)]
        f = lambda i: sgl.fp8_sparse24_gemm(xq, xs, *ops[i % len(ops)], y)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    f(len(ops) - 1)
    torch.cuda.synchronize()
    for i in range(reps):
        f(i)
    torch.cuda.synchronize()
    print(json.dumps({"profile_case": name, "kind": kind, "shape": shape, "M": M, "N": N, "K": K, "reps": reps,
                      "weight_copies": len(ops)}))


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the FP8 linear layer is built and timed on a single MI355X; "
              "multi-GPU runs are not part of this library.", file=sys.stderr)
        sys.exit(2)
    if args.profile_case:
        profile_case(args.profile_case)
        return

    import numpy as np
    import torch

    import sparse_gemm_linears_amd as sgl
    import synth_inputs as si

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sgl.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M = si.PREFILL_M

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    # ------------------------------------------------------------ inputs ----
    layers = []
    for name, K, N in si.LLAMA3_8B:
        x = bf16(si.activations(M, K))
        w = bf16(si.weights(N, K))
        c = torch.from_numpy(si.column_norms(si.calibration_batch(K))).to(dev)
        L = dict(name=name, K=K, N=N, x=x, w=w, c=c,
                 xq=torch.empty((M, K), dtype=torch.uint8, device=dev),
                 xs=torch.empty((M, K // 128), dtype=torch.float32, device=dev),
                 wq=torch.empty((N, K), dtype=torch.uint8, device=dev),
                 ws=torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev),
                 wv=torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
                 wm=torch.empty((N, K // 8), dtype=torch.uint8, device=dev),
                 ws2=torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev),
                 y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                 y2=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
        layers.append(L)
    torch.cuda.synchronize()

    kernels = ("quant_act", "quant_wblock", "prune24", "dense_gemm", "sparse_gemm")

    def step(events=None, dominant=None):
        for li, L in enumerate(layers):
            calls = (
                lambda: sgl.fp8_quant_act(L["x"], L["xq"], L["xs"]),
                lambda: sgl.fp8_quant_weight_block(L["w"], L["wq"], L["ws"]),
                lambda: sgl.prune24_compress(L["w"], L["c"], L["wv"], L["wm"], L["ws2"]),
                lambda: sgl.fp8_block_gemm(L["xq"], L["xs"], L["wq"], L["ws"], L["y"]),
                lambda: sgl.fp8_sparse24_gemm(L["xq"], L["xs"], L["wv"], L["wm"], L["ws2"], L["y2"]),
            )
            for ki, f in enumerate(calls):
                if events is not None:
                    events[li][ki][0].record()
                if dominant is not None and li == dominant[0] and ki == 3:
                    dominant[1][0].record()
                    f()
                    dominant[1][1].record()
                else:
                    f()
                if events is not None:
                    events[li][ki][1].record()

    # Calibration copy for the HBM traffic counters: a plain device-to-device
    # copy of CALIB_BYTES, whose FETCH_SIZE / WRITE_SIZE readings under
    # rocprofv3 --pmc give the scale from counter KiB to bytes moved.
    calib_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ------------------------------------------------- timed whole steps ----
    # The dominant kernel (dense gate/up GEMM) is bracketed by events inside
    # the timed steps, on the stream the library launches on.
    gi = [L["name"] for L in layers].index("gate_up")
    dom_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(dominant=(gi, dom_ev[i]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    dom_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in dom_ev]))

    # ----------------------------------- per-kernel times (HIP events) ------
    # Steps back to back with one synchronisation at the end, so that the GPU
    # is always behind the host and an event pair brackets only its kernel;
    # the first step (which starts on an idle stream, with the host's launch
    # latency inside its first pair) is dropped.
    durations = {(li, ki): [] for li in range(len(layers)) for ki in range(len(kernels))}
    evs = [[[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in kernels] for _ in layers] for _ in range(args.steps + 1)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    for ev in evs[1:]:
        for li in range(len(layers)):
            for ki in range(len(kernels)):
                durations[(li, ki)].append(ev[li][ki][0].elapsed_time(ev[li][ki][1]) * 1e3)  # us

    def bytes_of(kname, K, N):
        if kname == "quant_act":
            return 2 * M * K + M * K + 4 * M * K // 128
        if kname == "quant_wblock":
            return 2 * N * K + N * K + 4 * (N // 128) * (K // 128)
        if kname == "prune24":
            return 2 * N * K + N * K // 2 + N * K // 8 + 4 * (N // 128) * (K // 128) + 4 * K
        return None

    per_kernel = {}
    dense_flops = sparse_flops = 0
    for li, L in enumerate(layers):
        K, N = L["K"], L["N"]
        dense_flops += 2 * M * N * K
        sparse_flops += M * N * K
        for ki, kname in enumerate(kernels):
            us = float(np.mean(durations[(li, ki)]))
            entry = {"us": round(us, 2)}
            if kname == "dense_gemm":
                tf = 2 * M * N * K / us / 1e6
                entry.update(tflops=round(tf, 1), frac_fp8_peak=round(tf / PEAK_FP8_TFLOPS, 4))
            elif kname == "sparse_gemm":
                tf = M * N * K / us / 1e6
                dense_us = float(np.mean(durations[(li, kernels.index("dense_gemm"))]))
                entry.update(tflops_algorithmic=round(tf, 1), tflops_dense_equivalent=round(2 * tf, 1),
                             frac_fp8_peak=round(tf / PEAK_FP8_TFLOPS, 4),
                             speedup_vs_dense=round(dense_us / us, 3))
            else:
                gbs = bytes_of(kname, K, N) / us / 1e3
                entry.update(gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
            per_kernel[f"{L['name']}.{kname}"] = entry

    gemm_flops = dense_flops + sparse_flops
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    # dominant kernel: the dense gate/up GEMM, timed inside the timed steps
    Lg = layers[gi]
    dom_flops = 2 * M * Lg["N"] * Lg["K"]
    achieved = dom_flops / dom_us / 1e6
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": measured_traffic(),
                "kernel": "fp8_block_gemm dense tile kernel, gate_up 4096x28672x4096",
                "avg_launch_us": round(dom_us, 2), "flops_per_launch": dom_flops,
                "algorithmic_bytes_per_launch": M * Lg["K"] + Lg["N"] * Lg["K"] + 4 * M * (Lg["K"] // 128)
                + 4 * (Lg["N"] // 128) * (Lg["K"] // 128) + 2 * M * Lg["N"]}

    # free the prefill working set before the decode measurements
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    dsv3, dsv3_rows = bench_dsv3(sgl, si, torch, np, dev, bf16, args.steps)
    per_tensor = bench_per_tensor(sgl, si, torch, np, dev, bf16, args.steps)
    swiglu = bench_swiglu(sgl, si, torch, np, dev, bf16, args.steps)
    grouped = bench_grouped(sgl, si, torch, np, dev, bf16, args.steps)
    ue8m0 = bench_ue8m0(sgl, si, torch, np, dev, bf16, args.steps)
    decode = None if args.no_decode else bench_decode(sgl, si, torch, np, dev, bf16)
    mid_m = None if args.no_decode else bench_mid_m(sgl, si, torch, np, dev, bf16, args.steps)
    cpu = None if args.no_cpu else cpu_baseline(si, np, args.cpu_rows, dsv3_rows)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "llama3_8b_linears_m4096: act quant + weight block quant + 2:4 prune/compress "
                               "+ dense and 2:4 block-scaled FP8 GEMM",
                   "tokens": M, "shapes_k_n": [[K, N] for _, K, N in si.LLAMA3_8B],
                   "gemm_flops_per_step": gemm_flops, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": per_kernel,
        "dsv3": dsv3,
        "per_tensor": per_tensor,
        "swiglu": swiglu,
        "grouped": grouped,
        "ue8m0": ue8m0,
        "decode": decode,
        "mid_m": mid_m,
    }
    print(json.dumps(out))


def time_calls(torch, f, reps):
    """Mean time of back-to-back calls of f, from HIP events on the current stream."""
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        f()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def bench_dsv3(sgl, si, torch, np, dev, bf16, steps):
    """The DeepSeek-V3 dense FFN linears at M = 8192 tokens (7168 -> 18432 and
    18432 -> 7168), Student-t (3 degrees of freedom) activations and N(0, 0.01)
    weights: the activation quantizer and the dense block-scaled GEMM, each the
    median of three batches of back-to-back calls (HIP events on the stream)."""
    M = si.DSV3_M
    res, sampled = {}, {}
    rows = si.sample_rows(M, 256, seed=5)
    for name, K, N in si.DSV3_FFN:
        xh = si.activations(M, K, dist="student_t3", outliers=False)
        sampled[name] = np.ascontiguousarray(xh[rows])  # the CPU oracle's sample of the same batch
        x = bf16(xh)
        del xh
        xq, xs = sgl.fp8_quant_act(x)
        wq, ws = sgl.fp8_quant_weight_block(bf16(si.weights(N, K, std=0.01)))
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        t_q = sorted(time_calls(torch, lambda: sgl.fp8_quant_act(x, xq, xs), steps) for _ in range(3))[1]
        t_g = sorted(time_calls(torch, lambda: sgl.fp8_block_gemm(xq, xs, wq, ws, y), steps) for _ in range(3))[1]
        tf = 2 * M * N * K / t_g / 1e6
        qbytes = 2 * M * K + M * K + 4 * M * (K // 128)
        res[name] = {"M": M, "K": K, "N": N, "gemm_us": round(t_g, 2), "gemm_tflops": round(tf, 1),
                     "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4), "quant_act_us": round(t_q, 2),
                     "quant_act_gbs": round(qbytes / t_q / 1e3, 1)}
        del x, xq, xs, wq, ws, y
    torch.cuda.empty_cache()
    return res, sampled


def bench_per_tensor(sgl, si, torch, np, dev, bf16, steps):
    """The dense and 2:4 GEMMs on per-tensor-scaled operands (fp8_quant_act_tensor
    activations; fp8_quant_weight_tensor or prune24_compress_tensor weights) on the
    four Llama-3-8B shapes at M = 4096, timed in alternating batches (medians of
    three).  Every scale product is then the same in every K block, so the 2:4 tile
    kernel sums unscaled block products and scales once (no VALU work per sparse
    MFMA); the dense kernel keeps its per-block scale FMAs."""
    M = si.PREFILL_M
    res = {}
    for name, K, N in si.LLAMA3_8B:
        x, w = bf16(si.activations(M, K)), bf16(si.weights(N, K))
        c = torch.from_numpy(si.column_norms(si.calibration_batch(K))).to(dev)
        xq, xs = sgl.fp8_quant_act_tensor(x)
        wq, ws = sgl.fp8_quant_weight_tensor(w)
        v, m, s2 = sgl.prune24_compress_tensor(w, c)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        t_d, t_s = [], []
        for _ in range(3):
            t_d.append(time_calls(torch, lambda: sgl.fp8_block_gemm(xq, xs, wq, ws, y), steps))
            t_s.append(time_calls(torch, lambda: sgl.fp8_sparse24_gemm(xq, xs, v, m, s2, y), steps))
        td, ts = sorted(t_d)[1], sorted(t_s)[1]
        res[name] = {"dense_us": round(td, 2), "dense_tflops": round(2 * M * N * K / td / 1e6, 1),
                     "sparse_us": round(ts, 2), "sparse_tflops_algorithmic": round(M * N * K / ts / 1e6, 1),
                     "speedup_vs_dense": round(td / ts, 3)}
        del x, w, c, xq, xs, wq, ws, v, m, s2, y
    torch.cuda.empty_cache()
    return res


def bench_ue8m0(sgl, si, torch, np, dev, bf16, steps):
    """UE8M0 (power-of-two) scales on the four Llama-3-8B shapes at M=4096: the two
    quantizers, and the GEMM whose scales the MFMA applies timed in alternating
    batches with the fp32-scale GEMM of the same shape (clock drift between
    separate runs is larger than the difference between the two)."""
    M = si.PREFILL_M
    res = {}
    for name, K, N in si.LLAMA3_8B:
        x, w = bf16(si.activations(M, K)), bf16(si.weights(N, K))
        xq, xe = sgl.fp8_quant_act_ue8m0(x)
        wq, we = sgl.fp8_quant_weight_block_ue8m0(w)
        xq4, xs4 = sgl.fp8_quant_act(x)
        wq4, ws4 = sgl.fp8_quant_weight_block(w)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        t_qa = time_calls(torch, lambda: sgl.fp8_quant_act_ue8m0(x, xq, xe), steps)
        t_qw = time_calls(torch, lambda: sgl.fp8_quant_weight_block_ue8m0(w, wq, we), steps)
        t_e8, t_f32 = [], []
        for _ in range(3):
            t_f32.append(time_calls(torch, lambda: sgl.fp8_block_gemm(xq4, xs4, wq4, ws4, y), steps))
            t_e8.append(time_calls(torch, lambda: sgl.fp8_block_gemm_ue8m0(xq, xe, wq, we, y), steps))
        t_g, t_f = sorted(t_e8)[1], sorted(t_f32)[1]
        tf = 2 * M * N * K / t_g / 1e6
        res[name] = {"quant_act_us": round(t_qa, 2), "quant_wblock_us": round(t_qw, 2), "gemm_us": round(t_g, 2),
                     "gemm_tflops": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                     "fp32_scale_gemm_us": round(t_f, 2)}
        del x, w, xq, xe, wq, we, xq4, xs4, wq4, ws4, y
    torch.cuda.empty_cache()
    return res


def bench_grouped(sgl, si, torch, np, dev, bf16, steps):
    """The grouped (MoE) GEMM on DeepSeek-V3 routed-expert shapes: 16384 routed token
    rows over 32 experts with a seeded uneven routing (some experts empty), beside the
    plain GEMM of the same M x N x K, timed in alternating batches (medians of three).
    The experts hold copies of one quantized weight at distinct addresses: the same
    bytes move as with 32 different weights."""
    M, G = 16384, 32
    res = {}
    for name, K, N in si.DSV3_EXPERTS:
        xq, xs = sgl.fp8_quant_act(bf16(si.activations(M, K, dist="student_t3", outliers=False)))
        wq1, ws1 = sgl.fp8_quant_weight_block(bf16(si.weights(N, K, std=0.01)))
        wq = wq1.unsqueeze(0).repeat(G, 1, 1).contiguous()
        ws = ws1.unsqueeze(0).repeat(G, 1, 1).contiguous()
        offs = torch.from_numpy(si.routed_offsets(M, G, seed=7)).to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        t_g, t_p = [], []
        for _ in range(3):
            t_g.append(time_calls(torch, lambda: sgl.fp8_grouped_gemm(xq, xs, wq, ws, offs, y), steps))
            t_p.append(time_calls(torch, lambda: sgl.fp8_block_gemm(xq, xs, wq1, ws1, y), steps))
        tg, tp = sorted(t_g)[1], sorted(t_p)[1]
        tf = 2 * M * N * K / tg / 1e6
        res[name] = {"M": M, "experts": G, "N": N, "K": K, "grouped_us": round(tg, 2), "grouped_tflops": round(tf, 1),
                     "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4), "plain_gemm_us": round(tp, 2),
                     "expert_weight_mb": round(G * N * K / 1e6, 1)}
        del xq, xs, wq1, ws1, wq, ws, offs, y
    torch.cuda.empty_cache()
    return res


def bench_swiglu(sgl, si, torch, np, dev, bf16, steps):
    """The gated-MLP up projection at M=4096 (gate/up 4096 -> 2 x 14336): the fused
    GEMM + SwiGLU call with h and its e4m3 codes for the down projection, with the
    codes only (h not stored), and with h only, beside the plain GEMM of the same
    weight and fp8_quant_act of h."""
    M, K, I = si.PREFILL_M, 4096, 14336
    xq, xs = sgl.fp8_quant_act(bf16(si.activations(M, K)))
    wq, ws = sgl.fp8_quant_weight_block(bf16(si.weights(2 * I, K)))
    y = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    h = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    hq = torch.empty((M, I), dtype=torch.uint8, device=dev)
    hs = torch.empty((M, I // 128), dtype=torch.float32, device=dev)
    runs = {
        "gemm_swiglu_quant": lambda: sgl.fp8_block_gemm_swiglu(xq, xs, wq, ws, h, True, hq, hs),
        "gemm_swiglu_quant_only": lambda: sgl.fp8_block_gemm_swiglu(xq, xs, wq, ws, None, True, hq, hs, keep_h=False),
        "gemm_swiglu": lambda: sgl.fp8_block_gemm_swiglu(xq, xs, wq, ws, h, False),
        "gemm_only": lambda: sgl.fp8_block_gemm(xq, xs, wq, ws, y),
        "quant_act_of_h": lambda: sgl.fp8_quant_act(h, hq, hs),
    }
    # three alternating rounds, medians: the order of separate runs shifts the
    # clock by more than the differences measured here
    times = {name: [] for name in runs}
    for _ in range(3):
        for name, f in runs.items():
            times[name].append(time_calls(torch, f, steps))
    res = {}
    for name in runs:
        us = sorted(times[name])[1]
        entry = {"us": round(us, 2)}
        if name != "quant_act_of_h":
            entry["tflops"] = round(2 * M * 2 * I * K / us / 1e6, 1)
        res[name] = entry
    del y, h, hq, hs, wq, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(sgl, si, torch, np, dev, bf16):
    """Decode-M GEMMs: dense at M in {1,8,16,32,64}, 2:4 at M=16, each shape with
    enough weight copies (>= 1 GiB in total) that every call reads its weight
    from HBM; beside each, the fused-quantization call and the two-call path it
    replaces.  Each call is timed as a HIP-graph replay of back-to-back calls."""
    res = {}
    for name, K, N in si.LLAMA3_8B:
        wq_bytes = N * K
        copies = max(2, math.ceil((1 << 30) / wq_bytes))
        w = bf16(si.weights(N, K))
        c = torch.from_numpy(si.column_norms(si.calibration_batch(K))).to(dev)
        wq0, ws0 = sgl.fp8_quant_weight_block(w)
        wv0, wm0, ws20 = sgl.prune24_compress(w, c)
        dense_w = [(wq0.clone(), ws0.clone()) for _ in range(copies)]
        sparse_w = [(wv0.clone(), wm0.clone(), ws20.clone()) for _ in range(copies)]
        del w, wq0, wv0, wm0
        for M in (1, 8, 16, 32, 64):
            x = bf16(si.activations(M, K))
            xq, xs = sgl.fp8_quant_act(x)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            # "dense"/"sparse": the GEMM on codes already quantized; "*_linear": the fused call on
            # bf16 activations; "*_two_call": fp8_quant_act then the GEMM, the path the fused call replaces
            runs = {"dense": lambda i: sgl.fp8_block_gemm(xq, xs, dense_w[i][0], dense_w[i][1], y),
                    "dense_linear": lambda i: sgl.fp8_block_linear(x, dense_w[i][0], dense_w[i][1], y),
                    "dense_two_call": lambda i: (sgl.fp8_quant_act(x, xq, xs),
                                                 sgl.fp8_block_gemm(xq, xs, dense_w[i][0], dense_w[i][1], y))}
            if M == 16:
                runs["sparse"] = lambda i: sgl.fp8_sparse24_gemm(xq, xs, *sparse_w[i], y)
                runs["sparse_linear"] = lambda i: sgl.fp8_sparse24_linear(x, *sparse_w[i], y)
                runs["sparse_two_call"] = lambda i: (sgl.fp8_quant_act(x, xq, xs),
                                                     sgl.fp8_sparse24_gemm(xq, xs, *sparse_w[i], y))
            for kind, f in runs.items():
                us = time_graph(torch, f, copies)
                wbytes = N * K if kind.startswith("dense") else N * K // 2 + N * K // 8
                # activation bytes: fp8 codes + scales for the GEMM, bf16 for the fused call
                xbytes = 2 * M * K if kind.endswith("linear") else M * K + 4 * M * (K // 128)
                nbytes = wbytes + 4 * (N // 128) * (K // 128) + xbytes + 2 * M * N
                gbs = nbytes / us / 1e3
                res[f"{name}.M{M}.{kind}"] = {"us": round(us, 2), "gbs": round(gbs, 1),
                                              "frac_hbm": round(gbs / 8000.0, 4)}
            if "sparse" in runs:
                res[f"{name}.M16.sparse"]["speedup_vs_dense"] = round(
                    res[f"{name}.M16.dense"]["us"] / res[f"{name}.M16.sparse"]["us"], 3)
        del dense_w, sparse_w
        torch.cuda.empty_cache()
    return res


def bench_mid_m(sgl, si, torch, np, dev, bf16, steps):
    """Mid-size batches (M in {128, 512}) on the four Llama-3-8B shapes, dense and
    2:4: the tile kernels with the tile height and K split chosen for the
    shape (back-to-back calls; the weight of one shape fits the MALL, so these
    are the compute-side times)."""
    res = {}
    for name, K, N in si.LLAMA3_8B:
        w = bf16(si.weights(N, K))
        wq, ws = sgl.fp8_quant_weight_block(w)
        wv, wm, ws2 = sgl.prune24_compress(w)
        for M in (128, 512):
            xq, xs = sgl.fp8_quant_act(bf16(si.activations(M, K)))
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            for kind, f in (("dense", lambda: sgl.fp8_block_gemm(xq, xs, wq, ws, y)),
                            ("sparse", lambda: sgl.fp8_sparse24_gemm(xq, xs, wv, wm, ws2, y))):
                us = time_calls(torch, f, steps)
                flops = 2 * M * N * K * (1 if kind == "dense" else 0.5)
                res[f"{name}.M{M}.{kind}"] = {"us": round(us, 2), "tflops": round(flops / us / 1e6, 1)}
        del w, wq, ws, wv, wm, ws2
    torch.cuda.empty_cache()
    return res


def time_graph(torch, f, copies, reps=3):
    """Average time per call of f(i), i cycling over the weight copies, from a
    captured HIP graph of `copies` back-to-back calls replayed `reps` times."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(min(copies, 3)):
            f(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(copies):
            f(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * copies)


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(si, np, rows, dsv3_sampled):
    """The CPU oracle on a bounded sample of the step: for each of the four
    shapes, activation quant of `rows` tokens, weight block quant and 2:4
    prune/compress of the whole weight, and the dense and 2:4 GEMMs of those
    `rows` tokens.  Reported in the step's unit (algorithmic GEMM TFLOP/s);
    input generation is not timed.  Beside it, the DeepSeek-V3 FFN GEMMs on the
    seeded 256-row sample of the 8192 tokens in `dsv3_sampled` (activation
    quant of those rows, weight block quant, the GEMM of those rows), with the
    full-size time extrapolated by rows and labelled so."""
    import oracle

    oracle.build()
    inputs = [(si.activations(rows, K), si.weights(N, K), si.column_norms(si.calibration_batch(K)), K, N)
              for _, K, N in si.LLAMA3_8B]
    flops = 0
    t0 = time.perf_counter()
    for x, w, c, K, N in inputs:
        xq, xs = oracle.quant_act(x)
        wq, ws = oracle.quant_wblock(w)
        v, m, s2 = oracle.prune24_compress(w, c)
        oracle.gemm(xq, xs, wq, ws)
        oracle.sparse24_gemm(xq, xs, v, m, s2)
        flops += 3 * rows * N * K
    total = time.perf_counter() - t0

    dsv3 = {}
    for name, K, N in si.DSV3_FFN:
        x = dsv3_sampled[name]  # rows of the 8192-token Student-t batch the GPU leg used
        dsv3_rows = x.shape[0]
        w = si.weights(N, K, std=0.01)
        t1 = time.perf_counter()
        wq, ws = oracle.quant_wblock(w)
        t2 = time.perf_counter()
        xq, xs = oracle.quant_act(x)
        oracle.gemm(xq, xs, wq, ws)
        t3 = time.perf_counter()
        rows_sec = t3 - t2
        dsv3[name] = {"rows": int(dsv3_rows), "weight_quant_seconds": round(t2 - t1, 2),
                      "rows_seconds": round(rows_sec, 2),
                      "gemm_tflops": round(2 * dsv3_rows * N * K / rows_sec / 1e12, 6),
                      "full_seconds_extrapolated": round((t2 - t1) + rows_sec * si.DSV3_M / dsv3_rows, 1),
                      "note": f"extrapolated: the whole weight quantization plus {si.DSV3_M // dsv3_rows} times the "
                              f"act quant + GEMM of the {dsv3_rows}-row sample"}
    return {"value": round(flops / total / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(total, 2),
            "sample": f"each Llama-3-8B shape: quant of {rows} token rows, block quant and 2:4 prune of the "
                      f"whole weight, dense + 2:4 GEMM of the {rows} rows (fp64 oracle, OpenMP over rows)",
            "dsv3_ffn_m8192": dsv3}


if __name__ == "__main__":
    main()
