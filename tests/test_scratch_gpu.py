"""The library's scratch memory (split-K partials, quantized tokens of the fused
linear calls, SwiGLU partials), kept between calls per stream and per capture.
Calls whose needs grow on a fresh stream with no synchronisation between them,
calls on two streams at once, a graph replayed on one stream while the same
calls run eagerly on another, two graphs captured on one stream replayed on
two streams at once, and captures past the memory kept for captures: every
output equals that of the call run alone, bit for bit (the calls themselves
are checked against the oracle elsewhere)."""
from __future__ import annotations

import pytest
import torch

import synth_inputs as si
from test_parity_gpu import bf16_dev, dev, llama_acts, llama_sparse_weight, llama_weight

pytestmark = pytest.mark.gpu


def shape(name):
    return next(s for s in si.LLAMA3_8B if s[0] == name)


class Inputs:
    """Device inputs shared by every copy of the cases (read-only)."""

    def __init__(self):
        self.dense = {}
        for M, name in ((8, "o_proj"), (40, "gate_up"), (48, "down"), (128, "qkv"), (256, "down")):
            _, K, N = shape(name)
            x, (xq, xs) = llama_acts(M, K)
            _, (wq, ws) = llama_weight(K, N)
            self.dense[(M, name)] = (bf16_dev(x), dev(xq), dev(xs), dev(wq), dev(ws))
        _, K, N = shape("down")
        _, (xq, xs) = llama_acts(256, K)
        _, (vals, meta, ws) = llama_sparse_weight(K, N, True)
        self.sparse = (dev(xq), dev(xs), dev(vals), dev(meta), dev(ws))
        _, K, N2 = shape("gate_up")
        _, (xq, xs) = llama_acts(16, K)
        _, (wq, ws) = llama_weight(K, N2)
        self.swiglu = (dev(xq), dev(xs), dev(wq), dev(ws))


def make_cases(gpu_lib, inp: Inputs):
    """(fn, outputs): each fn writes its outputs with one library call that
    uses scratch memory; a second call to make_cases gives fresh outputs."""
    cases = []

    def out(*shape_, dtype=torch.bfloat16):
        return torch.zeros(shape_, dtype=dtype, device="cuda")

    for (M, name), (x, xq, xs, wq, ws) in inp.dense.items():
        y = out(M, wq.shape[0])
        cases.append((lambda xq=xq, xs=xs, wq=wq, ws=ws, y=y: gpu_lib.fp8_block_gemm(xq, xs, wq, ws, y), [y]))
        if M <= 64:
            y2 = out(M, wq.shape[0])
            cases.append((lambda x=x, wq=wq, ws=ws, y=y2: gpu_lib.fp8_block_linear(x, wq, ws, y), [y2]))
    xq, xs, vals, meta, ws = inp.sparse
    y = out(xq.shape[0], vals.shape[0])
    cases.append((lambda y=y: gpu_lib.fp8_sparse24_gemm(xq, xs, vals, meta, ws, y), [y]))
    sxq, sxs, swq, sws = inp.swiglu
    M, I = sxq.shape[0], swq.shape[0] // 2
    h, hq, hs = out(M, I), out(M, I, dtype=torch.uint8), out(M, I // 128, dtype=torch.float32)
    cases.append((lambda: gpu_lib.fp8_block_gemm_swiglu(sxq, sxs, swq, sws, h, True, hq, hs), [h, hq, hs]))
    return cases


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8)


@pytest.fixture(scope="module")
def setup(gpu_lib):
    inp = Inputs()
    cases = make_cases(gpu_lib, inp)
    refs = []
    for fn, outs in cases:
        fn()
        torch.cuda.synchronize()
        refs.append([o.clone() for o in outs])
    return inp, refs


def check(cases, refs, what):
    for i, ((_, outs), ref) in enumerate(zip(cases, refs)):
        for o, r in zip(outs, ref):
            assert torch.equal(bits(o), bits(r)), f"{what}: case {i}"


def test_growing_needs_on_a_fresh_stream(gpu_lib, setup):
    inp, refs = setup
    cases = make_cases(gpu_lib, inp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for fn, _ in cases + cases[::-1] + cases:
            fn()
    torch.cuda.synchronize()
    check(cases, refs, "one stream")


def test_two_streams_at_once(gpu_lib, setup):
    inp, refs = setup
    a, b = make_cases(gpu_lib, inp), make_cases(gpu_lib, inp)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(2):
        for (fa, _), (fb, _) in zip(a, b[::-1]):
            with torch.cuda.stream(s1):
                fa()
            with torch.cuda.stream(s2):
                fb()
    torch.cuda.synchronize()
    check(a, refs, "stream 1")
    check(b, refs, "stream 2")


def capture(cases):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn, _ in cases:
            fn()
    torch.cuda.synchronize()
    return g


def zero(cases):
    for _, outs in cases:
        for o in outs:
            o.zero_()


def test_graph_replay_beside_eager_calls(gpu_lib, setup):
    inp, refs = setup
    graphed, eager = make_cases(gpu_lib, inp), make_cases(gpu_lib, inp)
    g = capture(graphed)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(3):
        zero(graphed)
        zero(eager)
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            g.replay()
        with torch.cuda.stream(s2):
            for fn, _ in eager[::-1]:
                fn()
        torch.cuda.synchronize()
        check(graphed, refs, f"replay {i}")
        check(eager, refs, f"eager beside replay {i}")


def test_two_graphs_from_one_stream_replayed_at_once(gpu_lib, setup):
    inp, refs = setup
    a, b = make_cases(gpu_lib, inp), make_cases(gpu_lib, inp)
    ga, gb = capture(a), capture(b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(3):
        zero(a)
        zero(b)
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            ga.replay()
        with torch.cuda.stream(s2):
            gb.replay()
        torch.cuda.synchronize()
        check(a, refs, f"graph a, replay {i}")
        check(b, refs, f"graph b, replay {i}")


def test_captures_past_the_kept_limit(gpu_lib, setup):
    """Captures keep their scratch memory (up to 1 GiB in all); past that a
    capture allocates inside its graph instead.  Forty captures of a split-K
    GEMM needing 33.5 or 67 MB each (down projection, 256 tokens: 8 or 16
    splits of 256 x 4096 fp32, by the tile height chosen) cross the limit;
    every graph, replayed afterwards, gives the eager result."""
    _, K, N = shape("down")
    _, (xq, xs) = llama_acts(256, K)
    _, (wq, ws) = llama_weight(K, N)
    a, b, c, d = dev(xq), dev(xs), dev(wq), dev(ws)
    ref = gpu_lib.fp8_block_gemm(a, b, c, d)
    torch.cuda.synchronize()
    ys, graphs = [], []
    for _ in range(40):
        y = torch.zeros_like(ref)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gpu_lib.fp8_block_gemm(a, b, c, d, y)
        ys.append(y)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(2):
        for y, g in zip(ys, graphs):
            y.zero_()
            g.replay()
        torch.cuda.synchronize()
        for j, y in enumerate(ys):
            assert torch.equal(bits(y), bits(ref)), f"pass {i}, graph {j}"
    del graphs
    import gc
    gc.collect()
    torch.cuda.synchronize()
    # every graph that held the kept buffers is gone: they can be freed, and a
    # new capture afterwards keeps (and uses) fresh ones
    gpu_lib.fp8lin_release_graph_scratch()
    y = torch.zeros_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_lib.fp8_block_gemm(a, b, c, d, y)
    for _ in range(2):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(ref)), "capture after the release"


def test_threads_sharing_one_stream(gpu_lib, setup):
    """Two host threads issue scratch-using calls on one stream at once: a call
    holds the scratch lock until its launches are enqueued, so each call's
    kernels use a buffer no other call frees or reuses in between."""
    import threading
    inp, refs = setup
    a, b = make_cases(gpu_lib, inp), make_cases(gpu_lib, inp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    errors = []

    def run(cases, order):
        try:
            with torch.cuda.stream(s):
                for _ in range(3):
                    for fn, _ in (cases if order else cases[::-1]):
                        fn()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    ts = [threading.Thread(target=run, args=(a, True)), threading.Thread(target=run, args=(b, False))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    check(a, refs, "thread 1")
    check(b, refs, "thread 2")


def test_per_thread_default_stream(gpu_lib, setup):
    """hipStreamPerThread is one handle value naming a different stream in each
    thread: two threads passing it run on two streams, and their calls must not
    share a scratch buffer."""
    import ctypes
    import threading
    inp, refs = setup
    lib = gpu_lib.load_library()
    per_thread = ctypes.c_void_p(2)  # hipStreamPerThread
    _, K, N = shape("down")
    _, (xq, xs) = llama_acts(256, K)
    _, (wq, ws) = llama_weight(K, N)
    a, b_, c, d = dev(xq), dev(xs), dev(wq), dev(ws)
    ref = gpu_lib.fp8_block_gemm(a, b_, c, d)
    _, (xq2, xs2) = llama_acts(128, K)
    a2, b2 = dev(xq2), dev(xs2)
    ref2 = gpu_lib.fp8_block_gemm(a2, b2, c, d)
    torch.cuda.synchronize()
    outs = [[torch.zeros_like(ref) for _ in range(4)], [torch.zeros_like(ref2) for _ in range(4)]]
    status = []

    def run(x, s, ys):
        for y in ys:
            status.append(lib.fp8_block_gemm(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                                             ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(d.data_ptr()),
                                             x.shape[0], N, K, ctypes.c_void_p(y.data_ptr()), per_thread))

    ts = [threading.Thread(target=run, args=(a, b_, outs[0])), threading.Thread(target=run, args=(a2, b2, outs[1]))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert status == [0] * 8, status
    for y in outs[0]:
        assert torch.equal(bits(y), bits(ref))
    for y in outs[1]:
        assert torch.equal(bits(y), bits(ref2))
