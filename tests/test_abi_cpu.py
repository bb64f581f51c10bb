"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import sparse_gemm_linears_amd as sgl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8lin.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:fp8l_status|const char \*)\s*(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    return sgl.load_library()


def test_header_declares_every_exported_call():
    names = header_functions()
    assert set(names) == set(sgl.EXPORTS)
    assert len(names) == len(set(names))


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in range(9):
        assert sgl.status_str(st) != "unknown status"
    assert sgl.status_str(999) == "unknown status"


# fake, 16-byte aligned, non-overlapping host addresses: validation fails before
# any HIP call, so nothing dereferences them
A = 1 << 32
B = 2 << 32
C = 3 << 32
D = 4 << 32
E = 5 << 32
F = 6 << 32


def call(lib, name, *args):
    fn = getattr(lib, name)
    conv = [ctypes.c_void_p(a) if isinstance(a, int) and a >= (1 << 31) else a for a in args]
    return fn(*conv)


def P(v):
    return None if v == 0 else ctypes.c_void_p(v)


def test_quant_act_validation(lib):
    assert lib.fp8_quant_act(P(A), 4, 100, P(B), P(C), None) == sgl.FP8L_ERR_SHAPE
    assert lib.fp8_quant_act(P(A), -1, 128, P(B), P(C), None) == sgl.FP8L_ERR_SHAPE
    assert lib.fp8_quant_act(P(A), 4, 0, P(B), P(C), None) == sgl.FP8L_ERR_SHAPE
    assert lib.fp8_quant_act(P(A), 4, 1 << 25, P(B), P(C), None) == sgl.FP8L_ERR_SHAPE
    assert lib.fp8_quant_act(None, 4, 128, P(B), P(C), None) == sgl.FP8L_ERR_NULL
    assert lib.fp8_quant_act(P(A), 4, 128, None, P(C), None) == sgl.FP8L_ERR_NULL
    assert lib.fp8_quant_act(P(A + 8), 4, 128, P(B), P(C), None) == sgl.FP8L_ERR_ALIGN
    assert lib.fp8_quant_act(P(A), 4, 128, P(A + 512), P(C), None) == sgl.FP8L_ERR_ALIAS
    assert lib.fp8_quant_act(P(A), 4, 128, P(B), P(B + 256), None) == sgl.FP8L_ERR_ALIAS
    # empty batch: OK without looking at pointers
    assert lib.fp8_quant_act(None, 0, 128, None, None, None) == sgl.FP8L_OK


def test_weight_quant_validation(lib):
    assert lib.fp8_quant_weight_block(P(A), 100, 128, P(B), P(C), None) == sgl.FP8L_ERR_SHAPE
    assert lib.fp8_quant_weight_block(P(A), 0, 128, P(B), P(C), None) == sgl.FP8L_ERR_SHAPE
    assert lib.fp8_quant_weight_block(P(A), 128, 128, None, P(C), None) == sgl.FP8L_ERR_NULL
    assert lib.fp8_quant_weight_block(P(A), 128, 128, P(B), P(C + 4), None) == sgl.FP8L_ERR_ALIGN
    assert lib.fp8_quant_weight_block(P(A), 128, 128, P(A), P(C), None) == sgl.FP8L_ERR_ALIAS


def test_tensor_scale_quant_validation(lib):
    t = lib.fp8_quant_act_tensor
    assert t(P(A), 4, 100, P(B), P(C), None) == sgl.FP8L_ERR_SHAPE
    assert t(P(A), 4, 128, None, P(C), None) == sgl.FP8L_ERR_NULL
    assert t(P(A), 4, 128, P(B), P(C + 8), None) == sgl.FP8L_ERR_ALIGN
    assert t(P(A), 4, 128, P(B), P(A + 16), None) == sgl.FP8L_ERR_ALIAS
    assert t(None, 0, 128, None, None, None) == sgl.FP8L_OK
    st = lib.fp8_quant_act_static
    assert st(P(A), P(D), 4, 100, P(B), P(C), None) == sgl.FP8L_ERR_SHAPE
    assert st(P(A), None, 4, 128, P(B), P(C), None) == sgl.FP8L_ERR_NULL
    assert st(P(A), P(D + 2), 4, 128, P(B), P(C), None) == sgl.FP8L_ERR_ALIGN
    assert st(P(A), P(C + 4), 4, 128, P(B), P(C), None) == sgl.FP8L_ERR_ALIAS     # scale inside s
    assert st(P(A), P(B + 12), 4, 128, P(B), P(C), None) == sgl.FP8L_ERR_ALIAS    # scale inside q
    assert st(None, None, 0, 128, None, None, None) == sgl.FP8L_OK
    w = lib.fp8_quant_weight_tensor
    assert w(P(A), 100, 128, P(B), P(C), None) == sgl.FP8L_ERR_SHAPE
    assert w(P(A), 128, 128, P(B), None, None) == sgl.FP8L_ERR_NULL
    assert w(P(A), 128, 128, P(B + 4), P(C), None) == sgl.FP8L_ERR_ALIGN
    assert w(P(A), 128, 128, P(B), P(B + 64), None) == sgl.FP8L_ERR_ALIAS


def test_prune_validation(lib):
    f = lib.prune24_compress
    assert f(P(A), None, 128, 130, P(B), P(C), P(D), None) == sgl.FP8L_ERR_SHAPE
    assert f(P(A), None, 128, 128, P(B), None, P(D), None) == sgl.FP8L_ERR_NULL
    assert f(P(A), P(E + 4), 128, 128, P(B), P(C), P(D), None) == sgl.FP8L_ERR_ALIGN
    assert f(P(A), P(B), 128, 128, P(B), P(C), P(D), None) == sgl.FP8L_ERR_ALIAS      # vals over col_norm
    assert f(P(A), None, 128, 128, P(B), P(B + 4096), P(D), None) == sgl.FP8L_ERR_ALIAS  # vals/meta overlap


def test_prune_tensor_validation(lib):
    f = lib.prune24_compress_tensor
    assert f(P(A), None, 128, 130, P(B), P(C), P(D), None) == sgl.FP8L_ERR_SHAPE
    assert f(P(A), None, 100, 128, P(B), P(C), P(D), None) == sgl.FP8L_ERR_SHAPE
    assert f(P(A), None, 128, 128, P(B), P(C), None, None) == sgl.FP8L_ERR_NULL
    assert f(P(A), P(E + 4), 128, 128, P(B), P(C), P(D), None) == sgl.FP8L_ERR_ALIGN
    assert f(P(A), None, 128, 128, P(B), P(C), P(B + 64), None) == sgl.FP8L_ERR_ALIAS     # s inside vals


def test_gemm_validation(lib):
    g = lib.fp8_block_gemm
    assert g(P(A), P(B), P(C), P(D), 16, 100, 128, P(E), None) == sgl.FP8L_ERR_SHAPE
    assert g(P(A), P(B), P(C), P(D), 16, 128, 96, P(E), None) == sgl.FP8L_ERR_SHAPE
    assert g(P(A), P(B), P(C), None, 16, 128, 128, P(E), None) == sgl.FP8L_ERR_NULL
    assert g(P(A), P(B), P(C), P(D), 16, 128, 128, P(E + 2), None) == sgl.FP8L_ERR_ALIGN
    assert g(P(A), P(B), P(C), P(D), 16, 128, 128, P(C + 16), None) == sgl.FP8L_ERR_ALIAS
    assert g(None, None, P(C), P(D), 0, 128, 128, None, None) == sgl.FP8L_OK
    n = lib.fp8_block_gemm_noalloc  # the same checks, in the same order
    assert n(P(A), P(B), P(C), P(D), 16, 100, 128, P(E), None) == sgl.FP8L_ERR_SHAPE
    assert n(P(A), P(B), P(C), None, 16, 128, 128, P(E), None) == sgl.FP8L_ERR_NULL
    assert n(P(A), P(B), P(C), P(D), 16, 128, 128, P(E + 2), None) == sgl.FP8L_ERR_ALIGN
    assert n(P(A), P(B), P(C), P(D), 16, 128, 128, P(C + 16), None) == sgl.FP8L_ERR_ALIAS
    assert n(None, None, P(C), P(D), 0, 128, 128, None, None) == sgl.FP8L_OK
    h = lib.fp8_sparse24_gemm
    assert h(P(A), P(B), P(C), P(D), P(E), 16, 128, 100, P(F), None) == sgl.FP8L_ERR_SHAPE
    assert h(P(A), P(B), None, P(D), P(E), 16, 128, 128, P(F), None) == sgl.FP8L_ERR_NULL
    assert h(P(A), P(B), P(C), P(D + 1), P(E), 16, 128, 128, P(F), None) == sgl.FP8L_ERR_ALIGN
    assert h(P(A), P(B), P(C), P(D), P(E), 16, 128, 128, P(D), None) == sgl.FP8L_ERR_ALIAS


def test_swiglu_validation(lib):
    f = lib.fp8_block_gemm_swiglu
    # I must be a multiple of 128 itself (2I = 128 is not enough)
    assert f(P(A), P(B), P(C), P(D), 16, 64, 128, P(E), None, None, None) == sgl.FP8L_ERR_SHAPE
    assert f(P(A), P(B), P(C), P(D), 16, 0, 128, P(E), None, None, None) == sgl.FP8L_ERR_SHAPE
    assert f(P(A), P(B), P(C), P(D), 16, 128, 128, P(E), P(F), None, None) == sgl.FP8L_ERR_NULL  # hq without hs
    assert f(P(A), P(B), P(C), P(D), 16, 128, 128, None, None, None, None) == sgl.FP8L_ERR_NULL  # nothing to produce
    assert f(P(A), P(B), P(C), P(D), 16, 128, 128, None, P(F), None, None) == sgl.FP8L_ERR_NULL  # h omitted, hs missing
    assert f(P(A), P(B), P(C), P(D), 16, 128, 128, None, P(F + 4), P(E), None) == sgl.FP8L_ERR_ALIGN
    assert f(P(A), P(B), P(C), P(D), 16, 128, 128, None, P(F), P(D), None) == sgl.FP8L_ERR_ALIAS  # hs over ws
    assert f(P(A), P(B), P(C), P(D), 16, 128, 128, P(E + 2), None, None, None) == sgl.FP8L_ERR_ALIGN
    assert f(P(A), P(B), P(C), P(D), 16, 128, 128, P(D), None, None, None) == sgl.FP8L_ERR_ALIAS


def test_linear_validation(lib):
    """The fused-quantization calls: same checks as the GEMMs, plus M <= 64."""
    f = lib.fp8_block_linear
    assert f(P(A), P(C), P(D), 65, 128, 128, P(E), None) == sgl.FP8L_ERR_SHAPE
    assert f(P(A), P(C), P(D), 16, 100, 128, P(E), None) == sgl.FP8L_ERR_SHAPE
    assert f(P(A), P(C), P(D), 16, 128, 96, P(E), None) == sgl.FP8L_ERR_SHAPE
    assert f(P(A), None, P(D), 16, 128, 128, P(E), None) == sgl.FP8L_ERR_NULL
    assert f(P(A), P(C), P(D), 16, 128, 128, P(E + 8), None) == sgl.FP8L_ERR_ALIGN
    assert f(P(A), P(C), P(D), 16, 128, 128, P(A + 1024), None) == sgl.FP8L_ERR_ALIAS  # y over x
    assert f(None, P(C), P(D), 0, 128, 128, None, None) == sgl.FP8L_OK
    h = lib.fp8_sparse24_linear
    assert h(P(A), P(B), P(C), P(D), 65, 128, 128, P(E), None) == sgl.FP8L_ERR_SHAPE
    assert h(P(A), P(B), None, P(D), 16, 128, 128, P(E), None) == sgl.FP8L_ERR_NULL
    assert h(P(A), P(B), P(C + 4), P(D), 16, 128, 128, P(E), None) == sgl.FP8L_ERR_ALIGN
    assert h(P(A), P(B), P(C), P(D), 16, 128, 128, P(C), None) == sgl.FP8L_ERR_ALIAS
    assert h(None, P(B), P(C), P(D), 0, 128, 128, None, None) == sgl.FP8L_OK


def test_valid_call_without_gpu_reports_device(lib):
    """With valid arguments and no gfx950 device the call stops at the device check."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.fp8_quant_act(P(A), 4, 128, P(B), P(C), None) == sgl.FP8L_ERR_DEVICE
    assert lib.fp8_block_gemm(P(A), P(B), P(C), P(D), 16, 128, 128, P(E), None) == sgl.FP8L_ERR_DEVICE
    assert lib.fp8_block_linear(P(A), P(C), P(D), 16, 128, 128, P(E), None) == sgl.FP8L_ERR_DEVICE
    assert lib.fp8_block_gemm_noalloc(P(A), P(B), P(C), P(D), 16, 128, 128, P(E), None) == sgl.FP8L_ERR_DEVICE
    # nothing kept for graphs: releasing is a no-op that needs no device
    assert lib.fp8lin_release_graph_scratch() == sgl.FP8L_OK


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sgl.fp8_quant_act(x)
    with pytest.raises(TypeError):
        sgl.fp8_quant_act(x.float())
