"""The GPU quantizers' fast quotient, checked exhaustively on the CPU.

The quantizers encode x / s (s = fl(amax / 448), amax the largest |x| of the
group) without a division per element: q0 = fl(x * rs) with rs = fl(1 / s),
corrected once by two fused multiply-adds.  That corrected value can be one
ulp away from fl(x / s), which is what the definition rounds to e4m3; the
claim the kernels rest on is that the e4m3 codes never differ for a group
maximum of at least 2^-90, and that below it they can (so the kernels take
IEEE divisions there).  tests/quotient_check.c enumerates every bf16 group
maximum and every bf16 value up to it (about 10^9 pairs) in IEEE single
precision; its e4m3 encoder is first compared with the oracle's."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
TWO_POW_M90 = 0x1280       # bf16 pattern of 2^-90
SMALLEST_FINITE_RS = 0x03E1  # below this bf16 amax, 1 / (amax / 448) overflows to inf
INF = 0x7F80


@pytest.fixture(scope="module")
def qlib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("quotient") / "libquotient_check.so")
    flags = ["-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC"]
    with open("/proc/cpuinfo") as f:
        if " fma " in f.read():
            flags.append("-mfma")
    subprocess.run(["gcc", *flags, os.path.join(HERE, "quotient_check.c"), "-o", out, "-lm"], check=True)
    lib = ctypes.CDLL(out)
    lib.e4m3_code.argtypes = [ctypes.c_float]
    lib.e4m3_code.restype = ctypes.c_int
    lib.check_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32)]
    lib.check_range.restype = ctypes.c_int64
    return lib


def test_encoder_matches_the_oracle(qlib):
    """Every e4m3 value, every rounding midpoint and its fp32 neighbours, and
    random values over the whole range, encode as the oracle encodes them."""
    table = oracle.e4m3_decode_table()
    pos = np.unique(table[np.isfinite(table) & (table >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids, [464.0, 500.0, 1e6, 2.0 ** -10, 2.0 ** -11]]).astype(np.float32)
    near = np.concatenate([np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0)), pts])
    rng = np.random.default_rng(11)
    rand = (rng.standard_normal(20000) * np.exp2(rng.integers(-14, 10, 20000))).astype(np.float32)
    vals = np.concatenate([near, -near, rand])
    for v in vals:
        assert qlib.e4m3_code(float(v)) == oracle.e4m3_encode(float(v)), float(v)


def test_fast_quotient_codes_exact_above_2_pow_m90(qlib):
    largest = ctypes.c_uint32(0)
    bad = qlib.check_range(TWO_POW_M90, INF, ctypes.byref(largest))
    assert bad == 0, f"{bad} pairs differ, largest amax pattern 0x{largest.value:04x}"


def test_fast_quotient_needs_the_gate(qlib):
    """Below 2^-90 some codes do differ: the gate is needed, and the check
    can see a difference when there is one."""
    largest = ctypes.c_uint32(0)
    bad = qlib.check_range(SMALLEST_FINITE_RS, TWO_POW_M90, ctypes.byref(largest))
    assert bad > 0 and largest.value < TWO_POW_M90
