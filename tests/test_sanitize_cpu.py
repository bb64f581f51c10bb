"""Address and undefined-behaviour sanitizer runs of the host code (CPU only).

* The oracle (oracle/oracle.c) built with gcc -fsanitize=address,undefined and
  driven over every function on small inputs (tests/sanitize/oracle_driver.c).
* The library's host code (argument validation, launch plans, scratch
  bookkeeping) built with the sanitizers on the host side only, device code
  unchanged, and driven without a GPU (tests/sanitize/api_driver.cpp): invalid
  arguments must give the documented status, valid ones stop at the device
  check, and the split-K plans must stay within their bounds.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), which fails
the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_gemm_linears_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
LIB_SOURCES = ["api", "quant", "prune24", "gemm_dense", "gemm_sparse", "workspace", "fixed_scratch"]


def _run(cmd, env=None, timeout=600):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")
    res = _run([exe], env=env)
    assert "oracle sanitizer driver: ok" in res.stdout


def test_library_host_code_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ are not available")
    objs = []
    procs = []
    for name in LIB_SOURCES:
        obj = str(tmp_path / (name + ".o"))
        objs.append(obj)
        # sanitizers on the host side only (-Xarch_host before each); the device
        # code is compiled as in the product build
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, name + ".hip"), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for cmd, p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{' '.join(cmd)}\n{err}"
    exe = str(tmp_path / "api_driver")
    # host link (no .hip source on this line)
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", os.path.join(HERE, "api_driver.cpp"), *objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # the HIP runtime's own allocations are not this test's subject
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    res = _run([exe], env=env)
    assert "library host sanitizer driver: ok" in res.stdout
