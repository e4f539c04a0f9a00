"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU.

* The CPU oracle, compiled with gcc into a C driver that calls every one of its entry
  points (with traces, token subsets, a shared expert, ties and an all-zero block).
* The library's host side (argument checks and workspace sizing of the C ABI, in the
  ABI source file), compiled with the sanitizers on its host code, linked with stand-ins
  for the kernel launchers (which abort if reached) and driven from C with size queries
  at the extremes of every argument and calls that are rejected, or accepted with
  nothing to enqueue, before any GPU work.

A sanitizer report aborts the program (no recovery), so each driver must exit 0.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_routed_expert_router_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if res.returncode != 0:
        raise AssertionError(f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "c", "oracle_sanitize_driver.c"),
          "-o", str(exe), "-lm"])
    res = _run([str(exe)], env=ENV, timeout=300)
    assert "oracle driver ok" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr


def test_abi_host_side_under_asan_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("the ROCm compilers are not available")
    # the ABI file (argument checks, workspace sizing, entry points) with the kernel
    # launchers replaced by stand-ins that abort if reached; sanitizers on the host side
    objs = []
    for src in (os.path.join(CSRC, "qmoe.hip"), os.path.join(ROOT, "tests", "c", "launch_stubs.hip")):
        obj = tmp_path / (os.path.basename(src) + ".o")
        _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", str(obj)])
        objs.append(str(obj))
    drv = tmp_path / "abi_driver.o"
    _run([CLANG, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "c", "abi_sanitize_driver.c"), "-o", str(drv)])
    exe = tmp_path / "abi_driver"
    _run([CLANGXX, "-fsanitize=address,undefined", str(drv), *objs, "-L/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    # the HIP runtime's own start-up allocations are not this library's: leak checks off
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    res = _run([str(exe)], env=env, timeout=300)
    assert "abi driver: 0 mismatches" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
