"""The boundary from C: a strict C99 program built against include/qmoe.h and linked
against libqmoe.so agrees with the Python binding on every struct layout and gets the
documented statuses for calls rejected on the host (no GPU call is made)."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import pytest

from quantized_routed_expert_router_amd import qmoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe_output(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    out = tmp_path_factory.mktemp("cprobe") / "abi_probe"
    libdir = os.path.dirname(qmoe.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_probe.c"),
           "-L", libdir, "-lqmoe", f"-Wl,-rpath,{libdir}", "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(out)], check=True, capture_output=True, text=True, timeout=60)
    lines = {}
    for line in res.stdout.splitlines():
        key, _, val = line.rpartition(" ")
        lines[key] = val
    return lines, res.stdout


def test_struct_layouts_match_binding(probe_output):
    lines, _ = probe_output
    assert int(lines["sizeof moe_qmatrix"]) == ctypes.sizeof(qmoe._QMatrix)
    assert int(lines["sizeof moe_layer"]) == ctypes.sizeof(qmoe._Layer)
    assert int(lines["offsetof moe_layer.shared_gate"]) == qmoe._Layer.shared_gate.offset
    assert int(lines["offsetof moe_layer.router_w"]) == qmoe._Layer.router_w.offset
    assert int(lines["sizeof moe_routing"]) == ctypes.sizeof(qmoe._Routing)
    assert int(lines["sizeof moe_debug"]) == ctypes.sizeof(qmoe._Debug)


def test_rejected_calls_from_c(probe_output):
    _, out = probe_output
    assert ("status MOE_ERR_INVALID_ARGUMENT MOE_ERR_INVALID_ARGUMENT "
            "MOE_ERR_INVALID_ARGUMENT") in out
    assert "workspace 0" in out
