"""Compile the gfx950 shared libraries of this package in-tree with hipcc.

Two libraries are produced next to this file:

* ``libqmoe.so``       - the MoE layer library (C ABI declared in ``include/qmoe.h``);
* ``libqmoe_synth.so`` - the seeded input generator (host and device fill routines).

Run ``python -m quantized_routed_expert_router_amd.build`` or call :func:`build`.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code; -ffp-contract=off keeps every
# floating-point multiply and add separately rounded unless a kernel calls fma itself.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]

LIBS = {
    "libqmoe.so": ["qmoe.hip", "qmoe_route.hip", "qmoe_decode.hip", "qmoe_prefill.hip"],
    "libqmoe_synth.so": ["synth.hip"],
}


def _compile(out_name: str, sources: list[str], verbose: bool) -> None:
    out = os.path.join(PKG_DIR, out_name)
    tmp = out + ".tmp"
    srcs = [os.path.join(CSRC, s) for s in sources]
    cmd = [HIPCC, *COMMON_FLAGS, f"-I{os.path.join(REPO_DIR, 'include')}", f"-I{CSRC}", *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name and says so; drop that line
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {out_name}:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> None:
    for name, sources in LIBS.items():
        _compile(name, sources, verbose)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
