"""Host-side checks of the benchmark's step objects (no GPU)."""
from __future__ import annotations

import gc
import weakref

import pytest
import torch

import bench
from quantized_routed_expert_router_amd import qmoe


def _cpu_layer():
    mk = lambda r, c: qmoe.QMatrix(torch.zeros(64, dtype=torch.int32),  # noqa: E731
                                   torch.zeros(32, dtype=torch.int16), r, c, 4)
    return qmoe.Layer(64, 32, 4, 2, mk(32, 64), mk(32, 64), mk(64, 32))


@pytest.mark.parametrize("cls", [bench.Step, bench.PrefillStep])
def test_step_keeps_its_weights_alive(cls):
    # the step keeps raw device pointers (C structs); the tensors behind them must live as
    # long as the step, or freed memory is handed to the next layer instance (instances
    # then alias) and releasing the allocator's cache unmaps it under the step
    layer = _cpu_layer()
    probe = weakref.ref(layer.down.codes)
    lg = torch.zeros((2, 4))
    routing = qmoe.Routing.empty(2, 4, 2, device="cpu")

    class Q:  # the step only needs route_workspace from the binding here
        @staticmethod
        def route_workspace(n, E, k):
            return None

    step = cls(Q, layer, lg, torch.zeros((2, 64)), torch.zeros((2, 64)), routing,
               torch.zeros(16, dtype=torch.uint8))
    del layer
    gc.collect()
    assert probe() is not None, "the step dropped its layer's weight tensors"
    assert step.layer_s.down.codes == probe().data_ptr()
    # the step's launch methods are still methods (not shadowed by stored attributes)
    for name in ("full", "stages"):
        assert callable(getattr(step, name))
    if cls is bench.Step:
        assert callable(step.layer) and callable(step.gate_up)


def test_percentiles_and_host_cores():
    p = bench.percentiles([0.010, 0.020, 0.030, 0.040, 0.050])
    assert (p["p10"], p["p50"], p["p90"]) == (14.0, 30.0, 46.0) and p["steps"] == 5
    logical, allowed, physical = bench.host_cores()
    assert 1 <= physical <= allowed <= logical


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys

    res = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "exactly one" in res.stderr


def test_source_ids_track_the_library_sources(tmp_path, monkeypatch):
    ids = bench.source_ids()
    h = ids["library_sources_sha256_16"]
    assert len(h) == 16 and int(h, 16) >= 0
    assert ids["git_sha"] is None or len(ids["git_sha"]) == 40
    # the hash covers the header and the HIP sources: a copy of the tree with one source
    # byte changed hashes differently, and an unchanged copy (no git) the same
    import shutil

    root = tmp_path / "tree"
    for sub in ("include", "quantized_routed_expert_router_amd/csrc"):
        shutil.copytree(bench.os.path.join(bench.ROOT, sub), root / sub)
    monkeypatch.setattr(bench, "ROOT", str(root))
    same = bench.source_ids()
    assert same["library_sources_sha256_16"] == h and same["git_sha"] is None
    src = root / "quantized_routed_expert_router_amd/csrc/qmoe_prefill.hip"
    src.write_bytes(src.read_bytes() + b"\n")
    assert bench.source_ids()["library_sources_sha256_16"] != h
