"""A seeded sweep of small random layer shapes through the decode and prefill entry
points against the oracle: routing bit-exact, outputs to the tolerance. Each case prints
its parameters before it runs, so a failure names its case."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_routed_expert_router_amd import qmoe, synth, workloads

from gpu_common import assert_output_tolerance, check_routing, omat, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def _cases(seed, count):
    rng = np.random.default_rng(seed)
    for i in range(count):
        E = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 100, 256, 512]))
        k = int(rng.integers(1, min(E, 12) + 1))
        d = 32 * int(rng.integers(1, 17))
        f = 32 * int(rng.integers(1, 17))
        n = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 9, 17, 40, 65]))
        bits = int(rng.choice([2, 4]))
        logits = str(rng.choice(["normal", "zipf", "uniform"]))
        shared = bool(rng.random() < 0.3)
        yield i, E, k, d, f, n, bits, logits, shared


def _shared_ok(n, k, f):
    nbf = f // 32
    return n <= 8 and n * k <= 64 and k + 1 <= 16 and nbf <= 32 and \
        ((k + 2) // 2) * ((nbf + 7) // 8) <= 18


def test_decode_sweep():
    for i, E, k, d, f, n, bits, kind, shared in _cases(2024, 40):
        shared = shared and _shared_ok(n, k, f)
        print(f"decode case {i}: E={E} k={k} d={d} f={f} n={n} bits={bits} logits={kind} "
              f"shared={shared}", flush=True)
        w = synth.Workload("sweep", d, f, E, k, n, bits, kind, seed=100 + i)
        host = synth.host_layer(w, 0)
        sh = synth.host_shared(w, 0) if shared else None
        lg, x = synth.layer_inputs(w, 0)
        layer = workloads.layer_from_host(*host, k, shared=sh)
        res = to_dev(x)
        r = qmoe.layer_decode(layer, to_dev(lg), to_dev(x), res)
        torch.cuda.synchronize()
        ids, wt = check_routing(lg, k, r)
        out_o, _ = O.ffn_decode(*(omat(h) for h in host), E, x, ids, wt, x,
                                shared=None if sh is None else tuple(omat(h) for h in sh))
        out = res.cpu().numpy()
        assert_output_tolerance(out, out_o, what=f"case {i} residual")
        assert_output_tolerance(out - x, out_o - x, what=f"case {i} delta")


def test_prefill_sweep():
    for i, E, k, d, f, n, bits, kind, _ in _cases(2025, 16):
        n = 4 * n + 3  # longer chunks, ragged
        print(f"prefill case {i}: E={E} k={k} d={d} f={f} n={n} bits={bits} logits={kind}",
              flush=True)
        w = synth.Workload("sweep", d, f, E, k, n, bits, kind, seed=300 + i)
        host = synth.host_layer(w, 0)
        lg, x = synth.layer_inputs(w, 0)
        layer = workloads.layer_from_host(*host, k)
        xb = synth.to_bf16_bits(x)
        res = to_dev(x)
        r = qmoe.route(to_dev(lg), k)
        qmoe.ffn_prefill(layer, to_dev(xb.view(np.int16)), r, res)
        torch.cuda.synchronize()
        ids, wt = check_routing(lg, k, r)
        out_o, _ = O.ffn_prefill(*(omat(h) for h in host), E, xb, ids, wt, x)
        out = res.cpu().numpy()
        assert rel_l2(out, out_o) <= 1e-3, f"case {i} residual"
        assert rel_l2(out - x, out_o - x) <= 1e-3, f"case {i} delta"
