"""A decode chain captured as a HIP graph replays exactly like the eager launches.

Several layers of the routed-expert layer (moe_layer_decode, residual chained: x aliases
the residual) are captured once into a graph. The graph is then replayed several times,
with eager work of the program and synchronizations between the replays, the residual
reset before each replay; every replay must reproduce the eager residual and routing
bit for bit (the kernels are deterministic and the launches record no memset and no
allocation). The oracle ties the eager chain to the pages' definition elsewhere
(test_gpu_chain); here the graph is compared with the eager path only.
"""
from __future__ import annotations

import pytest
import torch

from quantized_routed_expert_router_amd import qmoe, synth, workloads

from gpu_common import to_dev

pytestmark = pytest.mark.gpu


def _layers(n, bits, count=4):
    out = []
    for l_ in range(count):
        w = synth.Workload("small", 512, 256, 64, 6, n, bits, "zipf", seed=11)
        host = synth.host_layer(w, l_)
        lg, _ = synth.layer_inputs(w, l_)
        out.append((workloads.layer_from_host(*host, w.k), to_dev(lg), w))
    return out


def _run(layers, res, routings, ws):
    # on the current stream (inside a capture: the capturing stream); x is the residual
    for (layer, lg, _), r, wsi in zip(layers, routings, ws):
        qmoe.layer_decode(layer, lg, res, res, routing=r, ws=wsi)


@pytest.mark.parametrize("n,bits", [(4, 4), (3, 2), (16, 4)])
def test_graph_replays_match_eager(n, bits):
    layers = _layers(n, bits)
    w = layers[0][2]
    x0 = to_dev(synth.activations(w.seed, 0, n, w.d))
    ws = [qmoe.workspace(layer, n) for layer, _, _ in layers]

    r_eager = [qmoe.Routing.empty(n, w.E, w.k) for _ in layers]
    res_e = x0.clone()
    _run(layers, res_e, r_eager, ws)
    torch.cuda.synchronize()

    r_graph = [qmoe.Routing.empty(n, w.E, w.k) for _ in layers]
    res_g = x0.clone()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        _run(layers, res_g, r_graph, ws)
    torch.cuda.synchronize()

    for rep in range(3):
        res_g.copy_(x0)
        for r in r_graph:  # stale routing from the previous replay must be overwritten
            r.topk_ids.fill_(-1)
            r.expert_offsets.fill_(-1)
            r.pair_index.fill_(-1)
        scratch = torch.randn(1 << 16, device="cuda")  # eager work between replays
        (scratch * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(res_g, res_e), f"replay {rep}: residual differs"
        for a, b in zip(r_graph, r_eager):
            assert torch.equal(a.topk_ids, b.topk_ids), f"replay {rep}: ids"
            assert torch.equal(a.topk_w, b.topk_w), f"replay {rep}: weights"
            assert torch.equal(a.expert_offsets, b.expert_offsets), f"replay {rep}: offsets"
            assert torch.equal(a.pair_index, b.pair_index), f"replay {rep}: pair index"
