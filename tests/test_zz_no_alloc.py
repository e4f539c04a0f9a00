"""moe_layer_decode_noalloc (the decode layer on the library's own per-GPU workspace)
against moe_layer_decode with a caller workspace: two calls in a row, the second with a
smaller window, each bit for bit equal to the existing entry point and within the decode
tolerance of the oracle; a window needing more workspace than the array is rejected on
the host."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_routed_expert_router_amd import qmoe, synth, workloads

from gpu_common import assert_output_tolerance, check_routing, omat, on_side_stream, to_dev

pytestmark = pytest.mark.gpu


def _pair(layer, w, lg, x):
    res_a = to_dev(x)
    r_a = qmoe.layer_decode(layer, to_dev(lg), to_dev(x), res_a)
    res_b = to_dev(x)
    r_b = qmoe.Routing.empty(x.shape[0], w.E, w.k)
    qmoe.layer_decode_noalloc(layer, to_dev(lg), to_dev(x), res_b, r_b)
    torch.cuda.synchronize()
    return res_a, r_a, res_b, r_b


def test_noalloc_matches_layer_decode_two_calls():
    w = synth.config(2)
    layer = workloads.device_layer(w, 0)
    for n, inst in ((5, 7), (2, 8)):  # the second call is smaller
        ww = synth.Workload(w.name, w.d, w.f, w.E, w.k, n, w.bits, w.logits)
        lg, x = synth.layer_inputs(ww, inst)
        res_a, r_a, res_b, r_b = _pair(layer, ww, lg, x)
        assert torch.equal(res_a, res_b), f"n={n}: residual differs from moe_layer_decode"
        for name in ("topk_ids", "topk_w", "expert_offsets"):
            assert torch.equal(getattr(r_a, name), getattr(r_b, name)), name
        assert torch.equal(r_a.pair_index[: n * w.k], r_b.pair_index[: n * w.k])
        ids, wt = check_routing(lg, w.k, r_b)
        host = synth.host_layer(w, 0, experts=np.unique(ids))
        out_o, _ = O.ffn_decode(*(omat(h) for h in host), w.E, x, ids, wt, x)
        out = res_b.cpu().numpy()
        assert_output_tolerance(out, out_o)
        assert_output_tolerance(out - x, out_o - x, what="moe delta")


def test_noalloc_larger_batch_then_small_window():
    # a 128-token batch (work-list path, grouping in the routing kernel; 15.7 MiB of
    # workspace at this shape, the largest window the array holds), then one token
    w = synth.Workload("b128", 2048, 768, 512, 10, 128, 2, "uniform")
    layer = workloads.device_layer(w, 2)
    assert qmoe.ffn_workspace_bytes(layer, 128) <= qmoe.NOALLOC_SCRATCH_BYTES
    for n in (128, 1):
        ww = synth.Workload(w.name, w.d, w.f, w.E, w.k, n, w.bits, w.logits)
        lg, x = synth.layer_inputs(ww, 3 + n)
        res_a, r_a, res_b, r_b = _pair(layer, ww, lg, x)
        assert torch.equal(res_a, res_b), f"n={n}"
        assert torch.equal(r_a.expert_offsets, r_b.expert_offsets)


def test_noalloc_rejects_windows_beyond_its_workspace():
    w = synth.config(2)
    layer = workloads.device_layer(w, 0)
    n = 256  # 31.4 MiB of workspace at this shape: more than the array holds
    assert qmoe.ffn_workspace_bytes(layer, n) > qmoe.NOALLOC_SCRATCH_BYTES
    lg = torch.zeros((n, w.E), device="cuda")
    x = torch.zeros((n, w.d), device="cuda")
    res = torch.full((n, w.d), 3.0, device="cuda")
    r = qmoe.Routing.empty(n, w.E, w.k)
    with pytest.raises(qmoe.MoeError) as ei:
        qmoe.layer_decode_noalloc(layer, lg, x, res, r)
    assert ei.value.status == 3  # MOE_ERR_WORKSPACE_TOO_SMALL, nothing enqueued
    torch.cuda.synchronize()
    assert bool((res == 3.0).all())


def test_noalloc_on_caller_stream():
    # the library's own workspace serves a call on a side stream whose inputs arrive behind
    # a spin: every stage on that stream, the result equal to moe_layer_decode's
    w = synth.config(2)
    layer = workloads.device_layer(w, 1)
    lg, x = synth.layer_inputs(w, 5)
    res_a = to_dev(x)
    r_a = qmoe.layer_decode(layer, to_dev(lg), to_dev(x), res_a)
    torch.cuda.synchronize()

    def call(lgs, xs, res):
        r = qmoe.Routing.empty(w.n, w.E, w.k)
        qmoe.layer_decode_noalloc(layer, lgs, xs, res, r)
        return r

    (_, _, res_b), r_b = on_side_stream([to_dev(lg), to_dev(x), to_dev(x)], call)
    assert torch.equal(res_a, res_b)
    for name in ("topk_ids", "topk_w", "expert_offsets"):
        assert torch.equal(getattr(r_a, name), getattr(r_b, name)), name


def test_noalloc_graph_replays_between_eager_calls():
    # the call captured in a HIP graph and replayed three times; before each replay an
    # eager call on a 40-token window leaves its own contents in the shared array, so every
    # replay also shows that a call sets up whatever it needs cleared
    w = synth.config(2)
    layer = workloads.device_layer(w, 0)
    lg, x = synth.layer_inputs(w, 9)
    lg_d, x_d = to_dev(lg), to_dev(x)
    res_e = x_d.clone()
    r_e = qmoe.layer_decode(layer, lg_d, x_d, res_e)
    wo = synth.Workload(w.name, w.d, w.f, w.E, w.k, 40, w.bits, w.logits)
    lg_o, x_o = (to_dev(a) for a in synth.layer_inputs(wo, 4))
    r_o = qmoe.Routing.empty(wo.n, w.E, w.k)

    def other_window():
        res_o = x_o.clone()
        qmoe.layer_decode_noalloc(layer, lg_o, x_o, res_o, r_o)
        return res_o

    other_ref = other_window()  # also resolves the array's address before the capture
    res_g = x_d.clone()
    r_g = qmoe.Routing.empty(w.n, w.E, w.k)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        qmoe.layer_decode_noalloc(layer, lg_d, x_d, res_g, r_g)
    torch.cuda.synchronize()
    for rep in range(3):
        assert torch.equal(other_window(), other_ref), f"eager call before replay {rep}"
        res_g.copy_(x_d)
        r_g.topk_ids.fill_(-1)
        r_g.expert_offsets.fill_(-1)
        r_g.pair_index.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(res_g, res_e), f"replay {rep}: residual"
        for name in ("topk_ids", "topk_w", "expert_offsets"):
            assert torch.equal(getattr(r_g, name), getattr(r_e, name)), f"replay {rep}: {name}"
        assert torch.equal(r_g.pair_index[: w.n * w.k], r_e.pair_index[: w.n * w.k])
