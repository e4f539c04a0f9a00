"""Every stage of every entry point runs on the stream the caller passes (here torch's
current stream). Each call is made on a side stream whose inputs are zero until a copy
that follows a spin kernel on that stream: a stage launched on any other stream would run
before the copy lands and read zeros. Results must equal, bit for bit, the same call made
on the default stream with its inputs in place."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from quantized_routed_expert_router_amd import qmoe, synth, workloads

from gpu_common import on_side_stream, to_dev

pytestmark = pytest.mark.gpu


def _same_routing(a: qmoe.Routing, b: qmoe.Routing, pairs: int):
    for name in ("topk_ids", "topk_w", "expert_offsets"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert torch.equal(a.pair_index[:pairs], b.pair_index[:pairs])


def _layer_decode_case(layer, lg, x, k):
    lg_d = None if lg is None else to_dev(lg)
    x_d = to_dev(x)
    res_ref = x_d.clone()
    r_ref = qmoe.layer_decode(layer, lg_d, x_d, res_ref)
    torch.cuda.synchronize()
    srcs = [x_d, x_d] if lg_d is None else [x_d, x_d, lg_d]

    def call(xs, res, lgs=None):
        return qmoe.layer_decode(layer, lgs, xs, res)

    (xs, res, *_), r = on_side_stream(srcs, call)
    assert torch.equal(res, res_ref), "residual differs from the default-stream call"
    _same_routing(r, r_ref, x.shape[0] * k)


def test_layer_decode_t4_window_on_caller_stream():
    w = synth.config(2)
    layer = workloads.device_layer(w, 0)
    lg, x = synth.layer_inputs(w, 1)
    _layer_decode_case(layer, lg, x, w.k)


@pytest.mark.parametrize("n", [9, 40])
def test_layer_decode_grouped_windows_on_caller_stream(n):
    # 9 tokens: ids path with the second chunk row; 40: routing spread over all CUs, then
    # the grouping launch and the expert-major down with the combine launch
    w = synth.Workload("streams", 256, 128, 64, 6, n, 4, "zipf", seed=70 + n)
    layer = workloads.layer_from_host(*synth.host_layer(w, 0), w.k)
    lg, x = synth.layer_inputs(w, 0)
    _layer_decode_case(layer, lg, x, w.k)


def test_router_projection_and_shared_expert_on_caller_stream():
    w = synth.Workload("streams", 256, 128, 32, 4, 4, 4, "normal", seed=77)
    layer = workloads.layer_from_host(*synth.host_layer(w, 0), w.k, shared=synth.host_shared(w, 0))
    layer.router = workloads.device_router(w, 0)
    x = synth.activations(77, 0, w.n, w.d)
    _layer_decode_case(layer, None, x, w.k)


def test_route_then_ffn_decode_on_caller_stream():
    w = synth.Workload("streams", 320, 96, 48, 5, 21, 2, "uniform", seed=78)
    layer = workloads.layer_from_host(*synth.host_layer(w, 0), w.k)
    lg, x = synth.layer_inputs(w, 0)
    lg_d, x_d = to_dev(lg), to_dev(x)
    res_ref = x_d.clone()
    r_ref = qmoe.route(lg_d, w.k)
    qmoe.ffn_decode(layer, x_d, r_ref, res_ref)
    torch.cuda.synchronize()

    def call(lgs, xs, res):
        r = qmoe.route(lgs, w.k)
        qmoe.ffn_decode(layer, xs, r, res)
        return r

    (_, _, res), r = on_side_stream([lg_d, x_d, x_d], call)
    assert torch.equal(res, res_ref)
    _same_routing(r, r_ref, w.n * w.k)


@pytest.mark.parametrize("bits", [4, 2])
def test_prefill_on_caller_stream(bits):
    w = synth.Workload("streams", 256, 160, 24, 3, 301, bits, "zipf", seed=79 + bits)
    layer = workloads.layer_from_host(*synth.host_layer(w, 0), w.k)
    lg, x = synth.layer_inputs(w, 0)
    xb = to_dev(synth.to_bf16_bits(x).view(np.int16))
    lg_d, x_d = to_dev(lg), to_dev(x)
    res_ref = x_d.clone()
    r_ref = qmoe.route(lg_d, w.k)
    qmoe.ffn_prefill(layer, xb, r_ref, res_ref)
    torch.cuda.synchronize()

    def call(lgs, xbs, res):
        r = qmoe.route(lgs, w.k)
        qmoe.ffn_prefill(layer, xbs, r, res)
        return r

    (_, _, res), r = on_side_stream([lg_d, xb, x_d], call)
    assert torch.equal(res, res_ref)
    _same_routing(r, r_ref, w.n * w.k)
