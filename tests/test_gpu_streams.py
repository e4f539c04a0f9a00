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

from gpu_common import SPIN_CYCLES, on_side_stream, to_dev

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


def test_two_streams_at_once():
    # a T=4 decode layer and a prefill chunk, each on its own stream behind a spin of the
    # same length, so their kernels run at the same time; each call has its own
    # workspace, and the results equal the same calls made one after the other
    wd = synth.config(2)
    dlayer = workloads.device_layer(wd, 2)
    dlg, dx = synth.layer_inputs(wd, 2)
    wp = synth.Workload("streams", 2048, 768, 16, 4, 517, 4, "zipf", seed=81)
    player = workloads.layer_from_host(*synth.host_layer(wp, 0), wp.k)
    plg, px = synth.layer_inputs(wp, 0)
    pxb = to_dev(synth.to_bf16_bits(px).view(np.int16))
    dsrc = [to_dev(dlg), to_dev(dx), to_dev(dx)]
    psrc = [to_dev(plg), pxb, to_dev(px)]

    def dcall(lgs, xs, res):
        return qmoe.layer_decode(dlayer, lgs, xs, res)

    def pcall(lgs, xbs, res):
        r = qmoe.route(lgs, wp.k)
        qmoe.ffn_prefill(player, xbs, r, res)
        return r

    ref_d = [t.clone() for t in dsrc]
    rd_ref = dcall(*ref_d)
    ref_p = [t.clone() for t in psrc]
    rp_ref = pcall(*ref_p)
    torch.cuda.synchronize()
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    outs = []
    for s, src, call in zip(streams, (dsrc, psrc), (dcall, pcall)):
        with torch.cuda.stream(s):
            dst = [torch.zeros_like(t) for t in src]
            torch.cuda._sleep(SPIN_CYCLES)
            for a, b in zip(dst, src):
                a.copy_(b)
            outs.append((dst, call(*dst)))
    assert not any(s.query() for s in streams)
    for s in streams:
        s.synchronize()
    (dd, rd), (pd, rp) = outs
    assert torch.equal(dd[2], ref_d[2]), "decode residual"
    assert torch.equal(pd[2], ref_p[2]), "prefill residual"
    _same_routing(rd, rd_ref, wd.n * wd.k)
    _same_routing(rp, rp_ref, wp.n * wp.k)
