"""GPU parity of the decode layer with an always-active shared expert against the oracle.

The shared expert runs for every token of the window on its own quantized input and is
added to the residual with weight 1 after the routed slots. Bars as for the routed layer:
bit-exact ids, int8 codes and int32 block dots (shared pairs n*k + t included); rel-L2 <=
1e-4 and max-abs <= 2e-3*rms(ref) on the fp32 output.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_routed_expert_router_amd import qmoe, synth, workloads

from gpu_common import (assert_output_tolerance, check_routing, compare_decode_traces, omat,
                        to_dev)

pytestmark = pytest.mark.gpu


def _case(E, d, f, k, n, bits, seed=0, layer=0, logits="normal"):
    w = synth.Workload("shared", d, f, E, k, n, bits, logits, seed=seed)
    return w, synth.host_layer(w, layer), synth.host_shared(w, layer), *synth.layer_inputs(w, layer)


def _parity(w, host, sh, lg, x, layer=None, residual=None, dots=True):
    if layer is None:
        layer = workloads.layer_from_host(*host, w.k, shared=sh)
    routing = qmoe.route(to_dev(lg), w.k)
    ids, wt = check_routing(lg, w.k, routing)
    res = x.copy() if residual is None else residual
    res_d = to_dev(res)
    dbg = qmoe.debug_buffers(layer, x.shape[0])
    if not dots:
        for key in ("gate_dots", "up_dots", "down_dots"):
            dbg.pop(key)
    qmoe.ffn_decode(layer, to_dev(x), routing, res_d, debug=dbg)
    torch.cuda.synchronize()
    out = res_d.cpu().numpy()
    out_o, tr = O.ffn_decode(*(omat(h) for h in host), w.E, x, ids, wt, res, trace=True,
                             shared=tuple(omat(h) for h in sh))
    compare_decode_traces(dbg, tr, host, ids, w.bits, shared_down=sh[2])
    np.testing.assert_allclose(dbg["y"].cpu().numpy(), tr["y"].astype(np.float32), rtol=1e-6,
                               atol=1e-7)
    assert_output_tolerance(out, out_o, what="residual out")
    assert_output_tolerance(out - res, out_o - res, what="moe delta")
    return out, out_o, layer


@pytest.mark.parametrize("E,d,f,k,n,bits", [
    (8, 256, 128, 2, 1, 4),     # one token, two routed slots
    (8, 96, 160, 3, 5, 4),      # f not a multiple of 64; five tokens (eight-pair chunks)
    (6, 160, 96, 2, 7, 2),      # ragged window, 2-bit
    (8, 64, 64, 8, 3, 4),       # k = E
    (16, 128, 64, 1, 8, 4),     # k = 1, the largest window (8 tokens)
    (32, 128, 256, 15, 4, 2),   # 16 slots a token (15 routed + shared), 60 routed pairs
    (16, 64, 1024, 7, 2, 4),    # the largest d_ff (32 blocks), 8 slots a token
    (6, 96, 64, 5, 6, 2),       # 6 tokens: split routed chunks and two shared chunks
    (5, 128, 96, 4, 8, 4),      # 8 tokens: every expert and the shared one in two chunks
])
def test_shared_small_shapes(E, d, f, k, n, bits):
    w, host, sh, lg, x = _case(E, d, f, k, n, bits, seed=3)
    res = synth.normal(3, 9, 0, (n, d))
    _parity(w, host, sh, lg, x, residual=res)


def test_shared_zero_expert_adds_exactly_nothing():
    # a shared expert whose scales and minimums are zero gives y = 0 exactly, so the output
    # equals the layer without it bit for bit (the routed slots are summed in the same order)
    w, host, sh, lg, x = _case(64, 256, 768, 10, 4, 4, seed=4)
    for m in sh:
        m.scale_min[:] = 0
    with_sh = workloads.layer_from_host(*host, w.k, shared=sh)
    without = workloads.layer_from_host(*host, w.k)
    routing = qmoe.route(to_dev(lg), w.k)
    outs = []
    for layer in (with_sh, without):
        res = to_dev(x)
        qmoe.ffn_decode(layer, to_dev(x), routing, res)
        outs.append(res)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_shared_stages_match_one_call():
    # prep, gate/up and down+combine as three calls reproduce the single call bit for bit
    w, host, sh, lg, x = _case(32, 256, 768, 10, 4, 4, seed=5)
    layer = workloads.layer_from_host(*host, w.k, shared=sh)
    routing = qmoe.route(to_dev(lg), w.k)
    ws = qmoe.workspace(layer, w.n)
    res_a = to_dev(x)
    qmoe.ffn_decode(layer, to_dev(x), routing, res_a, ws=ws)
    res_b = to_dev(x)
    for st in (qmoe.DECODE_PREP, qmoe.DECODE_GATE_UP, qmoe.DECODE_DOWN | qmoe.DECODE_COMBINE):
        qmoe.ffn_decode(layer, to_dev(x), routing, res_b, ws=ws, stages=st)
    torch.cuda.synchronize()
    assert torch.equal(res_a, res_b)


@pytest.mark.parametrize("E,d,f,k,n,bits", [
    (8, 256, 128, 2, 1, 4),
    (64, 128, 96, 8, 5, 2),
    (512, 256, 768, 10, 4, 4),
])
def test_shared_layer_decode_matches_two_calls(E, d, f, k, n, bits):
    # the fused entry point (routing, grouping and the layer) against route + decode
    w, host, sh, lg, x = _case(E, d, f, k, n, bits, seed=6, logits="zipf")
    layer = workloads.layer_from_host(*host, w.k, shared=sh)
    lg_d, x_d = to_dev(lg), to_dev(x)
    res_a = x_d.clone()
    r_a = qmoe.route(lg_d, w.k)
    qmoe.ffn_decode(layer, x_d, r_a, res_a)
    res_b = x_d.clone()
    r_b = qmoe.layer_decode(layer, lg_d, x_d, res_b)
    torch.cuda.synchronize()
    for name in ("topk_ids", "topk_w", "expert_offsets"):
        assert torch.equal(getattr(r_a, name), getattr(r_b, name)), name
    assert torch.equal(r_a.pair_index[: n * k], r_b.pair_index[: n * k])
    assert torch.equal(res_a, res_b)
    ids, wt = check_routing(lg, w.k, r_b)
    out_o, _ = O.ffn_decode(*(omat(h) for h in host), w.E, x, ids, wt, x,
                            shared=tuple(omat(h) for h in sh))
    assert_output_tolerance(res_b.cpu().numpy(), out_o)


def test_shared_unsupported_window_raises():
    w, host, sh, lg, x = _case(8, 64, 64, 2, 9, 4, seed=7)
    layer = workloads.layer_from_host(*host, w.k, shared=sh)
    routing = qmoe.route(to_dev(lg), w.k)
    with pytest.raises(qmoe.MoeError) as ei:
        qmoe.ffn_decode(layer, to_dev(x), routing, to_dev(x))
    assert ei.value.status == 2


@pytest.mark.parametrize("T", [1, 4, 5])
def test_shared_full_layer_shape(T):
    # d = 2048, d_ff = 768, 512 experts, top-10 and the shared expert, generated on the GPU
    w = synth.config(2)
    w = synth.Workload(w.name, w.d, w.f, w.E, w.k, T, w.bits, w.logits)
    layer = workloads.device_layer(w, 0, shared=True)
    lg, x = synth.layer_inputs(w, 30 + T)
    ids, _ = O.route(lg, w.k)
    host = synth.host_layer(w, 0, experts=np.unique(ids))
    sh = synth.host_shared(w, 0)
    for dm, hm in zip(layer.shared, sh):
        assert np.array_equal(dm.codes.cpu().numpy().view(np.uint32), hm.codes.reshape(-1))
        assert np.array_equal(dm.scale_min.cpu().numpy().view(np.uint16), hm.scale_min.reshape(-1))
    _parity(w, host, sh, lg, x, layer=layer, dots=(T == 4))
