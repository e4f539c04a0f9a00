"""GPU parity of the layer that projects its own router logits (moe_layer_decode without
logits, the layer carrying bf16 router rows) against the oracle.

The logits are binary64 sums rounded to fp32 on both sides, in different orders, so they
agree to the last bit nearly always and within one ulp always. The routing is a decision
taken on fp32 logits: the GPU's expert ids and weights must be exactly those the oracle's
router selects from the GPU's own logits. The layer output is checked against the oracle
layer on that routing, to the decode tolerance (rel-L2 <= 1e-4, max-abs <= 2e-3*rms).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_routed_expert_router_amd import qmoe, synth, workloads

from gpu_common import assert_output_tolerance, check_routing, omat, to_dev

pytestmark = pytest.mark.gpu


def _check_logits(got: np.ndarray, ref: np.ndarray):
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(got.astype(np.float64) - ref) <= np.maximum(ulp, 1e-12)), "logits"
    return float(np.mean(got == ref))


def _run(w, layer, x, host=None, layer_id=0):
    """Project + route + layer on the GPU (debug pass and fast passes); checks against the
    oracle. Returns the fraction of logits equal to the oracle's to the bit."""
    n = x.shape[0]
    W = layer.router.cpu().numpy().view(np.uint16)
    x_d = to_dev(x)
    # debug pass: logits and routing
    dbg = qmoe.debug_buffers(layer, n)
    res1 = x_d.clone()
    r1 = qmoe.layer_decode(layer, None, x_d, res1, debug=dbg)
    torch.cuda.synchronize()
    lg_gpu = dbg["logits"].cpu().numpy()
    same = _check_logits(lg_gpu, O.router_logits(W, x))
    ids, wt = check_routing(lg_gpu, w.k, r1)  # the oracle's router on the GPU's logits
    # fast passes: projecting, and routing the same logits handed in, agree bit for bit
    res2 = x_d.clone()
    r2 = qmoe.layer_decode(layer, None, x_d, res2)
    res3 = x_d.clone()
    r3 = qmoe.layer_decode(layer, to_dev(lg_gpu), x_d, res3)
    torch.cuda.synchronize()
    assert torch.equal(res2, res3)
    for name in ("topk_ids", "topk_w", "expert_offsets"):
        assert torch.equal(getattr(r2, name), getattr(r3, name)), name
        assert torch.equal(getattr(r1, name), getattr(r2, name)), name
    if host is None:
        host = synth.host_layer(w, layer_id, experts=np.unique(ids))
    out_o, _ = O.ffn_decode(*(omat(h) for h in host), w.E, x, ids, wt, x)
    for out in (res1.cpu().numpy(), res2.cpu().numpy()):
        assert_output_tolerance(out, out_o)
        assert_output_tolerance(out - x, out_o - x, what="moe delta")
    return same


def _small_layer(E, d, f, k, n, bits, seed):
    w = synth.Workload("router", d, f, E, k, n, bits, "normal", seed=seed)
    host = synth.host_layer(w, 0)
    layer = workloads.layer_from_host(*host, w.k)
    layer.router = workloads.device_router(w, 0)
    x = synth.activations(seed, 0, n, d)
    return w, host, layer, x


@pytest.mark.parametrize("E,d,f,k,n,bits", [
    (8, 256, 128, 2, 1, 4),     # the tiny shape, one token
    (37, 96, 64, 3, 5, 2),      # E not a multiple of the workgroup's 4 experts; d < 512
    (16, 4096, 64, 2, 3, 4),    # two staged column chunks
    (64, 128, 96, 8, 9, 4),     # three token groups, the last ragged
    (32, 64, 64, 4, 16, 2),     # the largest window routed inside the first layer kernel
    (32, 64, 64, 4, 17, 4),     # one token more: separate routing kernels
    (32, 64, 64, 4, 64, 2),     # 64 tokens, 256 pairs grouped by one workgroup
    (100, 160, 64, 3, 300, 4),  # a batch
])
def test_router_small_shapes(E, d, f, k, n, bits):
    w, host, layer, x = _small_layer(E, d, f, k, n, bits, seed=E + n)
    _run(w, layer, x, host=host)


def test_router_stages_match_one_call():
    w, host, layer, x = _small_layer(64, 256, 128, 6, 4, 4, seed=8)
    x_d = to_dev(x)
    ws = qmoe.workspace(layer, w.n)
    res_a = x_d.clone()
    qmoe.layer_decode(layer, None, x_d, res_a, ws=ws)
    res_b = x_d.clone()
    r = qmoe.Routing.empty(w.n, w.E, w.k)
    for st in (qmoe.DECODE_PREP, qmoe.DECODE_GATE_UP, qmoe.DECODE_DOWN | qmoe.DECODE_COMBINE):
        qmoe.layer_decode(layer, None, x_d, res_b, routing=r, ws=ws, stages=st)
    torch.cuda.synchronize()
    assert torch.equal(res_a, res_b)


def test_router_separate_down_and_combine_stages():
    # projected logits, then down and combine as separate stages: the expert-major down
    # builds its work list from the grouping the gate/up stage wrote; same result as the
    # single call up to the combine's summation order
    w, host, layer, x = _small_layer(64, 256, 128, 6, 4, 4, seed=10)
    x_d = to_dev(x)
    ws = qmoe.workspace(layer, w.n)
    res_a = x_d.clone()
    r_a = qmoe.layer_decode(layer, None, x_d, res_a, ws=ws)
    res_b = x_d.clone()
    r_b = qmoe.Routing.empty(w.n, w.E, w.k)
    for st in (qmoe.DECODE_PREP, qmoe.DECODE_GATE_UP, qmoe.DECODE_DOWN, qmoe.DECODE_COMBINE):
        qmoe.layer_decode(layer, None, x_d, res_b, routing=r_b, ws=ws, stages=st)
    torch.cuda.synchronize()
    assert torch.equal(r_a.topk_ids, r_b.topk_ids)
    np.testing.assert_allclose(res_b.cpu().numpy(), res_a.cpu().numpy(), rtol=1e-6, atol=1e-7)


def test_router_without_weights_needs_logits():
    w, host, layer, x = _small_layer(8, 64, 64, 2, 2, 4, seed=9)
    layer.router = None
    with pytest.raises(qmoe.MoeError) as ei:
        qmoe.layer_decode(layer, None, to_dev(x), to_dev(x))
    assert ei.value.status == 1


@pytest.mark.parametrize("E,T", [(512, 4), (256, 4), (512, 1), (512, 5)])
def test_router_full_layer_shape(E, T):
    # d = 2048, d_ff = 768, top-10, 4-bit, weights and router rows generated per layer
    w = synth.config(2, experts=E)
    w = synth.Workload(w.name, w.d, w.f, w.E, w.k, T, w.bits, w.logits)
    layer = workloads.device_layer(w, 5, router=True)
    x = synth.activations(0, 40 + T, T, w.d)
    same = _run(w, layer, x, layer_id=5)
    assert same >= 0.99  # equal to the bit nearly always


def test_router_with_shared_expert():
    # both optional parts at once: logits projected from x, then the routed experts and the
    # shared expert (weight 1, after the routed slots)
    w = synth.Workload("router_shared", 256, 128, 32, 4, 3, 4, "normal", seed=14)
    host = synth.host_layer(w, 0)
    sh = synth.host_shared(w, 0)
    layer = workloads.layer_from_host(*host, w.k, shared=sh)
    layer.router = workloads.device_router(w, 0)
    x = synth.activations(14, 0, w.n, w.d)
    x_d = to_dev(x)
    dbg = qmoe.debug_buffers(layer, w.n)
    res = x_d.clone()
    r = qmoe.layer_decode(layer, None, x_d, res, debug=dbg)
    torch.cuda.synchronize()
    lg_gpu = dbg["logits"].cpu().numpy()
    _check_logits(lg_gpu, O.router_logits(layer.router.cpu().numpy().view(np.uint16), x))
    ids, wt = check_routing(lg_gpu, w.k, r)
    out_o, _ = O.ffn_decode(*(omat(h) for h in host), w.E, x, ids, wt, x,
                            shared=tuple(omat(h) for h in sh))
    assert_output_tolerance(res.cpu().numpy(), out_o)
    assert_output_tolerance(res.cpu().numpy() - x, out_o - x, what="moe delta")


def test_router_layer_in_graph_replays():
    # the projecting layer captured in a HIP graph: every replay equals the eager call
    w, host, layer, x = _small_layer(64, 256, 128, 6, 4, 4, seed=15)
    x_d = to_dev(x)
    ws = qmoe.workspace(layer, w.n)
    r = qmoe.Routing.empty(w.n, w.E, w.k)
    ref = x_d.clone()
    qmoe.layer_decode(layer, None, x_d, ref, routing=r, ws=ws)
    torch.cuda.synchronize()
    res = x_d.clone()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        qmoe.layer_decode(layer, None, x_d, res, routing=r, ws=ws)
    for _ in range(3):
        res.copy_(x_d)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(res, ref)
