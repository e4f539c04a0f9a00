"""GPU parity of the 48-layer residual chain (one T=4 verify window through every layer).

Each layer reads the residual stream as its MoE input and adds its routed-expert output
into it in place (x aliases residual), so layer l+1 sees layer l's result: the serial
residual chain of the Strata explainer, section "Expert cache". Router logits are given
per layer (attention and the router projection are outside the path).

Two checks per run:
  * per layer, the oracle evaluated on the GPU's own input residual of that layer
    matches the GPU's output residual within the decode tolerance (each layer checked
    in isolation, no compounding);
  * the oracle chained on its own through all 48 layers matches the GPU's final
    residual within the same tolerance.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_routed_expert_router_amd import qmoe, synth, workloads

from gpu_common import assert_output_tolerance, check_routing, omat, to_dev

pytestmark = pytest.mark.gpu


def test_chain48_decode_matches_oracle():
    w = synth.config(4)
    assert w.layers == 48
    x0 = synth.activations(w.seed, 0, w.n, w.d)
    res = to_dev(x0)
    ws = None
    per_layer_in, per_layer_out, routings = [], [], []
    for l_ in range(w.layers):
        layer = workloads.device_layer(w, l_)
        lg = synth.logits(w.seed, l_, w.n, w.E, w.logits)
        routing = qmoe.route(to_dev(lg), w.k)
        if ws is None:
            ws = qmoe.workspace(layer, w.n)
        per_layer_in.append(res.cpu().numpy())
        qmoe.ffn_decode(layer, res, routing, res, ws=ws)  # x is the residual stream
        per_layer_out.append(res.cpu().numpy())
        torch.cuda.synchronize()
        routings.append((lg, routing))
        del layer  # 1.5 GB per layer; the GPU holds one at a time here
    torch.cuda.synchronize()

    chain = x0.copy()
    worst = 0.0
    for l_ in range(w.layers):
        lg, routing = routings[l_]
        ids, wt = check_routing(lg, w.k, routing)
        host = synth.host_layer(w, l_, experts=np.unique(ids))
        mats = [omat(h) for h in host]
        xin = per_layer_in[l_]
        out_o, _ = O.ffn_decode(*mats, w.E, xin, ids, wt, xin)
        got = per_layer_out[l_]
        r, _ = assert_output_tolerance(got, out_o, what=f"layer {l_} residual")
        assert_output_tolerance(got - xin, out_o - xin, what=f"layer {l_} moe delta")
        worst = max(worst, r)
        chain, _ = O.ffn_decode(*mats, w.E, chain, ids, wt, chain)
        del host, mats
    final = per_layer_out[-1]
    r_final, _ = assert_output_tolerance(final, chain, what="chained residual after 48 layers")
    assert_output_tolerance(final - x0, chain - x0, what="48-layer moe delta")
    print(f"chain48: worst per-layer rel-L2 {worst:.2e}, final chained rel-L2 {r_final:.2e}")
