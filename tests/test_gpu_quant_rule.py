"""The GPU's int8 quantizers against blocks that separate the stated rounding rule
(code = round half to even of x times the binary32 reciprocal 127/amax) from x/scale,
exact rounding and (x*127)/amax (tests/golden/quant_rule_cases.json, derived with exact
rational arithmetic). The x quantizer sees the blocks as activations; each h quantizer
(token-major down before and after its weight requests, the separate h quantization
launch, the 32-row gate/up epilogue) sees them as planted SwiGLU outputs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_routed_expert_router_amd import qmoe, synth, workloads

from gpu_common import assert_output_tolerance, omat, to_dev
from quant_rule_layer import expected_h, planted_layer, planted_x, rule_cases

pytestmark = pytest.mark.gpu


def _x_with_cases(n: int, d: int) -> np.ndarray:
    cases = rule_cases()
    v = np.array([c["x"] for c in cases], np.float32)
    nb = d // 32
    x = synth.activations(0, 31, n, d)
    for t in range(n):
        for b in range(nb):
            x[t, 32 * b:32 * b + 32] = v[(t + b) % len(v)] * np.float32(1 + (b % 3))
    return x


@pytest.mark.parametrize("entry", ["ffn_decode", "layer_decode"])
@pytest.mark.parametrize("bits", [4, 2])
def test_x_quantizer_rule_cases(entry, bits):
    E, d, f, k, n = 8, 256, 64, 2, 5
    w = synth.Workload("rule", d, f, E, k, n, bits, "normal")
    host = synth.host_layer(w, 0)
    layer = workloads.layer_from_host(*host, k)
    x = _x_with_cases(n, d)
    lg = synth.logits(0, 0, n, E, "normal")
    dbg = qmoe.debug_buffers(layer, n)
    res = to_dev(x)
    if entry == "ffn_decode":
        qmoe.ffn_decode(layer, to_dev(x), qmoe.route(to_dev(lg), k), res, debug=dbg)
    else:
        qmoe.layer_decode(layer, to_dev(lg), to_dev(x), res, debug=dbg)
    torch.cuda.synchronize()
    q_ref, s_ref = O.quant_act(x)
    # the multipliers 1, 2, 3 scale amax and x alike: 2 is exact, 3 changes the values, so
    # the reference codes come from the pinned oracle; the unscaled blocks from the file
    assert np.array_equal(dbg["xq"].cpu().numpy(), q_ref)
    assert np.array_equal(dbg["xs"].cpu().numpy(), s_ref)
    cases = rule_cases()
    xq = dbg["xq"].cpu().numpy().reshape(n, d // 32, 32)
    for t in range(n):
        for b in range(0, d // 32, 3):  # multiplier 1: the stored codes themselves
            c = cases[(t + b) % len(cases)]
            assert xq[t, b].tolist() == c["q"], (t, b, c["name"])


def _planted_run(E, d, f, k, n, bits, stages=None):
    g, u, dn = planted_layer(E, d, f, bits)
    layer = workloads.layer_from_host(g, u, dn, k)
    x = planted_x(n, d)
    lg = synth.logits(0, 5, n, E, "normal")
    routing = qmoe.route(to_dev(lg), k)
    dbg = qmoe.debug_buffers(layer, n)
    res = to_dev(x)
    if stages is None:
        qmoe.ffn_decode(layer, to_dev(x), routing, res, debug=dbg)
    else:
        ws = qmoe.workspace(layer, n)
        for st in stages:
            qmoe.ffn_decode(layer, to_dev(x), routing, res, ws=ws, debug=dbg, stages=st)
    torch.cuda.synchronize()
    return (g, u, dn), x, routing, dbg, res.cpu().numpy()


# (E, d, f, k, n, bits, stages): which h quantizer runs
H_PATHS = [
    pytest.param(4, 64, 128, 1, 1, 4, None, id="down_tok_8row_after_requests"),
    pytest.param(4, 64, 128, 2, 4, 2, None, id="down_tok_32row_after_requests"),
    pytest.param(4, 4096, 128, 1, 3, 4, None, id="down_tok_before_requests"),
    pytest.param(4, 64, 128, 2, 4, 4, (1, 2, 4, 8), id="hquant_launch"),
    pytest.param(4, 64, 128, 1, 20, 2, None, id="gateup_32row_epilogue"),
]


@pytest.mark.parametrize("E,d,f,k,n,bits,stages", H_PATHS)
def test_h_quantizer_rule_cases(E, d, f, k, n, bits, stages):
    host, x, routing, dbg, out = _planted_run(E, d, f, k, n, bits, stages)
    h_ref, q_ref, s_ref = expected_h(f)
    P = n * k
    h = dbg["h"].cpu().numpy()[:P]
    assert np.array_equal(h, np.broadcast_to(h_ref, h.shape)), "planted h"
    assert np.array_equal(dbg["hq"].cpu().numpy()[:P], np.broadcast_to(q_ref, (P, f)))
    assert np.array_equal(dbg["hs"].cpu().numpy()[:P], np.broadcast_to(s_ref, (P, f // 32)))
    ids = routing.topk_ids.cpu().numpy()
    wt = routing.topk_w.cpu().numpy()
    out_o, _ = O.ffn_decode(*(omat(m) for m in host), E, x, ids, wt, x)
    assert_output_tolerance(out, out_o)
    assert_output_tolerance(out - x, out_o - x, what="moe delta")
