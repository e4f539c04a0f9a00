"""The Python binding's own argument checks, without a GPU: a tensor of the wrong dtype,
layout, shape or extent, or one in host memory, is rejected with ValueError before its
pointer reaches the library (a bad pointer or extent would otherwise reach a kernel)."""
from __future__ import annotations

import pytest
import torch

from quantized_routed_expert_router_amd import qmoe


def _mat(E, rows, cols, bits=4, words=None, halves=None):
    nb = cols // 32
    codes = torch.zeros(E * nb * rows * bits if words is None else words, dtype=torch.int32)
    sm = torch.zeros(E * nb * rows * 2 if halves is None else halves, dtype=torch.int16)
    return qmoe.QMatrix(codes, sm, rows, cols, bits)


def _layer(E=4, d=64, f=32, k=2, **over):
    parts = dict(gate=_mat(E, f, d), up=_mat(E, f, d), down=_mat(E, d, f))
    parts.update(over)
    return qmoe.Layer(d, f, E, k, parts["gate"], parts["up"], parts["down"])


def _routing(n, E, k, **over):
    r = qmoe.Routing.empty(n, E, k, device="cpu")
    for key, v in over.items():
        setattr(r, key, v)
    return r


def _decode(layer=None, x=None, res=None, routing=None, n=3, logits=None, fn="ffn_decode"):
    layer = layer or _layer()
    x = torch.zeros(n, layer.d_model) if x is None else x
    res = torch.zeros(n, layer.d_model) if res is None else res
    routing = routing or _routing(n, layer.n_experts, layer.top_k)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    if fn == "ffn_decode":
        qmoe.ffn_decode(layer, x, routing, res, ws=ws)
    else:
        lg = torch.zeros(n, layer.n_experts) if logits is None else logits
        qmoe.layer_decode(layer, lg, x, res, routing=routing, ws=ws)


def test_host_tensors_are_rejected():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        _decode()
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        qmoe.route(torch.zeros(3, 8), 2, out=_routing(3, 8, 2))


@pytest.mark.parametrize("fn", ["ffn_decode", "layer_decode"])
def test_activation_dtype_shape_layout(fn):
    with pytest.raises(ValueError, match="x: dtype"):
        _decode(x=torch.zeros(3, 64, dtype=torch.float64), fn=fn)
    with pytest.raises(ValueError, match="residual: shape"):
        _decode(res=torch.zeros(3, 32), fn=fn)
    with pytest.raises(ValueError, match="x: must be contiguous"):
        _decode(x=torch.zeros(64, 3).t(), fn=fn)
    with pytest.raises(ValueError, match="x: expected"):
        _decode(x=torch.zeros(192), fn=fn)


def test_logits_shape():
    with pytest.raises(ValueError, match="logits: shape"):
        _decode(logits=torch.zeros(3, 5), fn="layer_decode")
    with pytest.raises(ValueError, match="logits: dtype"):
        qmoe.route(torch.zeros(3, 8, dtype=torch.float16), 2)
    with pytest.raises(ValueError, match="logits: expected"):
        qmoe.route(torch.zeros(8), 2)


def test_routing_extents():
    n, E, k = 3, 4, 2
    with pytest.raises(ValueError, match="topk_ids"):
        _decode(routing=_routing(n, E, k, topk_ids=torch.zeros(n * k - 1, dtype=torch.int32)))
    with pytest.raises(ValueError, match="topk_w: dtype"):
        _decode(routing=_routing(n, E, k, topk_w=torch.zeros(n, k, dtype=torch.float64)))
    with pytest.raises(ValueError, match="expert_offsets"):
        _decode(routing=_routing(n, E, k, expert_offsets=torch.zeros(E, dtype=torch.int32)))
    with pytest.raises(ValueError, match="pair_index"):
        _decode(routing=_routing(n, E, k, pair_index=torch.zeros(1, dtype=torch.int32)))


def test_weight_extents():
    E, d, f = 4, 64, 32
    short = _mat(E, f, d, words=E * 2 * f * 4 - 1)
    with pytest.raises(ValueError, match="gate.codes"):
        _decode(layer=_layer(gate=short))
    short_sm = _mat(E, d, f, halves=E * d * 2 - 2)
    with pytest.raises(ValueError, match="down.scale_min"):
        _decode(layer=_layer(down=short_sm))
    with pytest.raises(ValueError, match="up: 64x32"):
        _decode(layer=_layer(up=_mat(E, d, f)))
    with pytest.raises(ValueError, match="bad shape"):
        _decode(layer=_layer(gate=_mat(E, f, d, bits=3)))


def test_prefill_checks():
    layer = _layer()
    r = _routing(3, 4, 2)
    res = torch.zeros(3, 64)
    with pytest.raises(ValueError, match="x_bf16: dtype"):
        qmoe.ffn_prefill(layer, torch.zeros(3, 64), r, res)
    with pytest.raises(ValueError, match="x_bf16: shape"):
        qmoe.ffn_prefill(layer, torch.zeros(3, 32, dtype=torch.int16), r, res)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        qmoe.ffn_prefill(layer, torch.zeros(3, 64, dtype=torch.int16), r, res,
                         ws=torch.zeros(16, dtype=torch.uint8))
