"""The C ABI without a GPU: exported symbols, status strings, workspace sizes and the
argument checks that reject a call before anything is enqueued (no kernel is launched:
every call here is invalid, or has zero tokens)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from quantized_routed_expert_router_amd import qmoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")

INVALID, UNSUPPORTED, WS_SMALL, OK = 1, 2, 3, 0
FAKE = 0x7f0000000000  # a 256-byte aligned address that is never dereferenced here


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"^[a-z][\w\s\*]*?\b(moe_\w+)\s*\(", text, re.M)


def test_every_declared_function_is_exported():
    names = header_functions()
    assert set(names) == set(qmoe.EXPORTS)
    for name in names:
        assert hasattr(qmoe.lib, name), name


def test_status_strings():
    for code, name in qmoe.STATUS.items():
        assert qmoe.status_string(code) == name
    assert qmoe.status_string(99) == "MOE_ERR_UNKNOWN"


def _mat(rows, cols, bits, codes=FAKE, sm=FAKE + 0x100000):
    return qmoe._QMatrix(codes, sm, rows, cols, bits)


def _layer(d=256, f=128, E=8, k=2, bits=4, **over):
    L = qmoe._Layer(d, f, E, k, _mat(f, d, bits), _mat(f, d, bits), _mat(d, f, bits))
    for key, val in over.items():
        setattr(L, key, val)
    return L


def _routing():
    return qmoe._Routing(FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000, FAKE + 0x500000)


def _decode(L, n=4, x=FAKE + 0x600000, res=FAKE + 0x700000, ws=FAKE + 0x800000, ws_bytes=1 << 30,
            routing=None):
    r = routing if routing is not None else _routing()
    return qmoe.lib.moe_expert_ffn_decode(ctypes.byref(L) if L is not None else None, x, n,
                                          ctypes.byref(r), res, ws, ws_bytes, None, None)


def test_route_argument_checks():
    r = _routing()
    route = lambda n, E, k, rr=r: qmoe.lib.moe_route(FAKE, n, E, k, ctypes.byref(rr), None, 0,
                                                      None)  # noqa: E731
    assert route(-1, 8, 2) == INVALID
    assert route(4, 0, 1) == INVALID
    assert route(4, 8, 0) == INVALID
    assert route(4, 8, 9) == INVALID
    assert route(4, 2048, 2) == INVALID  # more than 1024 experts
    assert route(4, 512, 65) == INVALID  # more than 64 slots
    assert route(70000, 8, 2) == INVALID
    bad = qmoe._Routing(FAKE, 0, FAKE, FAKE)
    assert route(4, 8, 2, bad) == INVALID
    assert qmoe.lib.moe_route(None, 4, 8, 2, ctypes.byref(r), None, 0, None) == INVALID


def test_decode_argument_checks():
    assert _decode(None) == INVALID
    assert _decode(_layer(d=100)) == INVALID                  # d not a multiple of 32
    assert _decode(_layer(k=9)) == INVALID                    # k > E
    assert _decode(_layer(bits=3)) == UNSUPPORTED
    L = _layer()
    L.down = _mat(256, 128, 2)
    assert _decode(L) == UNSUPPORTED                          # mixed bit widths
    L = _layer()
    L.gate = _mat(128, 256, 4, codes=FAKE + 4)                # codes not 16-byte aligned
    assert _decode(L) == INVALID
    L = _layer()
    L.up = _mat(100, 256, 4)                                  # wrong rows
    assert _decode(L) == INVALID
    assert _decode(_layer(), n=513) == INVALID                # beyond the decode limit
    assert _decode(_layer(), n=-1) == INVALID
    assert _decode(_layer(), x=FAKE + 0x600004) == INVALID    # x not 16-byte aligned
    assert _decode(_layer(), ws=FAKE + 0x800010) == INVALID   # ws not 256-byte aligned
    assert _decode(_layer(), res=FAKE + 0x600100) == INVALID  # partial overlap with x
    need = qmoe.lib.moe_ffn_workspace_bytes(ctypes.byref(_layer()), 4, 0)
    assert need > 0
    assert _decode(_layer(), ws_bytes=need - 1) == WS_SMALL
    assert _decode(_layer(), ws=FAKE + 0x600000 - 256) == INVALID  # ws overlaps x


def test_zero_tokens_enqueue_nothing():
    assert _decode(_layer(), n=0, x=0, res=0, ws=0, ws_bytes=0) == OK


def test_workspace_bytes_grow_with_tokens():
    L = _layer(d=2048, f=768, E=512, k=10)
    sizes = [qmoe.lib.moe_ffn_workspace_bytes(ctypes.byref(L), n, 0) for n in (1, 4, 64, 512)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    assert all(s % 256 == 0 for s in sizes)
    assert qmoe.lib.moe_route_workspace_bytes(4, 512, 10) == 0
    # multi-workgroup grouping: one 512-expert histogram per 2048 pairs
    assert qmoe.lib.moe_route_workspace_bytes(8192, 512, 10) == 40 * 512 * 4
    assert qmoe.lib.moe_route_workspace_bytes(409, 512, 10) == 0  # 4090 pairs: one workgroup
    r = _routing()
    assert qmoe.lib.moe_route(FAKE, 8192, 512, 10, ctypes.byref(r), None, 0, None) == WS_SMALL
    assert qmoe.lib.moe_route(FAKE, 8192, 512, 10, ctypes.byref(r), FAKE + 0x10, 1 << 20,
                              None) == INVALID  # workspace not 256-byte aligned


def _prefill(L, n=300, x=FAKE + 0x600000, res=FAKE + 0x700000, ws=FAKE + 0x10000000,
             ws_bytes=1 << 34, routing=None):
    r = routing if routing is not None else _routing()
    return qmoe.lib.moe_expert_ffn_prefill(ctypes.byref(L) if L is not None else None, x, n,
                                           ctypes.byref(r), res, ws, ws_bytes, None)


def test_prefill_argument_checks():
    # every call is rejected before launch: each one breaks exactly one rule
    assert _prefill(None) == INVALID
    assert _prefill(_layer(d=100)) == INVALID
    assert _prefill(_layer(bits=3)) == UNSUPPORTED
    L = _layer()
    L.down = _mat(256, 128, 2)
    assert _prefill(L) == UNSUPPORTED                           # mixed bit widths
    assert _prefill(_layer(), n=8193) == INVALID                # beyond the prefill limit
    assert _prefill(_layer(), n=-1) == INVALID
    assert _prefill(_layer(), x=FAKE + 0x600008) == INVALID     # x not 16-byte aligned
    assert _prefill(_layer(), res=FAKE + 0x600000 + 16) == INVALID  # residual overlaps x
    assert _prefill(_layer(), res=FAKE + 0x700004) == INVALID  # residual not 16-byte aligned
    assert _prefill(_layer(), ws=FAKE + 0x10000010) == INVALID  # ws not 256-byte aligned
    assert _prefill(_layer(), routing=qmoe._Routing(FAKE, 0, FAKE, FAKE)) == INVALID
    need = qmoe.lib.moe_ffn_workspace_bytes(ctypes.byref(_layer()), 300, 1)
    assert need > 0
    assert _prefill(_layer(), ws_bytes=need - 1) == WS_SMALL
    assert _prefill(_layer(), ws=FAKE + 0x700000 - 256) == INVALID  # ws overlaps residual
    assert _prefill(_layer(), n=0, x=0, res=0, ws=0, ws_bytes=0) == OK
    stages = lambda st: qmoe.lib.moe_expert_ffn_prefill_stages(  # noqa: E731
        ctypes.byref(_layer()), FAKE + 0x600000, 300, ctypes.byref(_routing()), FAKE + 0x700000,
        FAKE + 0x10000000, 1 << 34, st, None)
    assert stages(0) == INVALID
    assert stages(16) == INVALID


def test_prefill_workspace_bytes():
    L = _layer(d=2048, f=768, E=512, k=10)
    sizes = [qmoe.lib.moe_ffn_workspace_bytes(ctypes.byref(L), n, 1) for n in (1, 64, 8192)]
    assert sizes == sorted(sizes) and sizes[0] > 0 and all(s % 256 == 0 for s in sizes)
    # h (bf16) and the pair outputs (fp32) dominate: (2 f + 4 d) bytes per pair
    P = 8192 * 10
    assert P * (2 * 768 + 4 * 2048) <= sizes[-1] < P * (2 * 768 + 4 * 2048 + 64) + (1 << 20)
    assert qmoe.lib.moe_ffn_workspace_bytes(ctypes.byref(L), 8193, 1) == 0


@pytest.mark.parametrize("name", ["libqmoe.so", "libqmoe_synth.so"])
def test_built_for_gfx950(name):
    path = os.path.join(os.path.dirname(qmoe.LIB_PATH), name)
    data = open(path, "rb").read()
    assert b"gfx950" in data


def test_layer_decode_argument_checks():
    r = _routing()
    call = lambda logits, n=4, stages=None: (  # noqa: E731
        qmoe.lib.moe_layer_decode(ctypes.byref(_layer()), logits, FAKE + 0x600000, n,
                                  ctypes.byref(r), FAKE + 0x700000, FAKE + 0x800000, 1 << 30,
                                  None, None)
        if stages is None else
        qmoe.lib.moe_layer_decode_stages(ctypes.byref(_layer()), logits, FAKE + 0x600000, n,
                                         ctypes.byref(r), FAKE + 0x700000, FAKE + 0x800000,
                                         1 << 30, None, stages, None))
    assert call(None) == INVALID                     # logits missing
    assert call(FAKE + 0x900000, n=513) == INVALID   # beyond the decode limit
    assert call(FAKE + 0x900002) == INVALID          # logits not 4-byte aligned
    assert call(FAKE + 0x900000, stages=0) == INVALID
    assert call(FAKE + 0x900000, stages=16) == INVALID
    L = _layer(bits=3)
    assert qmoe.lib.moe_layer_decode(ctypes.byref(L), FAKE + 0x900000, FAKE + 0x600000, 4,
                                     ctypes.byref(r), FAKE + 0x700000, FAKE + 0x800000, 1 << 30,
                                     None, None) == UNSUPPORTED


def _with_shared(L, bits=4, base=FAKE + 0x20000000):
    d, f = L.d_model, L.d_ff
    L.shared_gate = _mat(f, d, bits, codes=base, sm=base + 0x1000000)
    L.shared_up = _mat(f, d, bits, codes=base + 0x2000000, sm=base + 0x3000000)
    L.shared_down = _mat(d, f, bits, codes=base + 0x4000000, sm=base + 0x5000000)
    return L


def test_shared_expert_argument_checks():
    # a shared expert is validated like the routed matrices, and the decode entry points take
    # it only on their small-window path; every call here is rejected before launch
    L = _with_shared(_layer())
    L.shared_up = _mat(100, 256, 4)                                      # wrong rows
    assert _decode(L) == INVALID
    L = _with_shared(_layer())
    L.shared_down = _mat(256, 128, 2)                                    # other bit width
    assert _decode(L) == INVALID
    L = _with_shared(_layer())
    L.shared_gate = _mat(128, 256, 4, codes=FAKE + 4)                    # codes misaligned
    assert _decode(L) == INVALID
    assert _decode(_with_shared(_layer()), n=9) == UNSUPPORTED           # window above 8
    assert _decode(_with_shared(_layer(E=512, k=10)), n=7) == UNSUPPORTED  # 70 pairs
    assert _decode(_with_shared(_layer(E=512, k=16)), n=1) == UNSUPPORTED  # 17 slots a token
    assert _decode(_with_shared(_layer(f=2048)), n=1) == UNSUPPORTED     # d_ff above 1024
    assert _decode(_with_shared(_layer()), n=0, x=0, res=0, ws=0, ws_bytes=0) == OK
    # the down stage without the combine (expert-major down) has no shared slot
    r = _routing()
    st = lambda stages: qmoe.lib.moe_expert_ffn_decode_stages(  # noqa: E731
        ctypes.byref(_with_shared(_layer())), FAKE + 0x600000, 4, ctypes.byref(r),
        FAKE + 0x700000, FAKE + 0x800000, 1 << 30, None, stages, None)
    assert st(qmoe.DECODE_DOWN) == UNSUPPORTED
    assert st(qmoe.DECODE_COMBINE) == UNSUPPORTED
    assert st(qmoe.DECODE_PREP | qmoe.DECODE_GATE_UP | qmoe.DECODE_DOWN) == UNSUPPORTED
    # the prefill entry points have no shared expert
    assert _prefill(_with_shared(_layer())) == UNSUPPORTED
    # the workspace holds n more pairs
    a = qmoe.lib.moe_ffn_workspace_bytes(ctypes.byref(_layer(d=2048, f=768, E=512, k=10)), 4, 0)
    b = qmoe.lib.moe_ffn_workspace_bytes(
        ctypes.byref(_with_shared(_layer(d=2048, f=768, E=512, k=10))), 4, 0)
    assert b >= a + 4 * (768 + 4 * 2048)  # per pair: h codes, fp32 pair outputs
    need = b
    assert _decode(_with_shared(_layer(d=2048, f=768, E=512, k=10)), ws_bytes=need - 1) == WS_SMALL


def test_router_argument_checks():
    r = _routing()
    call = lambda L, logits=None, n=4: qmoe.lib.moe_layer_decode(  # noqa: E731
        ctypes.byref(L), logits, FAKE + 0x600000, n, ctypes.byref(r), FAKE + 0x700000,
        FAKE + 0x800000, 1 << 30, None, None)
    assert call(_layer()) == INVALID                        # no logits and no router rows
    L = _layer()
    L.router_w = FAKE + 0x30000008                          # router rows not 16-byte aligned
    assert call(L, FAKE + 0x900000) == INVALID
    # the workspace holds the projected logits
    base = _layer(d=2048, f=768, E=512, k=10)
    withr = _layer(d=2048, f=768, E=512, k=10)
    withr.router_w = FAKE + 0x30000000
    a = qmoe.lib.moe_ffn_workspace_bytes(ctypes.byref(base), 4, 0)
    b = qmoe.lib.moe_ffn_workspace_bytes(ctypes.byref(withr), 4, 0)
    assert b >= a + 4 * 512 * 4
    assert qmoe.lib.moe_layer_decode(ctypes.byref(withr), None, FAKE + 0x600000, 4,
                                     ctypes.byref(r), FAKE + 0x700000, FAKE + 0x1000000, b - 1,
                                     None, None) == WS_SMALL
