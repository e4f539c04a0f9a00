"""Helpers shared by the GPU parity tests: run the oracle and the library on the same
seeded inputs and compare them."""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as O
from quantized_routed_expert_router_amd import qmoe, synth, workloads

from refmath import unpack_codes


def omat(h: synth.HostMatrix) -> O.Matrix:
    return O.Matrix(h.codes, h.scale_min, h.rows, h.cols, h.bits)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def assert_output_tolerance(got, ref, rel=1e-4, abs_frac=2e-3, what="output"):
    """rel-L2 <= rel and max-abs <= abs_frac * rms(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(got, ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    mx = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert r <= rel, f"{what}: rel-L2 {r:.3e} > {rel:.1e}"
    assert mx <= abs_frac * rms + 1e-30, f"{what}: max-abs {mx:.3e} > {abs_frac:.1e}*rms {rms:.3e}"
    return r, mx


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_routing(lg: np.ndarray, k: int, routing: qmoe.Routing):
    """Bit-exact ids, offsets and pair lists; weights within 1 ulp of the oracle's."""
    E = lg.shape[1]
    ids_o, w_o = O.route(lg, k)
    off_o, pidx_o = O.group(ids_o, E)
    ids = routing.topk_ids.cpu().numpy()
    w = routing.topk_w.cpu().numpy()
    assert np.array_equal(ids, ids_o)
    np.testing.assert_array_max_ulp(w, w_o, maxulp=1)
    assert np.array_equal(routing.expert_offsets.cpu().numpy(), off_o)
    n = lg.shape[0]
    assert np.array_equal(routing.pair_index.cpu().numpy()[: n * k], pidx_o)
    return ids_o, w_o


def compare_decode_traces(dbg: dict, tr: dict, layer_host, ids: np.ndarray, bits: int,
                          shared_down=None):
    """Bit-exact checks of the integer intermediates; near-exact float intermediates.

    h is a binary64 sum on both sides rounded to fp32, so it agrees except where the two
    summation orders straddle an fp32 rounding boundary; an h code may then legitimately
    differ. Where h agrees, the codes must agree; everywhere, the GPU codes must be the
    quantization of the GPU's own h, and the GPU down dots must be the exact dots of the
    GPU's codes. With a shared expert (`shared_down` its down HostMatrix), pairs n*k + t
    are token t's shared pairs.
    """
    g_h, u_h, d_h = layer_host
    k = ids.shape[1]
    xq = dbg["xq"].cpu().numpy()
    assert np.array_equal(xq, tr["xq"]), "x codes"
    assert np.array_equal(dbg["xs"].cpu().numpy(), tr["xs"]), "x scales"
    if "gate_dots" in dbg:
        assert np.array_equal(dbg["gate_dots"].cpu().numpy(), tr["gate_dots"]), "gate dots"
        assert np.array_equal(dbg["up_dots"].cpu().numpy(), tr["up_dots"]), "up dots"
    g = dbg["g"].cpu().numpy()
    u = dbg["u"].cpu().numpy()
    np.testing.assert_allclose(g, tr["g"].astype(np.float32), rtol=2e-7, atol=1e-30)
    np.testing.assert_allclose(u, tr["u"].astype(np.float32), rtol=2e-7, atol=1e-30)
    h = dbg["h"].cpu().numpy()
    np.testing.assert_array_max_ulp(h, tr["h"], maxulp=2)
    hq = dbg["hq"].cpu().numpy()
    hs = dbg["hs"].cpu().numpy()
    q_self, s_self = O.quant_act(h)
    assert np.array_equal(hq, q_self) and np.array_equal(hs, s_self), "h codes of GPU h"
    same_h = (h == tr["h"]).reshape(h.shape[0], -1, 32).all(axis=2)  # per 32-block
    hq_b = hq.reshape(hq.shape[0], -1, 32)
    ref_b = tr["hq"].reshape(hq.shape[0], -1, 32)
    assert np.array_equal(hq_b[same_h], ref_b[same_h]), "h codes where h agrees"
    frac_diff = 1.0 - same_h.mean()
    if "down_dots" in dbg:
        dd = dbg["down_dots"].cpu().numpy()
        Qd = unpack_codes(d_h.codes, bits)
        Qs = None if shared_down is None else unpack_codes(shared_down.codes, bits)[0]
        d, f = d_h.rows, d_h.cols
        P = ids.size
        for p in range(hq.shape[0]):
            W = Qd[ids.ravel()[p]] if p < P else Qs
            ref = np.einsum("rbi,bi->rb", W.reshape(d, f // 32, 32),
                            hq[p].astype(np.int64).reshape(f // 32, 32))
            assert np.array_equal(dd[p], ref), f"down dots pair {p}"
    return frac_diff


def host_layer_for(w: synth.Workload, layer: int, ids: np.ndarray):
    return synth.host_layer(w, layer, experts=np.unique(ids))


def run_decode(layer: qmoe.Layer, lg: np.ndarray, x: np.ndarray, k: int, debug: bool = False,
               residual: np.ndarray | None = None):
    """Route + decode on the GPU; returns (routing, out residual np, debug dict)."""
    lg_d = to_dev(lg)
    x_d = to_dev(x)
    res_d = x_d.clone() if residual is None else to_dev(residual)
    routing = qmoe.route(lg_d, k)
    dbg = qmoe.debug_buffers(layer, x.shape[0]) if debug else None
    qmoe.ffn_decode(layer, x_d, routing, res_d, debug=dbg)
    torch.cuda.synchronize()
    return routing, res_d.cpu().numpy(), dbg


def device_layer_matches_host(dev: qmoe.Layer, host, experts, E: int):
    """The GPU-filled packed bytes equal the host generator's for the given experts."""
    for dm, hm in zip((dev.gate, dev.up, dev.down), host):
        nb = dm.cols // 32
        cw, sw = nb * dm.rows * dm.bits, nb * dm.rows * 2
        for e in experts:
            e = int(e)
            codes = dm.codes[e * cw:(e + 1) * cw].cpu().numpy().view(np.uint32)
            sm = dm.scale_min[e * sw:(e + 1) * sw].cpu().numpy().view(np.uint16)
            assert np.array_equal(codes, hm.codes[e].reshape(-1)), f"codes of expert {e}"
            assert np.array_equal(sm, hm.scale_min[e].reshape(-1)), f"scale/min of expert {e}"


SPIN_CYCLES = 50_000_000  # about 20 ms of the spin kernel


def on_side_stream(srcs, call):
    """Zero-filled copies of the device tensors `srcs`, filled on a side stream after a
    spin; `call(*copies)` is made on that stream and its result returned once it is done."""
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dst = [torch.zeros_like(t) for t in srcs]
        torch.cuda._sleep(SPIN_CYCLES)
        for a, b in zip(dst, srcs):
            a.copy_(b)
        out = call(*dst)
    # every call was enqueued while the spin still ran: a stage on another stream would
    # have found zeros, and the binding waited on nothing
    assert not s.query(), "the side stream finished before the calls were enqueued"
    s.synchronize()
    return dst, out
