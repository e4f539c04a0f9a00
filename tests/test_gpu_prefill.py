"""GPU parity of moe_expert_ffn_prefill (bf16 matrix-core path) against the CPU oracle.

The oracle mirrors the path's two bf16 roundings (dequantized weights and h) and sums in
binary64; the GPU accumulates in fp32 on the matrix cores, so the two differ by the fp32
summation order and by the rare h value whose bf16 rounding that order flips. The bar is
rel-L2 <= 1e-3 on both the updated residual and the MoE delta (out - residual).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quantized_routed_expert_router_amd import qmoe, synth, workloads

from gpu_common import check_routing, omat, rel_l2, to_dev

pytestmark = pytest.mark.gpu

REL = 1e-3


def _run_prefill(layer, lg, x, k, residual=None):
    xb = synth.to_bf16_bits(x)
    res = x.copy() if residual is None else residual
    res_d = to_dev(res)
    routing = qmoe.route(to_dev(lg), k)
    qmoe.ffn_prefill(layer, to_dev(xb.view(np.int16)), routing, res_d)
    torch.cuda.synchronize()
    return routing, res_d.cpu().numpy(), xb, res


def _check(out, out_o, res, tokens=None):
    sel = slice(None) if tokens is None else tokens
    r_out = rel_l2(out[sel], out_o)
    r_delta = rel_l2(out[sel] - res[sel], out_o - res[sel])
    print(f"prefill rel-L2: residual {r_out:.2e}, delta {r_delta:.2e}")
    assert r_out <= REL, f"residual out rel-L2 {r_out:.3e}"
    assert r_delta <= REL, f"moe delta rel-L2 {r_delta:.3e}"
    return r_delta


def _small_parity(E, d, f, k, n, bits, logits="normal", seed=0, layer=0):
    w = synth.Workload("small", d, f, E, k, n, bits, logits, seed=seed)
    host = synth.host_layer(w, layer)
    lg, x = synth.layer_inputs(w, layer)
    dev = workloads.layer_from_host(*host, k)
    routing, out, xb, res = _run_prefill(dev, lg, x, k)
    ids, wt = check_routing(lg, k, routing)
    out_o, _ = O.ffn_prefill(*(omat(h) for h in host), E, xb, ids, wt, res)
    return _check(out, out_o, res)


@pytest.mark.parametrize("bits", [4, 2])
def test_prefill_config1_shape(bits):
    # the tiny layer (d=256, f=128, E=8, top-2) over a ragged 300-token chunk
    _small_parity(8, 256, 128, 2, 300, bits)


@pytest.mark.parametrize("E,d,f,k,n,bits", [
    (4, 224, 96, 2, 200, 4),     # d and f not multiples of the 128-wide output tiles
    (16, 128, 160, 1, 513, 4),   # top-1, M-tiles with a 1-row tail
    (6, 256, 128, 6, 40, 2),     # k = E: every token visits every expert
    (64, 384, 256, 8, 33, 4),    # many experts with 0..few rows
    (1, 96, 64, 1, 700, 2),      # one expert: six M-tiles of one GEMM
])
def test_prefill_small_shapes(E, d, f, k, n, bits):
    _small_parity(E, d, f, k, n, bits)


@pytest.mark.parametrize("E,d,f,k,n,bits", [
    (2, 8192, 8192, 1, 2, 4),    # the largest d and f
    (3, 8192, 512, 2, 100, 2),   # the largest d over a ragged chunk
])
def test_prefill_largest_dimensions(E, d, f, k, n, bits):
    _small_parity(E, d, f, k, n, bits, seed=12)


def test_prefill_skewed_routing():
    # one expert takes most of the pairs (Zipf-biased logits, few experts)
    _small_parity(12, 256, 128, 3, 1000, 4, logits="zipf", seed=3)


def test_prefill_zero_expert_contributes_exactly_zero():
    E, d, f, k, n = 4, 128, 64, 1, 257
    w = synth.Workload("small", d, f, E, k, n, 4, "normal")
    host = synth.host_layer(w, 0)
    for h in host:  # scale = min = 0 for every block of every expert
        h.scale_min[:] = 0
    lg, x = synth.layer_inputs(w, 0)
    dev = workloads.layer_from_host(*host, k)
    _, out, _, res = _run_prefill(dev, lg, x, k)
    assert np.array_equal(out, res)


def test_prefill_zero_tokens_is_noop():
    w = synth.config(1)
    host = synth.host_layer(w, 0)
    dev = workloads.layer_from_host(*host, w.k)
    routing = qmoe.Routing.empty(0, w.E, w.k)
    qmoe.route(torch.empty((0, w.E), dtype=torch.float32, device="cuda"), w.k, out=routing)
    res = torch.zeros((1, w.d), dtype=torch.float32, device="cuda")
    qmoe.ffn_prefill(dev, torch.empty((0, w.d), dtype=torch.int16, device="cuda"), routing,
                     res[:0])
    torch.cuda.synchronize()
    assert not res.any()


def test_prefill_deterministic():
    w = synth.Workload("small", 256, 128, 8, 2, 300, 4, "normal")
    host = synth.host_layer(w, 0)
    lg, x = synth.layer_inputs(w, 0)
    dev = workloads.layer_from_host(*host, w.k)
    outs = [_run_prefill(dev, lg, x, w.k)[1] for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("bits", [4, 2])
def test_prefill_stages_match_single_call(bits):
    # moe_expert_ffn_prefill_stages with each stage in a call of its own (the benchmark's
    # instrumented pass issues them so) reproduces moe_expert_ffn_prefill bit for bit on a
    # shared workspace, and stays within the tolerance of the oracle; ragged shape
    w = synth.Workload("staged", 352, 160, 33, 3, 517, bits, "zipf", seed=5)
    host = synth.host_layer(w, 0)
    lg, x = synth.layer_inputs(w, 0)
    dev = workloads.layer_from_host(*host, w.k)
    xb = synth.to_bf16_bits(x)
    xb_d = to_dev(xb.view(np.int16))
    routing = qmoe.route(to_dev(lg), w.k)
    res_a = to_dev(x)
    qmoe.ffn_prefill(dev, xb_d, routing, res_a)
    res_b = to_dev(x)
    ws = qmoe.workspace(dev, w.n, prefill=True, device=xb_d.device)
    for st in (qmoe.PREFILL_PREP, qmoe.PREFILL_GATE_UP, qmoe.PREFILL_DOWN, qmoe.PREFILL_COMBINE):
        qmoe.ffn_prefill(dev, xb_d, routing, res_b, ws=ws, stages=st)
    torch.cuda.synchronize()
    assert torch.equal(res_a, res_b), "staged prefill differs from the single call"
    ids, wt = check_routing(lg, w.k, routing)
    out_o, _ = O.ffn_prefill(*(omat(h) for h in host), w.E, xb, ids, wt, x)
    _check(res_b.cpu().numpy(), out_o, x)


@pytest.fixture(scope="module")
def cfg5():
    w = synth.config(5)
    layer = workloads.device_layer(w, 0)
    lg, x = synth.layer_inputs(w, 0)
    routing, out, xb, res = _run_prefill(layer, lg, x, w.k)
    return w, lg, x, routing, out, xb, res


def test_prefill_config5_routing(cfg5):
    w, lg, _, routing, *_ = cfg5
    check_routing(lg, w.k, routing)
    counts = np.diff(routing.expert_offsets.cpu().numpy())
    assert counts.sum() == w.n * w.k
    assert counts.max() > 8 * counts.mean()  # Zipf: ragged per-expert row counts


PREFILL_TILE_ROWS = 256  # grouped pairs of one expert per M-tile of the prefill GEMMs


def mtile_edge_tokens(offsets: np.ndarray, pair_index: np.ndarray, k: int, rows: int):
    """Tokens holding the first and the last grouped row of every M-tile (runs of `rows`
    consecutive grouped pairs of one expert), and the number of tiles."""
    toks, ntiles = set(), 0
    for e in range(len(offsets) - 1):
        for s in range(int(offsets[e]), int(offsets[e + 1]), rows):
            t_end = min(s + rows, int(offsets[e + 1])) - 1
            toks.add(int(pair_index[s]) // k)
            toks.add(int(pair_index[t_end]) // k)
            ntiles += 1
    return np.array(sorted(toks), np.int32), ntiles


def test_prefill_config5_every_mtile(cfg5):
    # full chunk (8192 tokens, 81,920 pairs) on the GPU; the oracle on every token that
    # holds the first or the last grouped row of an M-tile, so every tile of every expert
    # (and every column tile of those rows) is compared
    w, lg, _, routing, out, xb, res = cfg5
    ids, wt = O.route(lg, w.k)
    off, pidx = O.group(ids, w.E)
    tokens, ntiles = mtile_edge_tokens(off, pidx, w.k, PREFILL_TILE_ROWS)
    print(f"{ntiles} M-tiles, {len(tokens)} tokens compared")
    assert ntiles > 300 and len(tokens) > 500
    host = synth.host_layer(w, 0, experts=np.unique(ids[tokens]))
    out_o, _ = O.ffn_prefill(*(omat(h) for h in host), w.E, xb, ids, wt, res, tokens=tokens)
    _check(out, out_o, res, tokens)


@pytest.fixture(scope="module")
def cfg5_2bit():
    # the 8192-token chunk with 2-bit weights (the same shape, logits and activations)
    import dataclasses

    w = dataclasses.replace(synth.config(5), name="prefill8192_2bit", bits=2)
    layer = workloads.device_layer(w, 0)
    lg, x = synth.layer_inputs(w, 0)
    routing, out, xb, res = _run_prefill(layer, lg, x, w.k)
    return w, lg, x, routing, out, xb, res


def test_prefill_config5_2bit_every_mtile(cfg5_2bit):
    # the 2-bit GEMM instances (half-word codes, row pairs in a code slot) over the full
    # chunk, compared on the tokens at the edges of every M-tile like the 4-bit chunk
    w, lg, _, routing, out, xb, res = cfg5_2bit
    ids, wt = check_routing(lg, w.k, routing)
    off, pidx = O.group(ids, w.E)
    tokens, ntiles = mtile_edge_tokens(off, pidx, w.k, PREFILL_TILE_ROWS)
    assert ntiles > 300 and len(tokens) > 500
    host = synth.host_layer(w, 0, experts=np.unique(ids[tokens]))
    out_o, _ = O.ffn_prefill(*(omat(h) for h in host), w.E, xb, ids, wt, res, tokens=tokens)
    _check(out, out_o, res, tokens)
    assert np.isfinite(out).all() and (out != res).any(axis=1).all()


def test_prefill_config5_untouched_tokens_finite_and_changed(cfg5):
    # every token of the chunk got an MoE update (no tile or row was skipped)
    _, _, _, _, out, _, res = cfg5
    assert np.isfinite(out).all()
    changed = (out != res).any(axis=1)
    assert changed.all(), f"{(~changed).sum()} tokens without an update"


# Pairs per expert spanning every row-group boundary of the M-tiles (1, 2, 4 or 8 groups of
# 32 rows computed in a 256-row tile) and tiles of one expert past the first.
PLANTED_COUNTS = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 513]


@pytest.mark.parametrize("bits", [4, 2])
def test_prefill_row_group_boundaries(bits):
    E, d, f, k = len(PLANTED_COUNTS), 128, 96, 1
    n = sum(PLANTED_COUNTS)
    w = synth.Workload("small", d, f, E, k, n, bits, "normal", seed=5)
    host = synth.host_layer(w, 0)
    _, x = synth.layer_inputs(w, 0)
    # top-1 routing planted through the logits: token t goes to expert owner[t], tokens in
    # a shuffled order so that every tile gathers scattered rows
    owner = np.repeat(np.arange(E), PLANTED_COUNTS)
    np.random.default_rng(5).shuffle(owner)
    lg = (0.1 * np.random.default_rng(6).standard_normal((n, E))).astype(np.float32)
    lg[np.arange(n), owner] = 10.0
    dev = workloads.layer_from_host(*host, k)
    routing, out, xb, res = _run_prefill(dev, lg, x, k)
    ids, wt = check_routing(lg, k, routing)
    assert np.array_equal(ids[:, 0], owner)
    counts = np.diff(routing.expert_offsets.cpu().numpy())
    assert counts.tolist() == PLANTED_COUNTS
    out_o, _ = O.ffn_prefill(*(omat(h) for h in host), E, xb, ids, wt, res)
    _check(out, out_o, res)
