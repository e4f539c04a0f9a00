"""Synthetic layers and inputs in device memory, for the tests and the benchmark.

Weights come from the seeded generator (`synth`), written either straight into device
memory by its GPU fill (large layers) or copied from host arrays (small layers and
hand-modified cases). Nothing here computes a step of the layer.
"""
from __future__ import annotations

import numpy as np
import torch

from . import qmoe, synth


def _stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def device_matrix(w: synth.Workload, layer: int, tensor: int, rows: int, cols: int,
                  device="cuda") -> qmoe.QMatrix:
    codes = torch.empty(synth.matrix_words(w.E, rows, cols, w.bits), dtype=torch.int32,
                        device=device)
    sm = torch.empty(synth.matrix_halves(w.E, rows, cols), dtype=torch.int16, device=device)
    synth.fill_matrix_device(codes.data_ptr(), sm.data_ptr(), w.seed, layer, tensor, w.E, rows,
                             cols, w.bits, stream=_stream_handle())
    return qmoe.QMatrix(codes, sm, rows, cols, w.bits)


def device_router(w: synth.Workload, layer: int, device="cuda") -> torch.Tensor:
    """The layer's router weights (bf16 bits [E][d], int16 storage) in device memory."""
    return torch.from_numpy(synth.host_router(w, layer).view(np.int16)).to(device)


def device_layer(w: synth.Workload, layer: int, device="cuda", shared: bool = False,
                 router: bool = False) -> qmoe.Layer:
    """All E experts of one layer instance generated on the GPU (and optionally its shared
    expert and router weights)."""
    return qmoe.Layer(w.d, w.f, w.E, w.k,
                      device_matrix(w, layer, synth.T_GATE, w.f, w.d, device),
                      device_matrix(w, layer, synth.T_UP, w.f, w.d, device),
                      device_matrix(w, layer, synth.T_DOWN, w.d, w.f, device),
                      device_shared(w, layer, device) if shared else None,
                      device_router(w, layer, device) if router else None)


def device_shared(w: synth.Workload, layer: int, device="cuda"):
    """(gate, up, down) of the layer's shared expert (one expert) generated on the GPU."""
    one = synth.Workload(w.name, w.d, w.f, 1, w.k, w.n, w.bits, w.logits, seed=w.seed)
    return (device_matrix(one, layer, synth.T_SHARED_GATE, w.f, w.d, device),
            device_matrix(one, layer, synth.T_SHARED_UP, w.f, w.d, device),
            device_matrix(one, layer, synth.T_SHARED_DOWN, w.d, w.f, device))


def matrix_from_host(m: synth.HostMatrix, device="cuda") -> qmoe.QMatrix:
    codes = torch.from_numpy(m.codes.reshape(-1).view(np.int32)).to(device)
    sm = torch.from_numpy(m.scale_min.reshape(-1).view(np.int16)).to(device)
    return qmoe.QMatrix(codes, sm, m.rows, m.cols, m.bits)


def layer_from_host(gate: synth.HostMatrix, up: synth.HostMatrix, down: synth.HostMatrix, k: int,
                    device="cuda", shared=None) -> qmoe.Layer:
    """Layer from host matrices; `shared`: optional (gate, up, down) HostMatrix, E = 1."""
    E = gate.codes.shape[0]
    sh = None if shared is None else tuple(matrix_from_host(m, device) for m in shared)
    return qmoe.Layer(gate.cols, gate.rows, E, k, matrix_from_host(gate, device),
                      matrix_from_host(up, device), matrix_from_host(down, device), sh)


def matrix_to_host(m: qmoe.QMatrix, E: int) -> synth.HostMatrix:
    nb = m.cols // 32
    codes = m.codes.cpu().numpy().view(np.uint32).reshape(E, nb, m.rows, m.bits)
    sm = m.scale_min.cpu().numpy().view(np.uint16).reshape(E, nb, m.rows, 2)
    return synth.HostMatrix(codes, sm, m.rows, m.cols, m.bits)
