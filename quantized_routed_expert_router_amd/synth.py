"""Seeded synthetic inputs for the routed-expert MoE layer (host and device).

The generator draws inputs only; it computes no step of the layer. The same bytes come
out of the host routine (any subset of experts, numpy arrays) and the device routine
(whole matrices written straight into GPU memory), so a layer of 1.5 GB can be created
on the GPU while a checker regenerates only the experts it needs on the host.

Workloads (all seed 0 unless stated; sizes are the layer shapes of the target model):

====  =========================================================================
cfg   recipe
====  =========================================================================
1     d=256, f=128, E=8, top-2, n=1 token, 4-bit; logits N(0,1); x N(0,1)
2     d=2048, f=768, E=512, top-10, n=T=4, 4-bit; logits N(0,1) + Zipf(1.1) bias
3     same shape, 2-bit; logits U[0,1); n = 64 sequences x T, T in {1, 4}
4     48 independent cfg-2 layers, residual chained layer to layer
5     cfg-2 layer, n=8192 prefill tokens, activations bf16 N(0,1), Zipf logits
====  =========================================================================

Weights are N(0, 0.02) before block quantization; the residual stream is the MoE
input itself (x == residual at the start of a layer).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(PKG_DIR, "libqmoe_synth.so")

# tensor ids of the counter-based streams
T_GATE, T_UP, T_DOWN, T_X, T_LOGITS, T_PERM = 1, 2, 3, 4, 5, 6
T_SHARED_GATE, T_SHARED_UP, T_SHARED_DOWN = 7, 8, 9  # the always-active shared expert
T_ROUTER = 10  # router weights

SIGMA_W = 0.02
ZIPF_S = 1.1
# standard deviation of the sum of four uniform bytes (Irwin-Hall, 4 terms)
BYTE_SUM_SD = math.sqrt(4.0 * (256.0 ** 2 - 1.0) / 12.0)

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run quantized_routed_expert_router_amd.build")
        L = ctypes.CDLL(LIB)
        u64, u32, i32, vp, f32 = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_float)
        L.qs_weights_host.argtypes = [u64, u32, u32, i32, i32, i32, i32, f32, vp, i32, vp, vp, i32]
        L.qs_weights_device.argtypes = [u64, u32, u32, i32, i32, i32, i32, f32, vp, vp, vp]
        L.qs_normal_host.argtypes = [u64, u32, u32, u64, f32, vp]
        L.qs_normal_host.restype = None
        L.qs_uniform_host.argtypes = [u64, u32, u32, u64, vp]
        L.qs_uniform_host.restype = None
        L.qs_perm_host.argtypes = [u64, u32, u32, i32, vp]
        L.qs_perm_host.restype = None
        _lib = L
    return _lib


def normal_scale(sigma: float) -> np.float32:
    return np.float32(sigma / BYTE_SUM_SD)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- small host tensors

def normal(seed: int, tensor: int, layer: int, shape, sigma: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    lib().qs_normal_host(seed, tensor, layer, n, normal_scale(sigma), _p(out))
    return out.reshape(shape)


def uniform(seed: int, tensor: int, layer: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    lib().qs_uniform_host(seed, tensor, layer, n, _p(out))
    return out.reshape(shape)


def perm(seed: int, tensor: int, layer: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().qs_perm_host(seed, tensor, layer, n, _p(out))
    return out


def zipf_bias(seed: int, layer: int, E: int, s: float = ZIPF_S) -> np.ndarray:
    """Per-expert popularity bias -s*ln(rank), rank = 1 + seeded permutation of 0..E-1."""
    rank = 1.0 + perm(seed, T_PERM, layer, E).astype(np.float64)
    return -s * np.log(rank)


def logits(seed: int, layer: int, n: int, E: int, kind: str) -> np.ndarray:
    if kind == "normal":
        return normal(seed, T_LOGITS, layer, (n, E))
    if kind == "zipf":
        z = normal(seed, T_LOGITS, layer, (n, E)).astype(np.float64)
        return (z + zipf_bias(seed, layer, E)[None, :]).astype(np.float32)
    if kind == "uniform":
        return uniform(seed, T_LOGITS, layer, (n, E))
    raise ValueError(kind)


def activations(seed: int, layer: int, n: int, d: int) -> np.ndarray:
    return normal(seed, T_X, layer, (n, d))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- packed weights

@dataclass
class HostMatrix:
    """Packed matrix for all E experts in host memory (experts not generated are zero):
    codes uint32 [E][cols/32][rows][bits], scale_min uint16 [E][cols/32][rows][2]."""
    codes: np.ndarray
    scale_min: np.ndarray
    rows: int
    cols: int
    bits: int


def empty_matrix(E: int, rows: int, cols: int, bits: int) -> HostMatrix:
    nb = cols // 32
    return HostMatrix(np.zeros((E, nb, rows, bits), np.uint32),
                      np.zeros((E, nb, rows, 2), np.uint16), rows, cols, bits)


def fill_matrix_host(M: HostMatrix, seed: int, layer: int, tensor: int, experts=None,
                     sigma: float = SIGMA_W, nthreads: int = 0) -> HostMatrix:
    E = M.codes.shape[0]
    ex = None if experts is None else np.ascontiguousarray(np.unique(experts), np.int32)
    rc = lib().qs_weights_host(seed, tensor, layer, E, M.rows, M.cols, M.bits, normal_scale(sigma),
                               None if ex is None else _p(ex), 0 if ex is None else len(ex),
                               _p(M.codes), _p(M.scale_min), nthreads)
    if rc != 0:
        raise ValueError("qs_weights_host: bad arguments")
    return M


def fill_matrix_device(codes_ptr: int, sm_ptr: int, seed: int, layer: int, tensor: int, E: int,
                       rows: int, cols: int, bits: int, stream: int = 0,
                       sigma: float = SIGMA_W) -> None:
    rc = lib().qs_weights_device(seed, tensor, layer, E, rows, cols, bits, normal_scale(sigma),
                                 ctypes.c_void_p(codes_ptr), ctypes.c_void_p(sm_ptr),
                                 ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"qs_weights_device failed ({rc})")


def matrix_words(E: int, rows: int, cols: int, bits: int) -> int:
    return E * (cols // 32) * rows * bits


def matrix_halves(E: int, rows: int, cols: int) -> int:
    return E * (cols // 32) * rows * 2


# ---------------------------------------------------------------- workloads

@dataclass
class Workload:
    name: str
    d: int
    f: int
    E: int
    k: int
    n: int
    bits: int
    logits: str
    layers: int = 1
    prefill: bool = False
    seed: int = 0
    extra: dict = field(default_factory=dict)


def config(cfg: int, T: int = 4, experts: int | None = None) -> Workload:
    """Workload `cfg`; `experts` replaces the expert count of configurations 2-5 (256: the
    pruned "Coder" model, 256 of every layer's 512 experts kept, still 10 active)."""
    w = _config(cfg, T)
    if experts is not None and experts != w.E:
        if cfg == 1:
            raise ValueError("the expert count of configuration 1 is fixed")
        w.name = w.name.replace(f"_e{w.E}_", f"_e{experts}_")
        w.E = experts
    return w


def _config(cfg: int, T: int) -> Workload:
    if cfg == 1:
        return Workload("tiny_d256_f128_e8_top2_t1", 256, 128, 8, 2, 1, 4, "normal")
    if cfg == 2:
        return Workload("decode_t4_d2048_f768_e512_top10_4bit", 2048, 768, 512, 10, 4, 4, "zipf")
    if cfg == 3:
        return Workload(f"decode_b64xt{T}_d2048_f768_e512_top10_2bit", 2048, 768, 512, 10, 64 * T,
                        2, "uniform", extra=dict(T=T, sequences=64))
    if cfg == 4:
        return Workload("chain48_t4_d2048_f768_e512_top10_4bit", 2048, 768, 512, 10, 4, 4, "zipf",
                        layers=48)
    if cfg == 5:
        return Workload("prefill8192_d2048_f768_e512_top10_4bit_bf16", 2048, 768, 512, 10, 8192, 4,
                        "zipf", prefill=True)
    raise ValueError(cfg)


def expert_bytes(d: int, f: int, bits: int) -> int:
    """Packed bytes of one expert: 3 matrices of f*d weights at bits/8 + 4 B per 32 weights."""
    return 3 * f * d * (bits + 1) // 8


def host_layer(w: Workload, layer: int, experts=None, nthreads: int = 0):
    """(gate, up, down) HostMatrix for `layer` with only `experts` generated (all if None)."""
    g = fill_matrix_host(empty_matrix(w.E, w.f, w.d, w.bits), w.seed, layer, T_GATE, experts,
                         nthreads=nthreads)
    u = fill_matrix_host(empty_matrix(w.E, w.f, w.d, w.bits), w.seed, layer, T_UP, experts,
                         nthreads=nthreads)
    dn = fill_matrix_host(empty_matrix(w.E, w.d, w.f, w.bits), w.seed, layer, T_DOWN, experts,
                          nthreads=nthreads)
    return g, u, dn


def host_shared(w: Workload, layer: int, nthreads: int = 0):
    """(gate, up, down) HostMatrix of the layer's shared expert (one expert, E = 1)."""
    g = fill_matrix_host(empty_matrix(1, w.f, w.d, w.bits), w.seed, layer, T_SHARED_GATE,
                         nthreads=nthreads)
    u = fill_matrix_host(empty_matrix(1, w.f, w.d, w.bits), w.seed, layer, T_SHARED_UP,
                         nthreads=nthreads)
    dn = fill_matrix_host(empty_matrix(1, w.d, w.f, w.bits), w.seed, layer, T_SHARED_DOWN,
                          nthreads=nthreads)
    return g, u, dn


def host_router(w: Workload, layer: int) -> np.ndarray:
    """Router weights of the layer: bf16 bits [E][d] of N(0, 1/d) values, so that the
    logits of N(0, 1) inputs are about N(0, 1)."""
    return to_bf16_bits(normal(w.seed, T_ROUTER, layer, (w.E, w.d), sigma=1.0 / math.sqrt(w.d)))


def layer_inputs(w: Workload, layer: int):
    """Router logits [n,E] fp32 and MoE input x [n,d] fp32 of one layer instance."""
    lg = logits(w.seed, layer, w.n, w.E, w.logits)
    x = activations(w.seed, layer, w.n, w.d)
    return lg, x
