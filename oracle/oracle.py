"""numpy-facing wrapper of the CPU oracle (``qmoe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke check and the
benchmark's CPU-baseline leg. It never imports the GPU library, and the GPU library never
imports it. Inputs are plain numpy arrays in the packed layout the input generator writes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmoe_oracle.c")
LIB = os.path.join(HERE, "liborc.so")

_lib = None


def build(verbose: bool = False) -> None:
    """Compile the oracle with gcc (plain C99, OpenMP over independent token-expert pairs)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout + res.stderr)
    os.replace(LIB + ".tmp", LIB)


class _Matrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale_min", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("bits", ctypes.c_int32)]


class _Trace(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("xq", "xs", "gate_dots", "up_dots", "g", "u", "h", "hq", "hs", "down_dots", "y")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        L.orc_route.argtypes = [vp, i32, i32, i32, vp, vp]
        L.orc_group.argtypes = [vp, i32, i32, i32, vp, vp]
        L.orc_router_logits.argtypes = [vp, vp, i32, i32, i32, vp]
        L.orc_quant_act.argtypes = [vp, ctypes.c_int64, vp, vp]
        L.orc_quant_act.restype = None
        L.orc_weight.argtypes = [ctypes.POINTER(_Matrix), i32, i32, i32]
        L.orc_weight.restype = ctypes.c_double
        L.orc_weight_bf16.argtypes = [ctypes.POINTER(_Matrix), i32, i32, i32]
        L.orc_weight_bf16.restype = ctypes.c_uint16
        L.orc_ffn_decode.argtypes = [ctypes.POINTER(_Matrix)] * 3 + [i32] * 4 + [
            vp, i32, vp, vp, vp, vp, i32, vp, ctypes.POINTER(_Trace), i32] + [
            ctypes.POINTER(_Matrix)] * 3
        L.orc_ffn_prefill.argtypes = [ctypes.POINTER(_Matrix)] * 3 + [i32] * 4 + [
            vp, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32]
        L.orc_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


@dataclass
class Matrix:
    """One packed matrix for all experts: codes uint32 [E][cols/32][rows][bits],
    scale_min uint16 [E][cols/32][rows][2]."""
    codes: np.ndarray
    scale_min: np.ndarray
    rows: int
    cols: int
    bits: int

    def _struct(self) -> _Matrix:
        assert self.codes.dtype == np.uint32 and self.codes.flags.c_contiguous
        assert self.scale_min.dtype == np.uint16 and self.scale_min.flags.c_contiguous
        return _Matrix(self.codes.ctypes.data, self.scale_min.ctypes.data, self.rows, self.cols,
                       self.bits)


def threads(n: int = 0) -> int:
    return int(lib().orc_threads(n))


def route(logits: np.ndarray, k: int):
    logits = _c(logits, np.float32)
    n, E = logits.shape
    ids = np.zeros((n, k), np.int32)
    w = np.zeros((n, k), np.float32)
    if lib().orc_route(_p(logits), n, E, k, _p(ids), _p(w)) != 0:
        raise ValueError("orc_route: bad arguments")
    return ids, w


def router_logits(W_bf16: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Router logits [n, E] fp32 of x [n, d] against bf16 rows W_bf16 [E, d] (uint16)."""
    W = _c(W_bf16, np.uint16)
    x = _c(x, np.float32)
    n, d = x.shape
    E = W.shape[0]
    assert W.shape == (E, d)
    out = np.zeros((n, E), np.float32)
    if lib().orc_router_logits(_p(W), _p(x), n, d, E, _p(out)) != 0:
        raise ValueError("orc_router_logits: bad arguments")
    return out


def group(ids: np.ndarray, E: int):
    ids = _c(ids, np.int32)
    n, k = ids.shape
    offsets = np.zeros(E + 1, np.int32)
    pair_index = np.zeros(n * k, np.int32)
    if lib().orc_group(_p(ids), n, k, E, _p(offsets), _p(pair_index)) != 0:
        raise ValueError("orc_group: bad arguments")
    return offsets, pair_index


def quant_act(x: np.ndarray):
    """int8 block-32 quantization of the last axis; returns (codes int8, scales fp32)."""
    x = _c(x, np.float32)
    assert x.shape[-1] % 32 == 0
    q = np.zeros(x.shape, np.int8)
    s = np.zeros(x.shape[:-1] + (x.shape[-1] // 32,), np.float32)
    lib().orc_quant_act(_p(x), x.size, _p(q), _p(s))
    return q, s


def weight(M: Matrix, e: int, r: int, c: int) -> float:
    st = M._struct()
    return float(lib().orc_weight(ctypes.byref(st), e, r, c))


def weight_bf16(M: Matrix, e: int, r: int, c: int) -> int:
    st = M._struct()
    return int(lib().orc_weight_bf16(ctypes.byref(st), e, r, c))


def ffn_decode(gate: Matrix, up: Matrix, down: Matrix, E: int, x, ids, w, residual,
               tokens=None, trace: bool = False, nthreads: int = 0, shared=None):
    """Decode-layer output for the selected tokens (all when None): returns (out, trace).
    `shared` = (gate, up, down) of one always-active expert added with weight 1 (its trace
    pairs follow the routed ones: pair n_sel*k + s for token position s)."""
    x = _c(x, np.float32)
    residual = _c(residual, np.float32)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    n, d = x.shape
    k = ids.shape[1]
    f = gate.rows
    tok = None if tokens is None else _c(tokens, np.int32)
    n_sel = n if tok is None else len(tok)
    out = np.zeros((n_sel, d), np.float32)
    tr = {}
    ts = None
    if trace:
        P = n_sel * k + (n_sel if shared is not None else 0)
        tr = dict(xq=np.zeros((n_sel, d), np.int8), xs=np.zeros((n_sel, d // 32), np.float32),
                  gate_dots=np.zeros((P, f, d // 32), np.int32),
                  up_dots=np.zeros((P, f, d // 32), np.int32),
                  g=np.zeros((P, f), np.float64), u=np.zeros((P, f), np.float64),
                  h=np.zeros((P, f), np.float32), hq=np.zeros((P, f), np.int8),
                  hs=np.zeros((P, f // 32), np.float32),
                  down_dots=np.zeros((P, d, f // 32), np.int32), y=np.zeros((P, d), np.float64))
        ts = _Trace(**{k_: v.ctypes.data for k_, v in tr.items()})
    sg, su, sd = gate._struct(), up._struct(), down._struct()
    sh = [None, None, None] if shared is None else [ctypes.byref(m._struct()) for m in shared]
    rc = lib().orc_ffn_decode(ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), d, f, E, k,
                              _p(x), n, _p(ids), _p(w), _p(residual), _p(tok), n_sel, _p(out),
                              ctypes.byref(ts) if ts is not None else None, nthreads, *sh)
    if rc != 0:
        raise ValueError("orc_ffn_decode: bad arguments")
    return out, tr


def ffn_prefill(gate: Matrix, up: Matrix, down: Matrix, E: int, x_bf16, ids, w, residual,
                tokens=None, trace: bool = False, nthreads: int = 0):
    """Prefill-layer output (bf16 weights/activations) for the selected tokens."""
    x_bf16 = _c(x_bf16, np.uint16)
    residual = _c(residual, np.float32)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    n, d = x_bf16.shape
    k = ids.shape[1]
    f = gate.rows
    tok = None if tokens is None else _c(tokens, np.int32)
    n_sel = n if tok is None else len(tok)
    out = np.zeros((n_sel, d), np.float32)
    tr = {}
    if trace:
        P = n_sel * k
        tr = dict(g=np.zeros((P, f), np.float64), u=np.zeros((P, f), np.float64),
                  hb=np.zeros((P, f), np.uint16), y=np.zeros((P, d), np.float64))
    sg, su, sd = gate._struct(), up._struct(), down._struct()
    rc = lib().orc_ffn_prefill(ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), d, f, E, k,
                               _p(x_bf16), n, _p(ids), _p(w), _p(residual), _p(tok), n_sel,
                               _p(out), _p(tr.get("g")), _p(tr.get("u")), _p(tr.get("hb")),
                               _p(tr.get("y")), nthreads)
    if rc != 0:
        raise ValueError("orc_ffn_prefill: bad arguments")
    return out, tr
