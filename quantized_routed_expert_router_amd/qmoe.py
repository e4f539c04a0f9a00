"""Python binding of libqmoe (C ABI in include/qmoe.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
PyTorch provides device memory and the current stream. There is no CPU fallback: if the
compiled library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libqmoe.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}

MAX_EXPERTS = 1024
MAX_TOP_K = 64
MAX_DECODE_TOKENS = 512
MAX_PREFILL_TOKENS = 8192

EXPORTS = ("moe_status_string", "moe_route_workspace_bytes", "moe_route",
           "moe_ffn_workspace_bytes", "moe_expert_ffn_decode", "moe_expert_ffn_decode_stages",
           "moe_layer_decode", "moe_layer_decode_stages", "moe_layer_decode_noalloc",
           "moe_expert_ffn_prefill", "moe_expert_ffn_prefill_stages")

NOALLOC_SCRATCH_BYTES = 16 << 20

DECODE_PREP, DECODE_GATE_UP, DECODE_DOWN, DECODE_COMBINE, DECODE_ALL = 1, 2, 4, 8, 15
PREFILL_PREP, PREFILL_GATE_UP, PREFILL_DOWN, PREFILL_COMBINE, PREFILL_ALL = 1, 2, 4, 8, 15


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class _QMatrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale_min", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("bits", ctypes.c_int32)]


class _Layer(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("gate", _QMatrix), ("up", _QMatrix), ("down", _QMatrix),
                ("shared_gate", _QMatrix), ("shared_up", _QMatrix), ("shared_down", _QMatrix),
                ("router_w", ctypes.c_void_p)]


class _Routing(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("pair_index", ctypes.c_void_p)]


DEBUG_FIELDS = ("xq", "xs", "gate_dots", "up_dots", "g", "u", "h", "hq", "hs", "down_dots", "y",
                "logits")


class _Debug(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in DEBUG_FIELDS]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m quantized_routed_expert_router_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_route_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_route_workspace_bytes.restype = sz
    L.moe_route.argtypes = [vp, i32, i32, i32, ctypes.POINTER(_Routing), vp, sz, vp]
    L.moe_ffn_workspace_bytes.argtypes = [ctypes.POINTER(_Layer), i32, i32]
    L.moe_ffn_workspace_bytes.restype = sz
    L.moe_expert_ffn_decode.argtypes = [ctypes.POINTER(_Layer), vp, i32, ctypes.POINTER(_Routing),
                                        vp, vp, sz, ctypes.POINTER(_Debug), vp]
    L.moe_expert_ffn_decode_stages.argtypes = [
        ctypes.POINTER(_Layer), vp, i32, ctypes.POINTER(_Routing), vp, vp, sz,
        ctypes.POINTER(_Debug), ctypes.c_uint, vp]
    L.moe_layer_decode.argtypes = [ctypes.POINTER(_Layer), vp, vp, i32, ctypes.POINTER(_Routing),
                                   vp, vp, sz, ctypes.POINTER(_Debug), vp]
    L.moe_layer_decode_stages.argtypes = [
        ctypes.POINTER(_Layer), vp, vp, i32, ctypes.POINTER(_Routing), vp, vp, sz,
        ctypes.POINTER(_Debug), ctypes.c_uint, vp]
    L.moe_layer_decode_noalloc.argtypes = [ctypes.POINTER(_Layer), vp, vp, i32,
                                           ctypes.POINTER(_Routing), vp, vp]
    L.moe_expert_ffn_prefill.argtypes = [ctypes.POINTER(_Layer), vp, i32, ctypes.POINTER(_Routing),
                                         vp, vp, sz, vp]
    L.moe_expert_ffn_prefill_stages.argtypes = [
        ctypes.POINTER(_Layer), vp, i32, ctypes.POINTER(_Routing), vp, vp, sz, ctypes.c_uint, vp]
    return L


lib = _load()


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


class _Args:
    """Checks of the tensors of one call before their pointers go to the library: first
    each tensor's dtype, layout and extent (need), then that all of them sit on one GPU
    (on_gpu). Raises ValueError."""

    def __init__(self):
        self.seen = []

    def need(self, t, name: str, dtypes, shape=None, min_numel=None):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
        if t.dtype not in dtypes:
            raise ValueError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if min_numel is not None and t.numel() < min_numel:
            raise ValueError(f"{name}: {t.numel()} elements, at least {min_numel} needed")
        self.seen.append((name, t))

    def on_gpu(self):
        dev = None
        for name, t in self.seen:
            if not t.is_cuda:
                raise ValueError(f"{name}: must be a GPU tensor (got device {t.device})")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name}: on {t.device}, the other arguments on {dev}")


F32 = (torch.float32,)
I32 = (torch.int32,)
TWO_BYTE = (torch.int16, torch.bfloat16, torch.float16, torch.uint16)
WORDS = (torch.int32, torch.uint32)
BYTES = (torch.uint8, torch.int8)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


@dataclass
class QMatrix:
    """Packed weights of one projection for all experts, in device memory.
    codes: int32 storage of uint32 [E][cols/32][rows][bits]; scale_min: int16 storage of
    fp16 pairs [E][cols/32][rows][2]."""
    codes: torch.Tensor
    scale_min: torch.Tensor
    rows: int
    cols: int
    bits: int

    def check(self, E: int, name: str, args: "_Args") -> None:
        """Extents of E experts' codes and scale/min words (see the class docstring)."""
        if self.bits not in (2, 4) or self.cols % 32 or self.rows <= 0:
            raise ValueError(f"{name}: bad shape rows={self.rows} cols={self.cols} "
                             f"bits={self.bits}")
        blocks = E * (self.cols // 32) * self.rows
        args.need(self.codes, f"{name}.codes", WORDS, min_numel=blocks * self.bits)
        args.need(self.scale_min, f"{name}.scale_min", TWO_BYTE, min_numel=blocks * 2)

    def _struct(self) -> _QMatrix:
        return _QMatrix(self.codes.data_ptr(), self.scale_min.data_ptr(), self.rows, self.cols,
                        self.bits)


@dataclass
class Layer:
    """One MoE layer: E routed experts, optionally one always-active shared expert
    (`shared` = its (gate, up, down), one expert each in the routed experts' format) and
    optionally the router's weights (`router`: bf16 bits [E][d] in a 2-byte tensor), which
    let layer_decode project its own logits."""
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    gate: QMatrix
    up: QMatrix
    down: QMatrix
    shared: tuple[QMatrix, QMatrix, QMatrix] | None = None
    router: torch.Tensor | None = None

    def _struct(self) -> _Layer:
        sh = [m._struct() for m in self.shared] if self.shared else [_QMatrix()] * 3
        rw = None
        if self.router is not None:
            assert self.router.element_size() == 2 and self.router.is_contiguous()
            assert tuple(self.router.shape) == (self.n_experts, self.d_model)
            rw = self.router.data_ptr()
        return _Layer(self.d_model, self.d_ff, self.n_experts, self.top_k, self.gate._struct(),
                      self.up._struct(), self.down._struct(), *sh, rw)

    def check(self, args: "_Args") -> None:
        """Every matrix holds n_experts experts (the shared ones one) of the layer's shape;
        the router rows are [n_experts, d_model] two-byte values."""
        d, f = self.d_model, self.d_ff
        for name, m, rows, cols, E in (("gate", self.gate, f, d, self.n_experts),
                                        ("up", self.up, f, d, self.n_experts),
                                        ("down", self.down, d, f, self.n_experts)):
            if (m.rows, m.cols) != (rows, cols):
                raise ValueError(f"{name}: {m.rows}x{m.cols}, expected {rows}x{cols}")
            m.check(E, name, args)
        if self.shared:
            for name, m, rows, cols in (("shared_gate", self.shared[0], f, d),
                                        ("shared_up", self.shared[1], f, d),
                                        ("shared_down", self.shared[2], d, f)):
                if (m.rows, m.cols) != (rows, cols):
                    raise ValueError(f"{name}: {m.rows}x{m.cols}, expected {rows}x{cols}")
                m.check(1, name, args)
        if self.router is not None:
            args.need(self.router, "router", TWO_BYTE, shape=(self.n_experts, d))

    def pairs(self, n: int) -> int:
        """Pair slots of an n-token window: n*k routed, plus n shared (pair n*k + t)."""
        return n * self.top_k + (n if self.shared else 0)


@dataclass
class Routing:
    topk_ids: torch.Tensor      # int32 [n, k]
    topk_w: torch.Tensor        # fp32 [n, k]
    expert_offsets: torch.Tensor  # int32 [E+1]
    pair_index: torch.Tensor    # int32 [n*k]

    @staticmethod
    def empty(n: int, E: int, k: int, device="cuda") -> "Routing":
        return Routing(torch.empty((n, k), dtype=torch.int32, device=device),
                       torch.empty((n, k), dtype=torch.float32, device=device),
                       torch.empty(E + 1, dtype=torch.int32, device=device),
                       torch.empty(max(n * k, 1), dtype=torch.int32, device=device))

    def check(self, n: int, E: int, k: int, args: "_Args") -> None:
        args.need(self.topk_ids, "topk_ids", I32, min_numel=n * k)
        args.need(self.topk_w, "topk_w", F32, min_numel=n * k)
        args.need(self.expert_offsets, "expert_offsets", I32, min_numel=E + 1)
        args.need(self.pair_index, "pair_index", I32, min_numel=n * k)

    def _struct(self) -> _Routing:
        return _Routing(self.topk_ids.data_ptr(), self.topk_w.data_ptr(),
                        self.expert_offsets.data_ptr(), self.pair_index.data_ptr())


def route_workspace(n: int, E: int, top_k: int, device="cuda") -> torch.Tensor | None:
    nbytes = int(lib.moe_route_workspace_bytes(n, E, top_k))
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def route(logits: torch.Tensor, top_k: int, out: Routing | None = None, stream=None,
          ws: torch.Tensor | None = None) -> Routing:
    """moe_route: top-k experts, routing weights and expert grouping of `logits` [n, E]."""
    if logits.dim() != 2:
        raise ValueError(f"logits: expected [n, E], got shape {tuple(logits.shape)}")
    n, E = logits.shape
    args = _Args()
    args.need(logits, "logits", F32)
    if out is None:
        out = Routing.empty(n, E, top_k, logits.device)
    if ws is None:
        ws = route_workspace(n, E, top_k, logits.device)
    out.check(n, E, top_k, args)
    if ws is not None:
        args.need(ws, "ws", BYTES)
    args.on_gpu()
    st = out._struct()
    rc = lib.moe_route(_ptr(logits), n, E, top_k, ctypes.byref(st), _ptr(ws),
                       0 if ws is None else ws.numel(), _stream(stream))
    if rc != MOE_OK:
        raise MoeError("moe_route", rc)
    return out


def ffn_workspace_bytes(layer: Layer, n_tokens: int, prefill: bool = False) -> int:
    st = layer._struct()
    return int(lib.moe_ffn_workspace_bytes(ctypes.byref(st), n_tokens, 1 if prefill else 0))


def workspace(layer: Layer, n_tokens: int, prefill: bool = False, device="cuda") -> torch.Tensor:
    nbytes = max(ffn_workspace_bytes(layer, n_tokens, prefill), 256)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def debug_buffers(layer: Layer, n: int, device="cuda") -> dict:
    d, f = layer.d_model, layer.d_ff
    P = layer.pairs(n)
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)  # noqa: E731
    return dict(xq=z((n, d), torch.int8), xs=z((n, d // 32), torch.float32),
                gate_dots=z((P, f, d // 32), torch.int32), up_dots=z((P, f, d // 32), torch.int32),
                g=z((P, f), torch.float32), u=z((P, f), torch.float32), h=z((P, f), torch.float32),
                hq=z((P, f), torch.int8), hs=z((P, f // 32), torch.float32),
                down_dots=z((P, d, f // 32), torch.int32), y=z((P, d), torch.float32),
                logits=z((n, layer.n_experts), torch.float32) if layer.router is not None else None)


def _check_decode_args(layer: Layer, x, residual, routing: Routing, logits, ws, debug) -> int:
    """Checks of a decode call's tensors; returns the token count."""
    args = _Args()
    layer.check(args)
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"x: expected [n, d_model], got {getattr(x, 'shape', type(x))}")
    n = x.shape[0]
    args.need(x, "x", F32, shape=(n, layer.d_model))
    args.need(residual, "residual", F32, shape=(n, layer.d_model))
    if logits is not None:
        args.need(logits, "logits", F32, shape=(n, layer.n_experts))
    routing.check(n, layer.n_experts, layer.top_k, args)
    if ws is not None:
        args.need(ws, "ws", BYTES)
    if debug is not None:
        # each debug buffer given holds at least what debug_buffers allocates
        ref = debug_buffers(layer, n, device="meta")
        for key, t in debug.items():
            if key not in DEBUG_FIELDS:
                raise ValueError(f"debug: unknown buffer {key!r}")
            if t is None:
                continue
            if ref[key] is None:
                raise ValueError(f"debug[{key!r}]: this layer writes no such buffer")
            args.need(t, f"debug[{key!r}]", (ref[key].dtype,), min_numel=ref[key].numel())
    args.on_gpu()
    return n


def ffn_decode(layer: Layer, x: torch.Tensor, routing: Routing, residual: torch.Tensor,
               ws: torch.Tensor | None = None, debug: dict | None = None, stream=None,
               stages: int | None = None) -> None:
    """moe_expert_ffn_decode: residual += routing-weighted expert outputs (in place).
    With `stages` (DECODE_* bits) the call goes through moe_expert_ffn_decode_stages."""
    n = _check_decode_args(layer, x, residual, routing, None, ws, debug)
    if ws is None:
        ws = workspace(layer, n, device=x.device)
    st, rs = layer._struct(), routing._struct()
    dbg = None
    if debug is not None:
        dbg = ctypes.byref(_Debug(**{k_: _ptr(debug.get(k_)) for k_ in DEBUG_FIELDS}))
    if stages is None:
        rc = lib.moe_expert_ffn_decode(ctypes.byref(st), _ptr(x), n, ctypes.byref(rs),
                                       _ptr(residual), _ptr(ws), ws.numel(), dbg, _stream(stream))
        fn = "moe_expert_ffn_decode"
    else:
        rc = lib.moe_expert_ffn_decode_stages(ctypes.byref(st), _ptr(x), n, ctypes.byref(rs),
                                              _ptr(residual), _ptr(ws), ws.numel(), dbg, stages,
                                              _stream(stream))
        fn = "moe_expert_ffn_decode_stages"
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def layer_decode(layer: Layer, logits: torch.Tensor | None, x: torch.Tensor,
                 residual: torch.Tensor, routing: Routing | None = None,
                 ws: torch.Tensor | None = None, debug: dict | None = None, stream=None,
                 stages: int | None = None) -> Routing:
    """moe_layer_decode: route `logits` (None: the layer's router projects them from x) and
    run the decode expert FFN (residual in place). Returns the routing it wrote."""
    n = x.shape[0]
    if routing is None:
        routing = Routing.empty(n, layer.n_experts, layer.top_k, x.device)
    _check_decode_args(layer, x, residual, routing, logits, ws, debug)
    if ws is None:
        ws = workspace(layer, n, device=x.device)
    st, rs = layer._struct(), routing._struct()
    dbg = None
    if debug is not None:
        dbg = ctypes.byref(_Debug(**{k_: _ptr(debug.get(k_)) for k_ in DEBUG_FIELDS}))
    if stages is None:
        rc = lib.moe_layer_decode(ctypes.byref(st), _ptr(logits), _ptr(x), n, ctypes.byref(rs),
                                  _ptr(residual), _ptr(ws), ws.numel(), dbg, _stream(stream))
        fn = "moe_layer_decode"
    else:
        rc = lib.moe_layer_decode_stages(ctypes.byref(st), _ptr(logits), _ptr(x), n,
                                         ctypes.byref(rs), _ptr(residual), _ptr(ws), ws.numel(),
                                         dbg, stages, _stream(stream))
        fn = "moe_layer_decode_stages"
    if rc != MOE_OK:
        raise MoeError(fn, rc)
    return routing


def layer_decode_noalloc(layer: Layer, logits: torch.Tensor | None, x: torch.Tensor,
                         residual: torch.Tensor, routing: Routing, stream=None) -> Routing:
    """moe_layer_decode_noalloc: layer_decode on the library's own per-GPU workspace (no
    workspace argument; the call allocates nothing). `routing` is written in place."""
    n = x.shape[0]
    _check_decode_args(layer, x, residual, routing, logits, None, None)
    st, rs = layer._struct(), routing._struct()
    rc = lib.moe_layer_decode_noalloc(ctypes.byref(st), _ptr(logits), _ptr(x), n,
                                      ctypes.byref(rs), _ptr(residual), _stream(stream))
    if rc != MOE_OK:
        raise MoeError("moe_layer_decode_noalloc", rc)
    return routing


def ffn_prefill(layer: Layer, x_bf16: torch.Tensor, routing: Routing, residual: torch.Tensor,
                ws: torch.Tensor | None = None, stream=None, stages: int | None = None) -> None:
    """moe_expert_ffn_prefill: bf16 matrix-core layer; residual updated in place.
    x_bf16 holds bf16 bit patterns (any 2-byte dtype). With `stages` (PREFILL_* bits) the
    call goes through moe_expert_ffn_prefill_stages."""
    n = x_bf16.shape[0]
    args = _Args()
    layer.check(args)
    args.need(x_bf16, "x_bf16", TWO_BYTE, shape=(n, layer.d_model))
    args.need(residual, "residual", F32, shape=(n, layer.d_model))
    routing.check(n, layer.n_experts, layer.top_k, args)
    if ws is not None:
        args.need(ws, "ws", BYTES)
    args.on_gpu()
    if ws is None:
        ws = workspace(layer, n, prefill=True, device=x_bf16.device)
    st, rs = layer._struct(), routing._struct()
    if stages is None:
        rc = lib.moe_expert_ffn_prefill(ctypes.byref(st), _ptr(x_bf16), n, ctypes.byref(rs),
                                        _ptr(residual), _ptr(ws), ws.numel(), _stream(stream))
        fn = "moe_expert_ffn_prefill"
    else:
        rc = lib.moe_expert_ffn_prefill_stages(ctypes.byref(st), _ptr(x_bf16), n,
                                               ctypes.byref(rs), _ptr(residual), _ptr(ws),
                                               ws.numel(), stages, _stream(stream))
        fn = "moe_expert_ffn_prefill_stages"
    if rc != MOE_OK:
        raise MoeError(fn, rc)
