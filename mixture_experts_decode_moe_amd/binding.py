"""Thin ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: torch tensors are passed as raw device pointers
and the current HIP stream; every step of the layer runs in the library's
kernels.  Importing this module fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_W_INT8_ROW = 1
MOE_W_INT4_B32 = 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() (hipcc, gfx950)")
_lib = ctypes.CDLL(LIB_PATH)


class MoeExperts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("gate_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_q", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("down_s", ctypes.c_void_p)]


class MoeResidual(ctypes.Structure):
    _fields_ = [("residual_in", ctypes.c_void_p), ("residual_out", ctypes.c_void_p),
                ("normed_out", ctypes.c_void_p), ("eps", ctypes.c_float), ("reserved", ctypes.c_int32)]


MOE_N_STAGES = 7
MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_PREFILL = 0, 1, 2
PATHS = {"auto": MOE_PATH_AUTO, "decode": MOE_PATH_DECODE, "prefill": MOE_PATH_PREFILL}


class MoeForwardOpts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("tail_skip", ctypes.c_int32), ("act_quant", ctypes.c_int32),
                ("reserved", ctypes.c_int32),
                ("stage_start", ctypes.c_void_p * MOE_N_STAGES), ("stage_stop", ctypes.c_void_p * MOE_N_STAGES)]


class MoeLayer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("routed", MoeExperts), ("shared", MoeExperts), ("shared_gate_w", ctypes.c_void_p)]


_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_PL = ctypes.POINTER(MoeLayer)
_PE = ctypes.POINTER(MoeExperts)
_PR = ctypes.POINTER(MoeResidual)
_PO = ctypes.POINTER(MoeForwardOpts)
_SIGS = {
    "moe_workspace_bytes": ([_PL, _i32], _sz),
    "moe_workspace_init": ([_vp, _sz, _vp], ctypes.c_int),
    "moe_route_workspace_bytes": ([_PL, _i32], _sz),
    "moe_route": ([_PL, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_permute_workspace_bytes": ([_i32, _i32, _i32], _sz),
    "moe_permute": ([_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_expert_ffn_workspace_bytes": ([_i32, _i32], _sz),
    "moe_expert_ffn": ([_PE, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_combine": ([_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _PR, _vp], ctypes.c_int),
    "moe_layer_forward": ([_PL, _vp, _i32, _vp, _PR, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_layer_forward_ex": ([_PL, _vp, _i32, _vp, _PR, _vp, _vp, _vp, _sz, _PO, _vp], ctypes.c_int),
    "moe_layer_forward_noalloc": ([_PL, _vp, _i32, _vp, _PR, _vp, _vp, _PO, _vp], ctypes.c_int),
    "moe_stack_forward": ([_PL, _i32, _vp, _i32, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _sz, _vp],
                          ctypes.c_int),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_calib_mfma": ([_i32, _i32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double), _vp],
                       ctypes.c_int),
    "moe_calib_read": ([_vp, _sz, ctypes.POINTER(ctypes.c_float), _vp], ctypes.c_int),
}
for _name, (_args, _ret) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _ret

EXPORTED = tuple(_SIGS)


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({_lib.moe_status_string(status).decode()})")
        self.status = status


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


# ------------------------------------------------------------ device layer

@dataclass
class Experts:
    """Device-resident expert set (torch tensors in the ABI's formats)."""
    fmt: int
    n_experts: int
    ffn: int
    gate_q: torch.Tensor
    gate_s: torch.Tensor
    up_q: torch.Tensor
    up_s: torch.Tensor
    down_q: torch.Tensor
    down_s: torch.Tensor

    def c(self) -> MoeExperts:
        return MoeExperts(self.fmt, self.n_experts, self.ffn, 0, *[_ptr(t) for t in (
            self.gate_q, self.gate_s, self.up_q, self.up_s, self.down_q, self.down_s)])


@dataclass
class Layer:
    hidden: int
    n_experts: int
    top_k: int
    renorm: int
    router_w: torch.Tensor
    router_bias: torch.Tensor | None
    routed: Experts
    shared: Experts | None = None
    shared_gate_w: torch.Tensor | None = None

    def c(self) -> MoeLayer:
        sh = self.shared.c() if self.shared is not None else MoeExperts()
        return MoeLayer(self.hidden, self.n_experts, self.top_k, self.renorm, _ptr(self.router_w),
                        _ptr(self.router_bias), self.routed.c(), sh, _ptr(self.shared_gate_w))


def experts_to_device(ex, device="cuda") -> Experts:
    """Upload a host expert set (numpy arrays, the synth module's layout)."""
    def up(a):
        return torch.from_numpy(a).to(device)
    gs, us, ds = ex.gate_s, ex.up_s, ex.down_s
    if ex.fmt == MOE_W_INT4_B32:
        gs, us, ds = (a.view("int16") for a in (gs, us, ds))  # binary16 bits
    return Experts(ex.fmt, ex.n_experts, ex.ffn, up(ex.gate_q), up(gs), up(ex.up_q), up(us), up(ex.down_q), up(ds))


def layer_to_device(layer, device="cuda") -> Layer:
    bias = None if layer.router_bias is None else torch.from_numpy(layer.router_bias).to(device)
    gate = getattr(layer, "shared_gate_w", None)
    return Layer(layer.hidden, layer.n_experts, layer.top_k, layer.renorm,
                 torch.from_numpy(layer.router_w).to(device), bias, experts_to_device(layer.routed, device),
                 None if layer.shared is None else experts_to_device(layer.shared, device),
                 None if gate is None else torch.from_numpy(gate).to(device))


# ------------------------------------------------------------ entry points

def workspace_bytes(layer: Layer, max_tokens: int) -> int:
    c = layer.c()
    return int(_lib.moe_workspace_bytes(ctypes.byref(c), max_tokens))


def make_workspace(layer: Layer, max_tokens: int, device="cuda", stream=None) -> torch.Tensor:
    n = workspace_bytes(layer, max_tokens)
    if n == 0:
        raise MoeError("moe_workspace_bytes", MOE_ERR_INVALID_ARG)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check("moe_workspace_init", _lib.moe_workspace_init(_ptr(ws), n, _stream(stream)))
    return ws


def route_workspace_bytes(layer: Layer, T: int) -> int:
    c = layer.c()
    return int(_lib.moe_route_workspace_bytes(ctypes.byref(c), T))


def route(layer: Layer, x_bf16: torch.Tensor, topk_ids, topk_w, logits=None, ws=None, stream=None,
          shared_gate=None):
    """Router + top-k (+ the shared gate's sigmoid into shared_gate [T]).
    ws None: a workspace of route_workspace_bytes is allocated here when the
    call needs one (see moe_route)."""
    c = layer.c()
    T = x_bf16.shape[0]
    if ws is None:
        need = int(_lib.moe_route_workspace_bytes(ctypes.byref(c), T))
        if need and (logits is None or T > 16):
            ws = torch.empty(need, dtype=torch.uint8, device=x_bf16.device)
    _check("moe_route", _lib.moe_route(ctypes.byref(c), _ptr(x_bf16), T, _ptr(topk_ids), _ptr(topk_w),
                                       _ptr(logits), _ptr(shared_gate), _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(stream)))


def permute(topk_ids, topk_w, E: int, out: dict, ws: torch.Tensor, stream=None):
    T, K = topk_ids.shape
    _check("moe_permute", _lib.moe_permute(
        _ptr(topk_ids), _ptr(topk_w), T, K, E, _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["row_tok"]),
        _ptr(out["row_w"]), _ptr(out["inv_pos"]), _ptr(out["active"]), _ptr(out["n_active"]), _ptr(ws),
        ws.numel(), _stream(stream)))


def permute_workspace_bytes(T, K, E) -> int:
    return int(_lib.moe_permute_workspace_bytes(T, K, E))


def expert_ffn_workspace_bytes(n_rows, ffn) -> int:
    return int(_lib.moe_expert_ffn_workspace_bytes(n_rows, ffn))


def expert_ffn(experts: Experts, hidden: int, x_bf16, n_rows: int, offsets, active, n_active, row_tok, row_w,
               rows_out, ws, stream=None):
    c = experts.c()
    T = x_bf16.shape[0]
    _check("moe_expert_ffn", _lib.moe_expert_ffn(
        ctypes.byref(c), hidden, _ptr(x_bf16), T, n_rows, _ptr(offsets), _ptr(active), _ptr(n_active),
        _ptr(row_tok), _ptr(row_w), _ptr(rows_out), _ptr(ws), ws.numel(), _stream(stream)))


def residual(residual_in, residual_out, normed_out=None, eps=1e-6) -> MoeResidual:
    """Residual epilogue descriptor: residual_out = bf16(residual_in + y),
    normed_out = bf16(rmsnorm(residual_out)) if given."""
    return MoeResidual(_ptr(residual_in), _ptr(residual_out), _ptr(normed_out), eps, 0)


def combine(rows_out, inv_pos, T: int, K: int, H: int, shared_out, y, res: MoeResidual | None = None,
            stream=None, shared_gate=None):
    _check("moe_combine", _lib.moe_combine(_ptr(rows_out), _ptr(inv_pos), T, K, H, _ptr(shared_out),
                                           _ptr(shared_gate), _ptr(y),
                                           ctypes.byref(res) if res is not None else None, _stream(stream)))


STAGES = {"route": 1, "permute": 2, "gateup": 3, "down": 4, "shared": 5, "combine": 6}


def forward_opts(path="auto", events=None, tail_skip=0, act_quant=0) -> MoeForwardOpts:
    """Per-call options: path "auto" | "decode" | "prefill"; tail_skip N (0 =
    off); act_quant 1 for the W8A8 variant; events a dict stage name ->
    (start, stop) torch.cuda.Event pairs (already created, e.g. by one
    record) that the call records around that stage."""
    o = MoeForwardOpts()
    o.path = PATHS[path]
    o.tail_skip = int(tail_skip)
    o.act_quant = int(act_quant)
    for name, (a, b) in (events or {}).items():
        o.stage_start[STAGES[name]] = a.cuda_event
        o.stage_stop[STAGES[name]] = b.cuda_event
    return o


def layer_forward(layer: Layer, x_bf16, y, ws, res: MoeResidual | None = None, topk_ids=None, topk_w=None,
                  stream=None, c_layer: MoeLayer | None = None, opts: MoeForwardOpts | None = None):
    c = layer.c() if c_layer is None else c_layer
    T = x_bf16.shape[0]
    if opts is None:
        _check("moe_layer_forward", _lib.moe_layer_forward(
            ctypes.byref(c), _ptr(x_bf16), T, _ptr(y), ctypes.byref(res) if res is not None else None,
            _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream)))
    else:
        _check("moe_layer_forward_ex", _lib.moe_layer_forward_ex(
            ctypes.byref(c), _ptr(x_bf16), T, _ptr(y), ctypes.byref(res) if res is not None else None,
            _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(), ctypes.byref(opts), _stream(stream)))


def layer_forward_noalloc(layer: Layer, x_bf16, y, res: MoeResidual | None = None, topk_ids=None, topk_w=None,
                          stream=None, c_layer: MoeLayer | None = None, opts: MoeForwardOpts | None = None):
    """moe_layer_forward_noalloc: the layer with the library's own per-device
    scratch array as its workspace."""
    c = layer.c() if c_layer is None else c_layer
    T = x_bf16.shape[0]
    _check("moe_layer_forward_noalloc", _lib.moe_layer_forward_noalloc(
        ctypes.byref(c), _ptr(x_bf16), T, _ptr(y), ctypes.byref(res) if res is not None else None,
        _ptr(topk_ids), _ptr(topk_w), ctypes.byref(opts) if opts is not None else None, _stream(stream)))


def stack_arrays(layers) -> ctypes.Array:
    """A contiguous host array of the layers' C structs (for stack_forward)."""
    arr = (MoeLayer * len(layers))()
    for i, l in enumerate(layers):
        arr[i] = l if isinstance(l, MoeLayer) else l.c()
    return arr


def stack_forward(c_layers, x_bf16, residual_in, residual_out, normed_out, y, ws, eps=1e-6, topk_ids=None,
                  topk_w=None, stream=None):
    """moe_stack_forward over a stack_arrays() array of layers."""
    T = x_bf16.shape[0]
    _check("moe_stack_forward", _lib.moe_stack_forward(
        c_layers, len(c_layers), _ptr(x_bf16), T, _ptr(residual_in), _ptr(residual_out), _ptr(normed_out), eps,
        _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream)))


def calib_mfma(kind: int, iters: int, stream=None):
    """moe_calib_mfma: (ms, operations) of one launch of the matrix-core
    issue-rate kernel (kind 0 fp16, 1 bf16, 2 int8)."""
    ms, ops = ctypes.c_float(), ctypes.c_double()
    _check("moe_calib_mfma", _lib.moe_calib_mfma(kind, iters, ctypes.byref(ms), ctypes.byref(ops), _stream(stream)))
    return ms.value, ops.value


def calib_read(buf: torch.Tensor, nbytes: int, stream=None) -> float:
    """moe_calib_read: ms of one launch reading the first nbytes of buf."""
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    ms = ctypes.c_float()
    _check("moe_calib_read", _lib.moe_calib_read(_ptr(buf), nbytes, ctypes.byref(ms), _stream(stream)))
    return ms.value


def raw_lib():
    """The loaded ctypes library (for tests of the ABI itself)."""
    return _lib
