"""CPU oracle of the routed mixture-of-experts FFN layer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  This package states what the layer computes in
plain double-precision C++ (``moe_oracle.cpp``); only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it.  It shares no code
with the GPU library and never imports it.

Every function here takes and returns numpy arrays in the formats described
in ``moe_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC = os.path.join(_HERE, "moe_oracle.cpp")


def build(verbose=False):
    """Compile the oracle with the host compiler (no GPU code involved)."""
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-pthread",
           SRC, "-o", LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)


class _Experts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("gate_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_q", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("down_s", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("routed", _Experts), ("shared", ctypes.POINTER(_Experts)), ("shared_gate_w", ctypes.c_void_p)]


class _Opts(ctypes.Structure):
    _fields_ = [("tail_skip", ctypes.c_int32), ("act_quant", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = f64
        L.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_double.restype = f64
        L.oracle_double_to_bf16.argtypes = [f64]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_weight.argtypes = [i32, vp, vp, i64, i64, i64, i64, i64]
        L.oracle_weight.restype = f64
        L.oracle_dequant.argtypes = [i32, vp, vp, i64, i64, i64, vp]
        L.oracle_dequant.restype = ctypes.c_int
        L.oracle_router_logits.argtypes = [ctypes.POINTER(_Layer), vp, i32, vp]
        L.oracle_router_logits.restype = None
        L.oracle_select.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.oracle_select.restype = None
        L.oracle_expert_apply.argtypes = [ctypes.POINTER(_Experts), i32, vp, vp]
        L.oracle_expert_apply.restype = ctypes.c_int
        L.oracle_permute.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_permute.restype = None
        L.oracle_layer_forward.argtypes = [ctypes.POINTER(_Layer), vp, i32, vp, vp, vp, vp, vp, i32]
        L.oracle_layer_forward.restype = ctypes.c_int
        L.oracle_layer_forward_ex.argtypes = [ctypes.POINTER(_Layer), vp, i32, vp, ctypes.POINTER(_Opts), vp, vp,
                                              vp, vp, i32]
        L.oracle_layer_forward_ex.restype = ctypes.c_int
        L.oracle_quantize_row.argtypes = [vp, i64, vp, vp]
        L.oracle_quantize_row.restype = None
        L.oracle_expert_rows.argtypes = [ctypes.POINTER(_Experts), vp, vp, vp, vp, i32, vp, i32]
        L.oracle_expert_rows.restype = ctypes.c_int
        L.oracle_residual.argtypes = [vp, vp, i64, vp]
        L.oracle_residual.restype = None
        L.oracle_rmsnorm.argtypes = [vp, i64, i64, f64, vp]
        L.oracle_rmsnorm.restype = None
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous numpy"
    return a.ctypes.data


def _experts_struct(ex, keep):
    """ex: any object with fmt, n_experts, hidden, ffn and the six arrays."""
    arrs = [np.ascontiguousarray(a) for a in (ex.gate_q, ex.gate_s, ex.up_q, ex.up_s, ex.down_q, ex.down_s)]
    keep.extend(arrs)
    return _Experts(ex.fmt, ex.n_experts, ex.hidden, ex.ffn, *[_p(a) for a in arrs])


def _layer_struct(layer, keep):
    wr = np.ascontiguousarray(layer.router_w, np.float32)
    keep.append(wr)
    b = None
    if layer.router_bias is not None:
        b = np.ascontiguousarray(layer.router_bias, np.float32)
        keep.append(b)
    routed = _experts_struct(layer.routed, keep) if layer.routed is not None else _Experts()
    sh = None
    if layer.shared is not None:
        s = _experts_struct(layer.shared, keep)
        keep.append(s)
        sh = ctypes.pointer(s)
    g = None
    if getattr(layer, "shared_gate_w", None) is not None:
        g = np.ascontiguousarray(layer.shared_gate_w, np.float32)
        keep.append(g)
    st = _Layer(layer.hidden, layer.n_experts, layer.top_k, layer.renorm, _p(wr), _p(b), routed, sh, _p(g))
    keep.append(st)
    return st


# ------------------------------------------------------------------ wrappers

def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits))


def f16_to_double(bits: int) -> float:
    return lib().oracle_f16_to_double(int(bits))


def double_to_bf16(v: float) -> int:
    return lib().oracle_double_to_bf16(float(v))


def weight(fmt, q, s, e, rows, kin, n, k) -> float:
    return lib().oracle_weight(fmt, _p(q), _p(s), e, rows, kin, n, k)


def dequant(fmt, q, s, n_mat, rows, kin):
    out = np.empty((n_mat, rows, kin), np.float64)
    rc = lib().oracle_dequant(fmt, _p(np.ascontiguousarray(q)), _p(np.ascontiguousarray(s)), n_mat, rows, kin,
                              _p(out))
    return out, rc


def router_logits(layer, x_bf16):
    keep = []
    st = _layer_struct(layer, keep)
    x = np.ascontiguousarray(x_bf16, np.uint16)
    T = x.shape[0]
    out = np.empty((T, layer.n_experts), np.float64)
    lib().oracle_router_logits(ctypes.byref(st), _p(x), T, _p(out))
    return out


def select(logits, K, renorm=1):
    logits = np.ascontiguousarray(logits, np.float64)
    T, E = logits.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    lib().oracle_select(_p(logits), T, E, K, renorm, _p(ids), _p(w))
    return ids, w


def expert_apply(experts, e, x_f64):
    keep = []
    st = _experts_struct(experts, keep)
    x = np.ascontiguousarray(x_f64, np.float64)
    out = np.empty(experts.hidden, np.float64)
    rc = lib().oracle_expert_apply(ctypes.byref(st), e, _p(x), _p(out))
    if rc != 0:
        raise ValueError("malformed expert weights (int4 nibble 0)")
    return out


def permute(ids, w, E):
    ids = np.ascontiguousarray(ids, np.int32)
    T, K = ids.shape
    wf = None if w is None else np.ascontiguousarray(w, np.float32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_tok = np.empty(T * K, np.int32)
    row_w = np.empty(T * K, np.float32)
    inv_pos = np.empty((T, K), np.int32)
    active = np.empty(E, np.int32)
    n_active = np.zeros(1, np.int32)
    lib().oracle_permute(_p(ids), _p(wf), T, K, E, _p(counts), _p(offsets), _p(row_tok), _p(row_w), _p(inv_pos),
                         _p(active), _p(n_active))
    na = int(n_active[0])
    return dict(counts=counts, offsets=offsets, row_tok=row_tok, row_w=row_w, inv_pos=inv_pos,
                active=active[:na].copy(), n_active=na)


def layer_forward(layer, x_bf16, ids=None, nthreads=0, tail_skip=0, act_quant=0):
    """Returns y [T][H] float64, ids [T][K], w [T][K], logits [T][E].
    tail_skip / act_quant: the variants of oracle_opts (0 = off)."""
    keep = []
    st = _layer_struct(layer, keep)
    x = np.ascontiguousarray(x_bf16, np.uint16)
    T = x.shape[0]
    K = layer.top_k
    y = np.empty((T, layer.hidden), np.float64)
    ids_out = np.empty((T, K), np.int32)
    w_out = np.empty((T, K), np.float64)
    logits = np.empty((T, layer.n_experts), np.float64)
    ids_in = None if ids is None else np.ascontiguousarray(ids, np.int32)
    opts = _Opts(int(tail_skip), int(act_quant))
    rc = lib().oracle_layer_forward_ex(ctypes.byref(st), _p(x), T, _p(ids_in), ctypes.byref(opts), _p(y),
                                       _p(ids_out), _p(w_out), _p(logits), nthreads)
    if rc != 0:
        raise ValueError("malformed expert weights (int4 nibble 0)")
    return y, ids_out, w_out, logits


def quantize_row(v):
    """Per-row int8 quantisation in float32: returns (q int8 [n], d float32)."""
    v = np.ascontiguousarray(v, np.float32)
    q = np.empty(v.shape, np.int8)
    d = np.zeros(1, np.float32)
    lib().oracle_quantize_row(_p(v), v.size, _p(q), _p(d))
    return q, d[0]


def expert_rows(experts, x_bf16, offsets, row_tok, row_w, nthreads=0):
    keep = []
    st = _experts_struct(experts, keep)
    x = np.ascontiguousarray(x_bf16, np.uint16)
    offsets = np.ascontiguousarray(offsets, np.int32)
    n_rows = int(offsets[-1])
    rt = None if row_tok is None else np.ascontiguousarray(row_tok, np.int32)
    rw = None if row_w is None else np.ascontiguousarray(row_w, np.float32)
    out = np.empty((n_rows, experts.hidden), np.float64)
    rc = lib().oracle_expert_rows(ctypes.byref(st), _p(x), _p(offsets), _p(rt), _p(rw), n_rows, _p(out), nthreads)
    if rc != 0:
        raise ValueError("malformed expert rows")
    return out


def residual(x_bf16, y):
    x = np.ascontiguousarray(x_bf16, np.uint16)
    y = np.ascontiguousarray(y, np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_residual(_p(x), _p(y), x.size, _p(out))
    return out


def rmsnorm(r_bf16, eps=1e-6):
    r = np.ascontiguousarray(r_bf16, np.uint16)
    T, H = r.shape
    out = np.empty_like(r)
    lib().oracle_rmsnorm(_p(r), T, H, eps, _p(out))
    return out


def threads() -> int:
    return int(lib().oracle_threads())
