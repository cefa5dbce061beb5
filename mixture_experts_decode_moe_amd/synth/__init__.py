"""Seeded synthetic inputs for the routed MoE FFN layer.

This module draws random numbers and lays them out in the layer's weight
formats.  It holds none of the layer's arithmetic, and both the CPU oracle's
tests and the GPU path (tests and benchmark) take their inputs from it.

The workloads mirror the model the pages describe: a Qwen3.6-35B-A3B-shaped
layer with 256 experts and top-8 routing ("Qwen3.6-35B-A3B: pictures, several
requests at once and speed", introduction), 40 MoE layers ("qwen36: CUDA VRAM
expert tier", Placement), a two-token MTP verify step ("Every Public GGUF of
This Model Is Missing Its Head", section 3), a 16-request decode batch
("Qwen3.6-35B-A3B ...", Several requests at once) and a 2048-token prompt
chunk ("Qwen3.6-35B-A3B ...", Speed (0.1.45), Prompt chunk).

Formats (row-major, the reduction dimension contiguous):
  int8 row-scaled : q int8 [E][N][Kin],        s float32 [E][N]
  int4 block-32   : q uint8 [E][N][Kin/2],     s float16 bits [E][N][Kin/32]
                    byte j holds element 2j in its low nibble and 2j+1 in
                    its high nibble, each stored as q + 8 with q in [-7, 7].
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoesynth.so")

FMT_INT8_ROW = 1
FMT_INT4_B32 = 2

# stream ids: one per tensor role, so every tensor is an independent stream
S_X, S_X_NOISE, S_ROUTER_W, S_ZIPF_PERM, S_SHARED_GATE = 1, 2, 3, 4, 5
S_GATE_Q, S_GATE_S, S_UP_Q, S_UP_S, S_DOWN_Q, S_DOWN_S = 10, 11, 12, 13, 14, 15
S_SH_OFFSET = 100  # shared expert streams = routed streams + this

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    u64, i32, f64, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, f64, f64, vp, u64, i32]
    lib.synth_normal_f32.argtypes = [u64, u64, u64, f64, f64, vp, u64, i32]
    lib.synth_normal_f64.argtypes = [u64, u64, u64, f64, f64, vp, u64, i32]
    lib.synth_uniform_int8.argtypes = [u64, u64, u64, i32, i32, vp, u64, i32]
    lib.synth_packed_int4.argtypes = [u64, u64, u64, i32, i32, vp, u64, i32]
    lib.synth_scale_f16.argtypes = [u64, u64, u64, f64, f64, f64, vp, u64, i32]
    lib.synth_scale_f32.argtypes = [u64, u64, u64, f64, f64, f64, vp, u64, i32]
    lib.synth_permutation.argtypes = [u64, u64, vp, ctypes.c_int32]
    lib.synth_f64_to_bf16.argtypes = [vp, vp, u64]
    lib.synth_words.argtypes = [u64, u64, u64, vp, u64]
    lib.synth_mix64.argtypes = [u64]
    lib.synth_mix64.restype = u64
    for f in (lib.synth_normal_bf16, lib.synth_normal_f32, lib.synth_normal_f64, lib.synth_uniform_int8,
              lib.synth_packed_int4, lib.synth_scale_f16, lib.synth_scale_f32, lib.synth_permutation,
              lib.synth_f64_to_bf16, lib.synth_words):
        f.restype = None
    _lib = lib
    return lib


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- primitives

def normal_bf16(seed, stream, n, mean=0.0, std=1.0, first=0, out=None):
    out = np.empty(n, np.uint16) if out is None else out
    _load().synth_normal_bf16(seed, stream, first, mean, std, _ptr(out), out.size, _threads())
    return out


def normal_f32(seed, stream, n, mean=0.0, std=1.0, first=0, out=None):
    out = np.empty(n, np.float32) if out is None else out
    _load().synth_normal_f32(seed, stream, first, mean, std, _ptr(out), out.size, _threads())
    return out


def normal_f64(seed, stream, n, mean=0.0, std=1.0, first=0):
    out = np.empty(n, np.float64)
    _load().synth_normal_f64(seed, stream, first, mean, std, _ptr(out), n, _threads())
    return out


def uniform_int8(seed, stream, n, lo=-127, hi=127, first=0, out=None):
    out = np.empty(n, np.int8) if out is None else out
    _load().synth_uniform_int8(seed, stream, first, lo, hi, _ptr(out), out.size, _threads())
    return out


def packed_int4(seed, stream, nbytes, lo=-7, hi=7, first=0, out=None):
    out = np.empty(nbytes, np.uint8) if out is None else out
    _load().synth_packed_int4(seed, stream, first, lo, hi, _ptr(out), out.size, _threads())
    return out


def scale_f16(seed, stream, n, lo, hi, mult, first=0, out=None):
    out = np.empty(n, np.uint16) if out is None else out
    _load().synth_scale_f16(seed, stream, first, lo, hi, mult, _ptr(out), out.size, _threads())
    return out


def scale_f32(seed, stream, n, lo, hi, mult, first=0, out=None):
    out = np.empty(n, np.float32) if out is None else out
    _load().synth_scale_f32(seed, stream, first, lo, hi, mult, _ptr(out), out.size, _threads())
    return out


def permutation(seed, stream, n):
    out = np.empty(n, np.int32)
    _load().synth_permutation(seed, stream, _ptr(out), n)
    return out


def f64_to_bf16(a: np.ndarray):
    a = np.ascontiguousarray(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().synth_f64_to_bf16(_ptr(a), _ptr(out), a.size)
    return out


def words(seed, stream, n, first=0):
    out = np.empty(n, np.uint64)
    _load().synth_words(seed, stream, first, _ptr(out), n)
    return out


# ---------------------------------------------------------------- layer recipes

@dataclass
class Shape:
    tokens: int
    hidden: int
    n_experts: int
    top_k: int
    ffn: int
    shared_ffn: int  # 0 = no shared expert
    fmt: int
    renorm: int = 1
    layers: int = 1
    zipf_s: float = 0.0  # > 0: router bias with Zipf(s) expert popularity
    correlated_sigma: float = 0.0  # > 0: token t>0 = bf16(token 0 + N(0, sigma^2))
    jitter_scales: bool = False  # int8: per-row scale u/(127 sqrt(Kin)), u ~ U[0.5,1.5]
    seed: int = 0
    shared_gate: bool = False  # a gate row for the shared expert, N(0, 0.02) like the router


# The five workloads.  Sizes follow the Qwen3.6-35B-A3B-shaped layer; see
# the module docstring for the passages each one stands in for.
CONFIGS = {
    0: Shape(tokens=4, hidden=1024, n_experts=64, top_k=4, ffn=256, shared_ffn=0, fmt=FMT_INT8_ROW, seed=0),
    1: Shape(tokens=1, hidden=2048, n_experts=256, top_k=8, ffn=512, shared_ffn=512, fmt=FMT_INT8_ROW, seed=1),
    2: Shape(tokens=2, hidden=2048, n_experts=256, top_k=8, ffn=512, shared_ffn=512, fmt=FMT_INT4_B32,
             correlated_sigma=0.3 / (0.02 * math.sqrt(2048.0)), seed=2),
    3: Shape(tokens=16, hidden=2048, n_experts=256, top_k=8, ffn=512, shared_ffn=512, fmt=FMT_INT4_B32,
             layers=40, zipf_s=1.1, seed=3),
    4: Shape(tokens=2048, hidden=2048, n_experts=256, top_k=8, ffn=512, shared_ffn=512, fmt=FMT_INT4_B32, seed=4),
}

CONFIG_NAMES = {
    0: "tiny int8 layer: T=4 H=1024 E=64 K=4 F=256",
    1: "decode layer int8: T=1 H=2048 E=256 K=8 F=512 + shared F=512",
    2: "MTP verify int4: T=2 H=2048 E=256 K=8 F=512 + shared, correlated tokens",
    3: "16-request decode batch int4: T=16, 40 distinct layers, Zipf(1.1) router bias, residual",
    4: "prefill chunk int4: T=2048 H=2048 E=256 K=8 F=512 + shared",
}


def layer_seed(shape: Shape, layer: int) -> int:
    """Config c uses seed c; layer l of a stack uses seed 1000 + l."""
    return 1000 + layer if shape.layers > 1 else shape.seed


@dataclass
class ExpertsHost:
    fmt: int
    n_experts: int
    hidden: int
    ffn: int
    gate_q: np.ndarray
    gate_s: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray

    def nbytes_per_expert(self):
        return sum(a.nbytes for a in (self.gate_q, self.gate_s, self.up_q, self.up_s, self.down_q,
                                      self.down_s)) // self.n_experts


@dataclass
class LayerHost:
    hidden: int
    n_experts: int
    top_k: int
    renorm: int
    router_w: np.ndarray  # float32 [E][H]
    router_bias: np.ndarray | None  # float32 [E] or None
    routed: ExpertsHost
    shared: ExpertsHost | None = None
    shared_gate_w: np.ndarray | None = None  # float32 [H] or None
    extras: dict = field(default_factory=dict)


def _matrix(fmt, seed, s_q, s_s, n_mat, rows, kin, jitter, expert_lo=0, expert_hi=None):
    """One weight role ([n_mat][rows][kin]) in the given format.  Experts
    [expert_lo, expert_hi) are drawn; counters are global so any slice draws
    the same values as the whole tensor."""
    expert_hi = n_mat if expert_hi is None else expert_hi
    ne = expert_hi - expert_lo
    if fmt == FMT_INT8_ROW:
        per = rows * kin
        q = uniform_int8(seed, s_q, ne * per, -127, 127, first=expert_lo * per).reshape(ne, rows, kin)
        if jitter:
            s = scale_f32(seed, s_s, ne * rows, 0.5, 1.5, 1.0 / (127.0 * math.sqrt(kin)),
                          first=expert_lo * rows).reshape(ne, rows)
        else:
            s = np.full((ne, rows), np.float32(1.0 / (127.0 * math.sqrt(kin))), np.float32)
        return q, s
    if fmt == FMT_INT4_B32:
        assert kin % 32 == 0
        per = rows * kin // 2
        q = packed_int4(seed, s_q, ne * per, first=expert_lo * per).reshape(ne, rows, kin // 2)
        nblk = rows * kin // 32
        s = scale_f16(seed, s_s, ne * nblk, 0.5, 1.5, 1.0 / (7.0 * math.sqrt(kin)),
                      first=expert_lo * nblk).reshape(ne, rows, kin // 32)
        return q, s
    raise ValueError(f"unknown weight format {fmt}")


def make_experts(fmt, seed, n_experts, hidden, ffn, shared=False, jitter=False, expert_lo=0, expert_hi=None):
    off = S_SH_OFFSET if shared else 0
    gq, gs = _matrix(fmt, seed, S_GATE_Q + off, S_GATE_S + off, n_experts, ffn, hidden, jitter, expert_lo, expert_hi)
    uq, us = _matrix(fmt, seed, S_UP_Q + off, S_UP_S + off, n_experts, ffn, hidden, jitter, expert_lo, expert_hi)
    dq, ds = _matrix(fmt, seed, S_DOWN_Q + off, S_DOWN_S + off, n_experts, hidden, ffn, jitter, expert_lo, expert_hi)
    ne = (n_experts if expert_hi is None else expert_hi) - expert_lo
    return ExpertsHost(fmt, ne, hidden, ffn, gq, gs, uq, us, dq, ds)


def make_router_bias(shape: Shape, seed: int):
    """Zipf(s) popularity as a log-prior: bias_e = -s * ln(1 + pi(e)), pi a
    seeded permutation of the experts (rank 1 = most popular)."""
    if shape.zipf_s <= 0:
        return None
    perm = permutation(seed, S_ZIPF_PERM, shape.n_experts)
    return (-shape.zipf_s * np.log1p(perm.astype(np.float64))).astype(np.float32)


def make_layer(shape: Shape, layer: int = 0, jitter=None, routed_range=None) -> LayerHost:
    seed = layer_seed(shape, layer)
    jitter = shape.jitter_scales if jitter is None else jitter
    wr = normal_f32(seed, S_ROUTER_W, shape.n_experts * shape.hidden, 0.0, 0.02).reshape(shape.n_experts,
                                                                                         shape.hidden)
    lo, hi = (0, shape.n_experts) if routed_range is None else routed_range
    routed = make_experts(shape.fmt, seed, shape.n_experts, shape.hidden, shape.ffn, jitter=jitter,
                          expert_lo=lo, expert_hi=hi)
    shared = None
    if shape.shared_ffn:
        shared = make_experts(shape.fmt, seed, 1, shape.hidden, shape.shared_ffn, shared=True, jitter=jitter)
    gate = None
    if shape.shared_gate and shape.shared_ffn:
        gate = normal_f32(seed, S_SHARED_GATE, shape.hidden, 0.0, 0.02)
    return LayerHost(shape.hidden, shape.n_experts, shape.top_k, shape.renorm, wr, make_router_bias(shape, seed),
                     routed, shared, gate)


def make_x(shape: Shape, tokens: int | None = None, seed: int | None = None) -> np.ndarray:
    """bf16 bits [T][H], N(0,1).  With correlated_sigma > 0, token t > 0 is
    bf16(token0 + N(0, sigma^2)) so its router logits are token 0's plus
    N(0, (0.02 sqrt(H) sigma)^2)."""
    T = shape.tokens if tokens is None else tokens
    seed = shape.seed if seed is None else seed
    H = shape.hidden
    if shape.correlated_sigma <= 0:
        return normal_bf16(seed, S_X, T * H).reshape(T, H)
    x0 = normal_bf16(seed, S_X, H)
    x0f = (x0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = np.empty((T, H), np.uint16)
    out[0] = x0
    if T > 1:
        noise = normal_f64(seed, S_X_NOISE, (T - 1) * H, 0.0, shape.correlated_sigma).reshape(T - 1, H)
        out[1:] = f64_to_bf16(x0f[None, :] + noise)
    return out
