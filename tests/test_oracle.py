"""Pins of the CPU oracle against things other than itself.

The pages print no worked example of this layer, so the oracle is pinned by
the IEEE definitions (checked against numpy's own conversions), hand-worked
cases, brute-force dense evaluation of every expert masked to the top-k,
closed forms (softmax identities, K = 1, K = E) and invariants.  Each test
is chosen so that a plausible slip in the oracle (a dropped term, a wrong
sign or index, a transposed operand, a swapped nibble) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from mixture_experts_decode_moe_amd import synth
from mixture_experts_decode_moe_amd.synth import ExpertsHost, LayerHost

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------- test-side helpers

def bf16_bits_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_dequant(ex, role):
    """Independent numpy dequantisation of one weight role -> [E][N][Kin]."""
    q = getattr(ex, role + "_q")
    s = getattr(ex, role + "_s")
    if ex.fmt == synth.FMT_INT8_ROW:
        return q.astype(np.float64) * s.astype(np.float64)[..., None]
    E, N, half = q.shape
    lo = (q & 0x0F).astype(np.int64) - 8
    hi = (q >> 4).astype(np.int64) - 8
    qq = np.stack([lo, hi], axis=-1).reshape(E, N, 2 * half)
    sc = s.view(np.float16).astype(np.float64)
    return qq * np.repeat(sc, 32, axis=-1)


def dense_forward(layer, x_bits):
    """Every expert on every token, then the top-k mask: the brute-force
    dense evaluation of the layer."""
    x = bf16_bits_to_f64(x_bits)
    l = x @ layer.router_w.astype(np.float64).T
    if layer.router_bias is not None:
        l = l + layer.router_bias.astype(np.float64)[None, :]
    T, E = l.shape
    K = layer.top_k
    G, U, D = (np_dequant(layer.routed, r) for r in ("gate", "up", "down"))
    g = np.einsum("th,efh->tef", x, G)
    u = np.einsum("th,efh->tef", x, U)
    a = g / (1.0 + np.exp(-g)) * u
    o = np.einsum("tef,ehf->teh", a, D)
    y = np.zeros((T, layer.hidden))
    sel_all = np.zeros((T, K), np.int64)
    for t in range(T):
        p = np.exp(l[t] - l[t].max())
        p /= p.sum()
        order = np.lexsort((np.arange(E), -l[t]))
        sel = order[:K]
        sel_all[t] = sel
        mask = np.zeros(E)
        mask[sel] = p[sel] / p[sel].sum() if layer.renorm else p[sel]
        y[t] = (mask[:, None] * o[t]).sum(axis=0)
    if layer.shared is not None:
        Gs, Us, Ds = (np_dequant(layer.shared, r)[0] for r in ("gate", "up", "down"))
        gs = x @ Gs.T
        us = x @ Us.T
        y += (gs / (1.0 + np.exp(-gs)) * us) @ Ds.T
    return y, sel_all


def tiny_layer(fmt, H, F, E, K, shared_F=0, seed=7, renorm=1, jitter=True, bias=False):
    shape = synth.Shape(tokens=3, hidden=H, n_experts=E, top_k=K, ffn=F, shared_ffn=shared_F, fmt=fmt,
                        renorm=renorm, jitter_scales=jitter, seed=seed)
    layer = synth.make_layer(shape)
    if bias:
        layer.router_bias = synth.normal_f32(seed, 99, E, 0.0, 0.5)
    return shape, layer


def rel_err(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ----------------------------------------------------------- IEEE decoders

def test_bf16_decoder_matches_numpy_on_all_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_double(b) for b in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero survives
    assert math.copysign(1.0, oracle.bf16_to_double(0x8000)) == -1.0


def test_f16_decoder_matches_numpy_on_all_patterns():
    ref = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(b) for b in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _rne_f32_bits(f32):
    b = np.asarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_rounding_ties_to_even_hand_cases():
    one = 0x3F80
    assert oracle.double_to_bf16(1.0) == one
    assert oracle.double_to_bf16(1.0 + 2.0 ** -8) == one  # exact tie -> even (fraction 0)
    assert oracle.double_to_bf16(1.0 + 3 * 2.0 ** -8) == one + 2  # tie between 1+2^-7 and 1+2^-6 -> even
    assert oracle.double_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == one + 1  # just above the tie
    assert oracle.double_to_bf16(-2.5) == 0xC020
    assert oracle.double_to_bf16(2.0 ** -133) == 0x0001  # smallest subnormal
    assert oracle.double_to_bf16(3.5e38) == 0x7F80  # overflow -> inf
    assert oracle.double_to_bf16(0.0) == 0


def test_bf16_rounding_matches_bit_trick_on_float32_values():
    rng = np.random.default_rng(0)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = _rne_f32_bits(f)
    got = np.array([oracle.double_to_bf16(float(v)) for v in f], np.uint16)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------- weight formats

def test_int4_nibble_layout_hand_bytes():
    # one row, Kin = 64: two 32-element blocks with scales 1.0 and 2.0
    q = np.full((1, 1, 32), 0x88, np.uint8)  # every element q = 0
    q[0, 0, 0] = 0x9F  # element 0 = 0xF - 8 = 7, element 1 = 0x9 - 8 = 1
    q[0, 0, 1] = 0x1E  # element 2 = 0xE - 8 = 6, element 3 = 0x1 - 8 = -7
    q[0, 0, 16] = 0x7A  # element 32 = 2 (block 1, x2), element 33 = -1 (x2)
    s = np.array([[[0x3C00, 0x4000]]], np.uint16)  # 1.0, 2.0
    W, rc = oracle.dequant(2, q, s, 1, 1, 64)
    assert rc == 0
    expect = np.zeros(64)
    expect[[0, 1, 2, 3]] = [7, 1, 6, -7]
    expect[[32, 33]] = [4, -2]
    assert np.array_equal(W[0, 0], expect)


def test_int4_forbidden_nibble_zero():
    q = np.full((1, 1, 16), 0x88, np.uint8)
    q[0, 0, 3] = 0x80  # element 6 has nibble 0 (q = -8)
    s = np.full((1, 1, 1), 0x3C00, np.uint16)
    W, rc = oracle.dequant(2, q, s, 1, 1, 32)
    assert rc == -1 and np.isnan(W[0, 0, 6]) and W[0, 0, 7] == 0.0


def test_int4_round_trip_every_value_and_parity():
    # pack every q in [-7, 7] at both nibble positions with a test-side packer
    vals = np.arange(-7, 8)
    elems = np.concatenate([vals, vals[::-1], np.zeros(2, np.int64)])  # 32 elements
    packed = ((elems[0::2] + 8) | ((elems[1::2] + 8) << 4)).astype(np.uint8)
    W, rc = oracle.dequant(2, packed.reshape(1, 1, 16), np.full((1, 1, 1), 0x3C00, np.uint16), 1, 1, 32)
    assert rc == 0 and np.array_equal(W[0, 0], elems.astype(np.float64))


def test_int8_dequant_exact_and_row_scale_index():
    rng = np.random.default_rng(1)
    q = rng.integers(-127, 128, size=(3, 5, 7), dtype=np.int8)
    s = rng.uniform(0.5, 1.5, size=(3, 5)).astype(np.float32)
    W, rc = oracle.dequant(1, q, s, 3, 5, 7)
    assert rc == 0
    assert np.array_equal(W, q.astype(np.float64) * s.astype(np.float64)[..., None])


def test_generated_int4_scales_index_by_block():
    shape, layer = tiny_layer(synth.FMT_INT4_B32, 64, 32, 4, 2)
    W, rc = oracle.dequant(2, layer.routed.gate_q, layer.routed.gate_s, 4, 32, 64)
    assert rc == 0
    assert np.array_equal(W, np_dequant(layer.routed, "gate"))


# ----------------------------------------------------------- router

def test_logits_one_hot_inputs_pick_router_columns():
    shape, layer = tiny_layer(synth.FMT_INT8_ROW, 32, 16, 6, 2, bias=True)
    H = 32
    x = np.zeros((H, H), np.uint16)
    for h in range(H):
        x[h, h] = 0x3F80  # 1.0
    l = oracle.router_logits(layer, x)
    expect = layer.router_w.astype(np.float64).T + layer.router_bias.astype(np.float64)[None, :]
    assert np.array_equal(l, expect)


def test_select_against_full_lexsort_and_ties():
    rng = np.random.default_rng(2)
    T, E, K = 50, 64, 8
    l = rng.standard_normal((T, E))
    # plant exact ties, including one straddling the K-th place
    l[0, 10] = l[0, 3]
    l[1, :] = 0.25
    srt = np.sort(l[2])[::-1]
    l[2, np.where(l[2] == srt[K])[0][0]] = srt[K - 1]
    ids, w = oracle.select(l, K)
    for t in range(T):
        ref = np.lexsort((np.arange(E), -l[t]))[:K]
        assert np.array_equal(ids[t], ref)
        chosen = set(ids[t].tolist())
        rest = [l[t, e] for e in range(E) if e not in chosen]
        assert min(l[t, ids[t]]) >= max(rest)
        assert len(chosen) == K
    assert np.array_equal(ids[1], np.arange(K))  # all tied -> lowest indices in order


def test_weights_closed_forms():
    rng = np.random.default_rng(3)
    T, E, K = 20, 32, 4
    l = rng.standard_normal((T, E)) * 3
    ids, w = oracle.select(l, K, renorm=1)
    ids0, w0 = oracle.select(l, K, renorm=0)
    assert np.array_equal(ids, ids0)
    for t in range(T):
        p = np.exp(l[t]) / np.exp(l[t]).sum()  # full softmax, no shift
        assert np.allclose(w0[t], p[ids[t]], rtol=1e-13, atol=0)
        assert np.allclose(w[t], p[ids[t]] / p[ids[t]].sum(), rtol=1e-13, atol=0)
        assert abs(w[t].sum() - 1.0) <= 1e-12
        assert np.all(np.diff(w[t]) <= 0)
    _, w1 = oracle.select(l, 1, renorm=1)
    assert np.all(w1 == 1.0)


# ----------------------------------------------------------- permutation

def test_permute_brute_force_and_invariants():
    rng = np.random.default_rng(4)
    T, K, E = 37, 4, 16
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(size=(T, K)).astype(np.float32)
    p = oracle.permute(ids, w, E)
    assert np.array_equal(p["counts"], np.bincount(ids.ravel(), minlength=E))
    assert p["offsets"][0] == 0 and p["offsets"][-1] == T * K
    assert np.array_equal(np.diff(p["offsets"]), p["counts"])
    rows = []
    for e in range(E):
        for t in range(T):
            for k in range(K):
                if ids[t, k] == e:
                    rows.append((t, k))
    assert len(rows) == T * K
    for r, (t, k) in enumerate(rows):
        assert p["row_tok"][r] == t
        assert p["row_w"][r] == w[t, k]
        assert p["inv_pos"][t, k] == r
    assert np.array_equal(p["active"], np.flatnonzero(p["counts"]))
    assert p["n_active"] == np.count_nonzero(p["counts"])


def test_permute_one_expert_takes_everything():
    ids = np.zeros((9, 1), np.int32) + 5
    p = oracle.permute(ids, None, 8)
    assert list(p["counts"]) == [0, 0, 0, 0, 0, 9, 0, 0]
    assert list(p["offsets"]) == [0, 0, 0, 0, 0, 0, 9, 9, 9]
    assert list(p["row_tok"]) == list(range(9))
    assert list(p["active"]) == [5]


# ----------------------------------------------------------- whole layer

def test_hand_micro_case():
    g = json.load(open(os.path.join(GOLDEN, "micro_case.json")))
    H, F, E = 4, 2, 2
    ex = g["experts"]
    s = np.float32(ex["scale"])
    routed = ExpertsHost(synth.FMT_INT8_ROW, E, H, F,
                         np.array(ex["gate_q"], np.int8), np.full((E, F), s, np.float32),
                         np.array(ex["up_q"], np.int8), np.full((E, F), s, np.float32),
                         np.array(ex["down_q"], np.int8), np.full((E, H), s, np.float32))
    layer = LayerHost(H, E, 1, 1, np.array(g["router_w"], np.float32), None, routed)
    x = synth.f64_to_bf16(np.array([g["x"]]))
    y, ids, w, logits = oracle.layer_forward(layer, x)
    assert np.array_equal(logits[0], g["logits"])
    assert ids[0, 0] == g["selected"] and w[0, 0] == g["weight"]
    assert np.allclose(y[0], g["y"], rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("renorm", [1, 0])
def test_dense_brute_force_config0(renorm):
    shape = synth.CONFIGS[0]
    shape = synth.Shape(**{**shape.__dict__, "renorm": renorm})
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    y, ids, w, _ = oracle.layer_forward(layer, x)
    yd, sel = dense_forward(layer, x)
    assert np.array_equal(ids, sel)
    assert rel_err(y, yd) <= 1e-12


@pytest.mark.parametrize("fmt", [synth.FMT_INT8_ROW, synth.FMT_INT4_B32])
def test_dense_brute_force_with_shared_bias_and_jitter(fmt):
    shape, layer = tiny_layer(fmt, 96, 64, 12, 3, shared_F=32, bias=True)
    x = synth.normal_bf16(11, 1, 5 * 96).reshape(5, 96)
    y, ids, w, _ = oracle.layer_forward(layer, x, nthreads=2)
    yd, sel = dense_forward(layer, x)
    assert np.array_equal(ids, sel)
    assert rel_err(y, yd) <= 1e-12


def test_k_equals_e_is_dense_softmax_moe():
    shape, layer = tiny_layer(synth.FMT_INT4_B32, 64, 32, 6, 6)
    x = synth.normal_bf16(12, 1, 4 * 64).reshape(4, 64)
    y, ids, w, logits = oracle.layer_forward(layer, x)
    xf = bf16_bits_to_f64(x)
    G, U, D = (np_dequant(layer.routed, r) for r in ("gate", "up", "down"))
    for t in range(4):
        p = np.exp(logits[t] - logits[t].max())
        p /= p.sum()
        acc = np.zeros(64)
        for e in range(6):
            g = G[e] @ xf[t]
            u = U[e] @ xf[t]
            acc += p[e] * (D[e] @ (g / (1 + np.exp(-g)) * u))
        assert rel_err(y[t], acc) <= 1e-12


def test_zero_gate_row_contributes_nothing():
    shape, layer = tiny_layer(synth.FMT_INT8_ROW, 32, 8, 4, 2)
    x = synth.normal_bf16(13, 1, 3 * 32).reshape(3, 32)
    layer.routed.gate_q[:, 5, :] = 0
    y1, *_ = oracle.layer_forward(layer, x)
    layer.routed.down_q[:, :, 5] = 99  # column 5 of every down matrix is now irrelevant
    y2, *_ = oracle.layer_forward(layer, x)
    assert np.array_equal(y1, y2)


def test_zero_routed_weights_leave_the_shared_expert():
    shape, layer = tiny_layer(synth.FMT_INT8_ROW, 32, 8, 4, 2, shared_F=16)
    x = synth.normal_bf16(14, 1, 3 * 32).reshape(3, 32)
    layer.routed.gate_q[:] = 0
    y, *_ = oracle.layer_forward(layer, x)
    xf = bf16_bits_to_f64(x)
    Gs, Us, Ds = (np_dequant(layer.shared, r)[0] for r in ("gate", "up", "down"))
    g, u = xf @ Gs.T, xf @ Us.T
    assert rel_err(y, (g / (1 + np.exp(-g)) * u) @ Ds.T) <= 1e-13
    layer.shared = None
    y0, *_ = oracle.layer_forward(layer, x)
    assert np.all(y0 == 0.0)


def test_selection_override_reweights_from_logits():
    shape, layer = tiny_layer(synth.FMT_INT8_ROW, 32, 8, 6, 2)
    x = synth.normal_bf16(15, 1, 2 * 32).reshape(2, 32)
    y, ids, w, logits = oracle.layer_forward(layer, x)
    y_same, ids_same, w_same, _ = oracle.layer_forward(layer, x, ids=ids)
    assert np.array_equal(y, y_same) and np.array_equal(w, w_same)
    other = np.array([[5, 0], [1, 4]], np.int32)
    y2, ids2, w2, _ = oracle.layer_forward(layer, x, ids=other)
    assert np.array_equal(ids2, other)
    for t in range(2):
        p = np.exp(logits[t, other[t]])
        assert np.allclose(w2[t], p / p.sum(), rtol=1e-14)


def test_expert_rows_sum_back_to_the_layer():
    shape, layer = tiny_layer(synth.FMT_INT4_B32, 64, 32, 8, 3)
    x = synth.normal_bf16(16, 1, 5 * 64).reshape(5, 64)
    y, ids, w, _ = oracle.layer_forward(layer, x)
    p = oracle.permute(ids, w.astype(np.float32), 8)
    rows = oracle.expert_rows(layer.routed, x, p["offsets"], p["row_tok"], p["row_w"])
    # the layer weights in double; rows carry float32 weights, so compare loosely
    recon = rows[p["inv_pos"]].sum(axis=1)
    assert rel_err(recon, y) <= 1e-6


def test_residual_rounds_to_nearest_even():
    x = synth.f64_to_bf16(np.array([1.0, 1.0, -3.0, 0.0]))
    y = np.array([2.0 ** -8, 3 * 2.0 ** -8, 0.0078125, 1e-40])
    out = oracle.residual(x, y)
    # -3 + 2^-7 sits halfway between -3 + 2^-6 (odd) and -3 (even); 1e-40 is
    # about 1.09 subnormal bf16 steps (2^-133)
    assert list(out) == [0x3F80, 0x3F82, 0xC040, 0x0001]


def test_rmsnorm_closed_forms():
    # a constant row c normalises to c / sqrt(c^2 + eps); alternating +-v to +-v / sqrt(v^2 + eps)
    H = 64
    r = np.zeros((3, H), np.uint16)
    r[0] = synth.f64_to_bf16(np.full(H, 3.0))
    r[1] = synth.f64_to_bf16(np.tile([2.0, -2.0], H // 2))
    r[2] = synth.f64_to_bf16(np.r_[np.full(H // 2, 1.0), np.full(H // 2, 7.0)])  # mean square 25
    out = oracle.rmsnorm(r, eps=0.0)
    f = bf16_bits_to_f64(out)
    assert np.all(f[0] == 1.0)
    assert np.all(f[1] == np.tile([1.0, -1.0], H // 2))
    assert np.all(f[2] == np.r_[np.full(H // 2, 0.2), np.full(H // 2, 1.4)].astype(np.float32).astype(
        np.float64)) or np.allclose(f[2], np.r_[np.full(H // 2, 0.2), np.full(H // 2, 1.4)], rtol=2 ** -8)
    out_eps = oracle.rmsnorm(r[:1], eps=7.0)  # 3 / sqrt(9 + 7) = 0.75 exactly
    assert np.all(bf16_bits_to_f64(out_eps) == 0.75)


# ----------------------------------------------------------- variants
# The shared expert's sigmoid gate ("Qwen3.6-35B-A3B: pictures, several
# requests at once and speed", Speed (0.1.45)), tail-skip ("Models and
# backends", What was tuned) and int8 activations (the W8A8 variant, "Strata
# on an Intel Arc", Arc Pro B70: the fused int8 expert path for the prompt).

def np_quantize_row(v):
    """Independent numpy float32 statement of the per-row quantiser."""
    v = np.asarray(v, np.float32)
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    if amax == 0:
        return np.zeros(v.shape, np.int8), np.float32(0)
    inv = np.float32(127) / amax
    d = amax / np.float32(127)
    q = np.clip(np.rint(v * inv), -127, 127).astype(np.int8)  # v * inv in float32, rint ties to even
    return q, d


def dense_forward_variant(layer, x_bits, tail_skip=0, act_quant=0):
    """Every expert on every token in numpy float64 (independent of the
    oracle), then the top-k mask, the tail-skip rule over the whole call and
    the shared gate; with act_quant the inputs of the gate/up and down
    products are quantised per row with np_quantize_row."""
    x = bf16_bits_to_f64(x_bits)
    T = x.shape[0]
    l = x @ layer.router_w.astype(np.float64).T
    if layer.router_bias is not None:
        l = l + layer.router_bias.astype(np.float64)[None, :]
    E, K = l.shape[1], layer.top_k
    sel = np.stack([np.lexsort((np.arange(E), -l[t]))[:K] for t in range(T)])
    keep = np.ones(E, bool)
    if tail_skip > 0:
        keep[:] = False
        keep[np.unique(sel[:, :tail_skip])] = True

    def qd(v):
        q, d = np_quantize_row(v.astype(np.float32))
        return q.astype(np.float64) * np.float64(d)

    def expert(ex, e, xt):
        G, U, D = (np_dequant(ex, r)[e] for r in ("gate", "up", "down"))
        xi = qd(xt) if act_quant else xt
        g, u = G @ xi, U @ xi
        a = g / (1.0 + np.exp(-g)) * u
        if act_quant:
            a = qd(a)
        return D @ a

    y = np.zeros((T, layer.hidden))
    for t in range(T):
        lv = l[t, sel[t]]
        w = np.exp(lv - lv[0])
        w /= w.sum()
        for k in range(K):
            if keep[sel[t, k]]:
                y[t] += w[k] * expert(layer.routed, sel[t, k], x[t])
        if layer.shared is not None:
            gate = 1.0
            if layer.shared_gate_w is not None:
                gate = 1.0 / (1.0 + np.exp(-(x[t] @ layer.shared_gate_w.astype(np.float64))))
            y[t] += gate * expert(layer.shared, 0, x[t])
    return y, sel, keep


def test_quantizer_hand_cases():
    g = json.load(open(os.path.join(GOLDEN, "int8_row_quant_cases.json")))
    for c in g["cases"]:
        q, d = oracle.quantize_row(np.array(c["v"], np.float32))
        assert q.tolist() == c["q"], c["note"]
        assert d == np.float32(c["d_num"]) / np.float32(c["d_den"]), c["note"]


def test_quantizer_against_numpy_and_invariants():
    rng = np.random.default_rng(21)
    for n, scale in ((2048, 1.0), (512, 3e-3), (33, 250.0), (7, 1e-30)):
        for _ in range(20):
            v = (rng.standard_normal(n) * scale).astype(np.float32)
            q, d = oracle.quantize_row(v)
            qn, dn = np_quantize_row(v)
            assert np.array_equal(q, qn) and d == dn
            i = int(np.argmax(np.abs(v)))
            assert abs(int(q[i])) == 127 and np.sign(q[i]) == np.sign(v[i])
            assert np.all(np.abs(q.astype(np.float64) * d - v) <= 0.5 * d * (1 + 2.0 ** -20))
            # a power-of-two rescale changes the scale, never the codes
            q2, d2 = oracle.quantize_row(v * np.float32(4.0))
            assert np.array_equal(q2, q) and d2 == d * 4


@pytest.mark.parametrize("fmt", [synth.FMT_INT8_ROW, synth.FMT_INT4_B32])
def test_w8a8_variant_dense_brute_force(fmt):
    shape, layer = tiny_layer(fmt, 96, 64, 12, 3, shared_F=32, bias=True)
    x = synth.normal_bf16(31, 1, 5 * 96).reshape(5, 96)
    y, ids, w, _ = oracle.layer_forward(layer, x, act_quant=1)
    yd, sel, _ = dense_forward_variant(layer, x, act_quant=1)
    assert np.array_equal(ids, sel)
    assert rel_err(y, yd) <= 1e-12
    # the quantisation is visible against the exact layer, at the size an
    # 8-bit grid implies (about 1% of the output scale, never 0)
    y0, _, _, _ = oracle.layer_forward(layer, x)
    assert 1e-4 < rel_err(y, y0) < 5e-2


def test_w8a8_variant_is_exact_on_the_int8_grid_input():
    """When x already lies on its int8 grid (integers with max |x| = 127),
    quantising it changes nothing: the gate/up products equal the exact
    layer's, so the variant differs only through the SwiGLU row's grid."""
    shape, layer = tiny_layer(synth.FMT_INT8_ROW, 64, 32, 6, 2, shared_F=0)
    rng = np.random.default_rng(3)
    xi = rng.integers(-127, 128, size=(2, 64)).astype(np.float64)
    xi[:, 0] = 127
    x = synth.f64_to_bf16(xi)
    q, d = oracle.quantize_row(bf16_bits_to_f64(x[0]).astype(np.float32))
    assert d == 1.0 and np.array_equal(q.astype(np.float64), xi[0])
    y, _, _, _ = oracle.layer_forward(layer, x, act_quant=1)
    yd, _, _ = dense_forward_variant(layer, x, act_quant=1)
    assert rel_err(y, yd) <= 1e-12


@pytest.mark.parametrize("N", [1, 2, 3])
def test_tail_skip_dense_brute_force(N):
    """Config 0 (4 tokens, top-4 of 64): the experts computed are those some
    token ranks among its first N; the others are left out and nothing is
    renormalised."""
    shape = synth.CONFIGS[0]
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    y, ids, w, _ = oracle.layer_forward(layer, x, tail_skip=N)
    yd, sel, keep = dense_forward_variant(layer, x, tail_skip=N)
    assert np.array_equal(ids, sel)
    assert rel_err(y, yd) <= 1e-12
    # the weights stay the router's (they still sum to 1 over all K slots)
    assert np.all(np.abs(w.sum(axis=1) - 1) <= 1e-12)
    dropped = ~keep[sel]
    assert dropped.any(), "the case should leave some slot out"
    assert not dropped[:, :N].any()


def test_tail_skip_keeps_a_late_slot_another_token_ranks_early():
    """Tail-skip looks at the whole call: a token's 4th pick is computed when
    another token of the call ranks that expert first, and left out when the
    token is alone."""
    shape = synth.CONFIGS[0]
    layer = synth.make_layer(shape)
    found = False
    for seed in range(200):
        x = synth.make_x(shape, seed=1000 + seed)
        l = bf16_bits_to_f64(x) @ layer.router_w.astype(np.float64).T
        sel = np.stack([np.lexsort((np.arange(shape.n_experts), -l[t]))[:shape.top_k] for t in range(4)])
        first = set(sel[:, 0].tolist())
        late = [(t, k) for t in range(4) for k in range(1, 4) if sel[t, k] in first]
        if late:
            t, k = late[0]
            found = True
            break
    assert found
    y_call, _, _, _ = oracle.layer_forward(layer, x, tail_skip=1)
    y_alone, _, _, _ = oracle.layer_forward(layer, x[t:t + 1], tail_skip=1)
    y_plain, _, _, _ = oracle.layer_forward(layer, x[t:t + 1])
    assert rel_err(y_call[t], y_alone[0]) > 1e-6  # the call kept slot k, the lone token did not
    yd, _, _ = dense_forward_variant(layer, x, tail_skip=1)
    assert rel_err(y_call, yd) <= 1e-12
    del y_plain


def test_tail_skip_at_or_beyond_k_is_the_plain_layer():
    shape = synth.CONFIGS[0]
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    y0, _, _, _ = oracle.layer_forward(layer, x)
    for N in (shape.top_k, shape.top_k + 3):
        y, _, _, _ = oracle.layer_forward(layer, x, tail_skip=N)
        assert np.array_equal(y, y0)


def _gated_pair(gate_w, x=None):
    shape, layer = tiny_layer(synth.FMT_INT4_B32, 64, 32, 6, 2, shared_F=32)
    if x is None:
        x = synth.normal_bf16(41, 1, 3 * 64).reshape(3, 64)
    y_plain, _, _, _ = oracle.layer_forward(layer, x)
    no_shared = LayerHost(layer.hidden, layer.n_experts, layer.top_k, layer.renorm, layer.router_w,
                          layer.router_bias, layer.routed, None)
    y_routed, _, _, _ = oracle.layer_forward(no_shared, x)
    layer.shared_gate_w = None if gate_w is None else np.asarray(gate_w(x), np.float32)
    y_gated, _, _, _ = oracle.layer_forward(layer, x)
    return layer, x, y_plain, y_routed, y_gated


def test_shared_gate_zero_row_halves_the_shared_expert():
    _, _, y_plain, y_routed, y_gated = _gated_pair(lambda x: np.zeros(64))
    assert rel_err(y_gated, 0.5 * (y_plain + y_routed)) <= 1e-12


def test_shared_gate_saturates_to_on_and_off():
    """A gate row along token 0's own input gives a logit of +-|x|^2 / 2
    (about 30): the gate is 1 (or 0) to double precision, i.e. the plain
    layer (or the routed experts alone)."""
    _, x, y_plain, y_routed, y_on = _gated_pair(lambda x: 0.5 * bf16_bits_to_f64(x[0]))
    assert rel_err(y_on[0], y_plain[0]) <= 1e-12
    _, _, _, _, y_off = _gated_pair(lambda x: -0.5 * bf16_bits_to_f64(x[0]))
    assert rel_err(y_off[0], y_routed[0]) <= 1e-12


def test_shared_gate_three_quarters():
    """A gate logit of ln 3 (a row along the token's input scaled to it)
    gives sigmoid = 3/4: y = routed + 3/4 shared = (y_routed + 3 y_plain)/4.
    A sign slip (sigmoid(-z) = 1/4) fails."""
    def row(x):
        xf = bf16_bits_to_f64(x[1])
        return xf * (math.log(3.0) / float(xf @ xf))
    _, _, y_plain, y_routed, y_g = _gated_pair(row)
    assert rel_err(y_g[1], 0.25 * y_routed[1] + 0.75 * y_plain[1]) <= 1e-6
    shape, layer = tiny_layer(synth.FMT_INT4_B32, 64, 32, 6, 2, shared_F=32)
    x = synth.normal_bf16(41, 1, 3 * 64).reshape(3, 64)
    layer.shared_gate_w = np.asarray(row(x), np.float32)
    yd, _, _ = dense_forward_variant(layer, x)
    assert rel_err(y_g, yd) <= 1e-12
