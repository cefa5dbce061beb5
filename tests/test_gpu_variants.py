"""GPU parity of the layer's variants against the oracle's modes: the shared
expert's sigmoid gate (its row formed with the router's product) and
tail-skip on decode batches.  Every expected value comes from the oracle
run on the same seeded inputs."""
import sys

import numpy as np
import pytest

from mixture_experts_decode_moe_amd import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mb():
    import torch  # noqa: F401
    from mixture_experts_decode_moe_amd import binding
    return binding


def _shape(cfg, **kw):
    base = synth.CONFIGS[cfg]
    return synth.Shape(**{**base.__dict__, **kw})


# ------------------------------------------------------------ shared gate

@pytest.mark.parametrize("cfg,T,extra,path", [
    (1, 1, {}, "auto"),       # int8, one-launch down + combine
    (2, 2, {}, "auto"),       # int4 MTP verify
    (2, 12, {}, "auto"),      # two-launch down and combine
    (2, 64, {}, "auto"),      # prefill GEMMs: the gate formed in the top-k launch
    (2, 40, {}, "decode"),    # the generic router kernel with the gate row beside the router rows
    (0, 4, {"n_experts": 512, "shared_ffn": 256}, "auto"),  # E > 256: routing in a block of its own
])
def test_shared_gate_layer_parity(mb, cfg, T, extra, path):
    import parity_util as pu
    shape = _shape(cfg, tokens=T, correlated_sigma=0.0, shared_gate=True, seed=700 + T + cfg, **extra)
    layer = synth.make_layer(shape)
    assert layer.shared_gate_w is not None
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    say(f"shared gate cfg{cfg} T={T} {extra} path {path}")
    if path == "auto":
        gpu = pu.run_layer(dl, pu.dev_u16(x), T)
    else:
        gpu = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False, opts=mb.forward_opts(path))
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    say(f"  rel err {err:.2e}, near ties {ties}")


def test_shared_gate_from_moe_route(mb):
    """moe_route's shared gate output is sigmoid(g . x) per token (float32
    product against the oracle's double one), on both router kernels."""
    import torch
    import parity_util as pu
    for T in (5, 40):
        shape = _shape(2, tokens=T, correlated_sigma=0.0, shared_gate=True, seed=750 + T)
        layer = synth.make_layer(shape)
        x = synth.make_x(shape)
        dl = mb.layer_to_device(layer)
        ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, shape.top_k), dtype=torch.float32, device="cuda")
        lg = torch.empty((T, shape.n_experts), dtype=torch.float32, device="cuda")
        g = torch.empty(T, dtype=torch.float32, device="cuda")
        mb.route(dl, pu.dev_u16(x), ids, w, lg, shared_gate=g)
        torch.cuda.synchronize()
        z = pu.bf16_to_f64(x) @ layer.shared_gate_w.astype(np.float64)
        ref = 1.0 / (1.0 + np.exp(-z))
        d = np.max(np.abs(g.cpu().numpy() - ref))
        say(f"moe_route shared gate T={T}: max |dg| {d:.2e}")
        assert d <= 1e-5


def test_shared_gate_one_and_two_launch_paths_same_bits(mb):
    import parity_util as pu
    shape = _shape(2, tokens=12, correlated_sigma=0.0, shared_gate=True, seed=760)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    say("shared gate: one-launch vs two-launch bits")
    full = pu.run_layer(dl, pu.dev_u16(x), 12, with_logits=False)
    for T in (1, 5, 8):
        part = pu.run_layer(dl, pu.dev_u16(x[:T]), T, with_logits=False)
        assert np.array_equal(part["y"], full["y"][:T]), f"T={T}"


# ------------------------------------------------------------ tail-skip

def _check_tail_skip(mb, layer, x, T, N, opts_path="auto"):
    """The GPU call with tail-skip N against the oracle's tail-skip mode on
    the GPU's own selection (identical to the oracle's away from near ties,
    checked), outputs within the tolerance."""
    import oracle
    import parity_util as pu
    dl = mb.layer_to_device(layer)
    gpu = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False, opts=mb.forward_opts(opts_path, tail_skip=N))
    y_sel, ids_ref, w_ref, logits_ref = oracle.layer_forward(layer, x)
    pu.check_selection(gpu["ids"], ids_ref, logits_ref, layer.top_k)
    y_ref, _, _, _ = oracle.layer_forward(layer, x, ids=gpu["ids"], tail_skip=N)
    err = pu.rel_max_err(gpu["y"], y_ref)
    plain, _, _, _ = oracle.layer_forward(layer, x, ids=gpu["ids"])
    moved = pu.rel_max_err(y_ref, plain)
    say(f"  N={N}: rel err {err:.2e} (tail-skip moves the output by {moved:.2e})")
    assert err <= pu.Y_REL
    return gpu, moved


@pytest.mark.parametrize("T,N", [(1, 6), (2, 6), (2, 7), (5, 5), (16, 6), (16, 3)])
def test_tail_skip_decode_parity(mb, T, N):
    """Decode batches of the 256-expert int4 layer with Zipf-popular experts
    (config 3's first layer)."""
    shape = _shape(3, tokens=T, layers=1, seed=800 + T)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    say(f"tail-skip T={T} N={N}")
    _, moved = _check_tail_skip(mb, layer, x, T, N)
    if T <= 2:
        assert moved > 1e-4, "the case should leave some expert out"


def test_tail_skip_more_than_256_experts(mb):
    shape = _shape(0, n_experts=512, top_k=8, seed=820)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    say("tail-skip E=512 T=4 N=4")
    _check_tail_skip(mb, layer, x, 4, 4)


def test_tail_skip_int8_one_launch(mb):
    shape = _shape(1, tokens=3, seed=830)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    say("tail-skip int8 T=3 N=5")
    _check_tail_skip(mb, layer, x, 3, 5)


def test_tail_skip_leaves_prompt_batches_alone(mb):
    """A 40-token call is a prompt batch: tail-skip does not touch it (the
    bits equal the call without it)."""
    import parity_util as pu
    shape = _shape(2, tokens=40, correlated_sigma=0.0, seed=840)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    say("tail-skip on a 40-token prompt batch")
    a = pu.run_layer(dl, pu.dev_u16(x), 40, with_logits=False)
    b = pu.run_layer(dl, pu.dev_u16(x), 40, with_logits=False, opts=mb.forward_opts(tail_skip=4))
    assert np.array_equal(a["y"], b["y"])


def test_tail_skip_at_k_is_the_plain_layer(mb):
    import parity_util as pu
    shape = _shape(3, tokens=7, layers=1, seed=850)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    say("tail-skip N=K gives the plain layer's bits")
    a = pu.run_layer(dl, pu.dev_u16(x), 7, with_logits=False)
    b = pu.run_layer(dl, pu.dev_u16(x), 7, with_logits=False, opts=mb.forward_opts(tail_skip=shape.top_k))
    assert np.array_equal(a["y"], b["y"])


def test_tail_skip_with_shared_gate_and_residual_norm(mb):
    """Both variants together on the two-launch path (residual epilogue with
    the normalised copy)."""
    import oracle
    import parity_util as pu
    T, N = 6, 5
    shape = _shape(3, tokens=T, layers=1, shared_gate=True, seed=860)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    r = synth.make_x(shape, seed=861)
    dl = mb.layer_to_device(layer)
    say("tail-skip + shared gate + residual/norm, T=6")
    r_dev = pu.dev_u16(r)
    gpu = pu.run_layer(dl, pu.dev_u16(x), T, residual=r_dev, with_logits=False,
                       opts=mb.forward_opts(tail_skip=N))
    y_ref, _, _, _ = oracle.layer_forward(layer, x, ids=gpu["ids"], tail_skip=N)
    assert pu.rel_max_err(gpu["y"], y_ref) <= pu.Y_REL
    assert np.array_equal(gpu["residual_out"], pu.residual_expected(r, gpu["y"]))


# ------------------------------------------------------------ W8A8

def _check_w8a8(mb, layer, x, T, path="auto"):
    """The W8A8 call against the oracle's int8-activation mode on the GPU's
    own selection (identical to the oracle's away from near ties, checked)."""
    import oracle
    import parity_util as pu
    dl = mb.layer_to_device(layer)
    gpu = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False, opts=mb.forward_opts(path, act_quant=1))
    _, ids_ref, _, logits_ref = oracle.layer_forward(layer, x)
    pu.check_selection(gpu["ids"], ids_ref, logits_ref, layer.top_k)
    y_ref, _, _, _ = oracle.layer_forward(layer, x, ids=gpu["ids"], act_quant=1)
    err = pu.rel_max_err(gpu["y"], y_ref)
    exact, _, _, _ = oracle.layer_forward(layer, x, ids=gpu["ids"])
    moved = pu.rel_max_err(y_ref, exact)
    say(f"  W8A8 T={T}: rel err {err:.2e} against the W8A8 oracle (quantisation moves the output by {moved:.2e})")
    assert err <= pu.Y_REL
    assert moved > 1e-4  # the variant is really quantised
    return gpu


@pytest.mark.parametrize("T,jitter", [(3, False), (40, True), (300, True)])
def test_w8a8_parity_real_shape(mb, T, jitter):
    """int8 weights at the real shape (H=2048, 256 experts, top-8, F=512 +
    shared expert), int8 activations."""
    shape = _shape(1, tokens=T, jitter_scales=jitter, seed=900 + T)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    say(f"W8A8 cfg1 shape T={T} jitter={jitter}")
    _check_w8a8(mb, layer, x, T)


def test_w8a8_parity_small_layer_with_gate_no_shared(mb):
    """H=1024, 64 experts, top-4, F=256: no shared expert, bias routing."""
    shape = _shape(0, tokens=70, seed=910, jitter_scales=True)
    layer = synth.make_layer(shape)
    layer.router_bias = synth.normal_f32(910, 99, shape.n_experts, 0.0, 0.5)
    x = synth.make_x(shape)
    say("W8A8 H=1024 E=64 K=4 F=256 T=70")
    _check_w8a8(mb, layer, x, 70)


def test_w8a8_with_shared_gate(mb):
    shape = _shape(1, tokens=33, seed=920, shared_gate=True)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    say("W8A8 with the shared gate, T=33")
    _check_w8a8(mb, layer, x, 33)


def test_w8a8_refuses_int4_weights(mb):
    import torch
    shape = _shape(2, tokens=4, correlated_sigma=0.0, seed=930)
    dl = mb.layer_to_device(synth.make_layer(shape))
    ws = mb.make_workspace(dl, 4)
    x = torch.zeros((4, shape.hidden), dtype=torch.int16, device="cuda")
    y = torch.empty((4, shape.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(mb.MoeError) as ei:
        mb.layer_forward(dl, x, y, ws, opts=mb.forward_opts(act_quant=1))
    assert ei.value.status == mb.MOE_ERR_UNSUPPORTED
