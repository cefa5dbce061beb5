"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Every input comes from the seeded generator; every expected value from the
oracle.  Selection must match except at near ties (8th and 9th logits within
1e-4), routing weights within 1e-6, outputs within 2e-3 of max|ref| per layer
call.  Larger configurations are checked on sampled tokens the oracle can
evaluate one by one.
"""
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


@pytest.mark.parametrize("cfg,variant", [(0, {}), (0, {"jitter_scales": True}), (0, {"renorm": 0}),
                                         (1, {}), (1, {"jitter_scales": True}), (2, {})])
def test_layer_parity_small_configs(mb, cfg, variant):
    import parity_util as pu
    shape = _shape(cfg, **variant)
    say(f"layer parity cfg{cfg} {variant}")
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    gpu = pu.run_layer(dl, pu.dev_u16(x), x.shape[0])
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    say(f"cfg{cfg}: rel err {err:.2e}, near ties {ties}")


@pytest.mark.parametrize("T", [1, 3, 16, 37, 64, 200])
def test_layer_parity_token_counts(mb, T):
    """Decode-sized and ragged token counts through the config-2 layer
    (several tiles of rows per expert, ragged tails)."""
    import parity_util as pu
    shape = _shape(2, tokens=T, correlated_sigma=0.0, seed=50 + T)
    say(f"layer parity cfg2 shape T={T}")
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    gpu = pu.run_layer(dl, pu.dev_u16(x), T)
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    say(f"T={T}: rel err {err:.2e}, near ties {ties}")


@pytest.mark.parametrize("fmt,ffn,shared_ffn", [(synth.FMT_INT4_B32, 512, 0), (synth.FMT_INT4_B32, 512, 512),
                                                 (synth.FMT_INT8_ROW, 256, 256)])
def test_layer_parity_other_shapes_many_tokens(mb, fmt, ffn, shared_ffn):
    """Batches above the decode size on a layer shape the pipelined prefill
    GEMMs do not take (H = 1024, 64 experts, top-4): int4 runs the generic
    prefill kernels, int8 the vector-unit item kernels."""
    import parity_util as pu
    T = 40
    shape = _shape(0, tokens=T, fmt=fmt, ffn=ffn, shared_ffn=shared_ffn, seed=130 + fmt + shared_ffn)
    say(f"layer parity H=1024 F={ffn} fmt {fmt} shared {shared_ffn} T={T}")
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    gpu = pu.run_layer(dl, pu.dev_u16(x), T)
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    say(f"  rel err {err:.2e}, near ties {ties}")


def test_prefill_repeated_calls_one_workspace(mb):
    """Prefill calls share the workspace's item queues: every call must leave
    them zero for the next one.  Three calls on one workspace, interleaved
    with a call of another size, give the same bits each time and match the
    oracle."""
    import parity_util as pu
    T = 200
    shape = _shape(2, tokens=T, correlated_sigma=0.0, seed=91)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    ws = mb.make_workspace(dl, T)
    say("prefill repeated calls T=200 on one workspace")
    first = pu.run_layer(dl, pu.dev_u16(x), T, ws=ws)
    pu.check_layer_against_oracle(layer, x, first)
    for rep in range(3):
        say(f"  call {rep + 2}")
        pu.run_layer(dl, pu.dev_u16(x[:64]), 64, ws=ws, with_logits=False)  # another size in between
        again = pu.run_layer(dl, pu.dev_u16(x), T, ws=ws, with_logits=False)
        assert np.array_equal(again["ids"], first["ids"])
        assert np.array_equal(again["y"], first["y"]), f"call {rep + 2}: bits differ from the first call"


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_small_batch_one_launch_down_combine(mb, cfg):
    """Decode batches of up to eight tokens without the normalised residual
    copy run the down projection and the combine as one launch; larger
    batches, and calls that ask for the normalised copy, take two.  A
    token's output and residual sum must carry the same bits either way
    (int8 and int4), and match the oracle."""
    import parity_util as pu
    shape = _shape(cfg, tokens=16, correlated_sigma=0.0, seed=70 + cfg, **({"layers": 1} if cfg == 3 else {}))
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    r = synth.make_x(shape, seed=170 + cfg)
    dl = mb.layer_to_device(layer)
    say(f"one-launch down+combine cfg{cfg}: T=16 two-launch reference")
    full = pu.run_layer(dl, pu.dev_u16(x), 16, residual=pu.dev_u16(r), normed=True, with_logits=False)
    for T in (1, 2, 5, 8, 9, 12, 16):
        say(f"  T={T}")
        part = pu.run_layer(dl, pu.dev_u16(x[:T]), T, residual=pu.dev_u16(r[:T]), normed=False)
        assert np.array_equal(part["ids"], full["ids"][:T])
        assert np.array_equal(part["y"], full["y"][:T]), f"T={T}: bits differ from the two-launch path"
        assert np.array_equal(part["residual_out"], full["residual_out"][:T]), f"T={T}: residual sum differs"
        if T in (5, 16):
            err, ties = pu.check_layer_against_oracle(layer, x[:T], part)
            say(f"  T={T}: rel err {err:.2e}, near ties {ties}")


def test_small_batch_residual_without_norm(mb):
    """The one-launch path's residual epilogue: bf16(r + y), no normalised
    copy."""
    import parity_util as pu
    import oracle
    shape = _shape(2, tokens=3, correlated_sigma=0.0, seed=77)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    r = synth.make_x(_shape(2, tokens=3, correlated_sigma=0.0, seed=78))
    dl = mb.layer_to_device(layer)
    say("residual without norm, T=3")
    gpu = pu.run_layer(dl, pu.dev_u16(x), 3, residual=pu.dev_u16(r), normed=False)
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    # the epilogue exactly: one float32 addition of the layer's own y, then
    # round to nearest even
    assert np.array_equal(gpu["residual_out"], pu.residual_expected(r, gpu["y"])), \
        "residual_out is not bf16_rne(float32(r) + y)"
    # and against the oracle's double-precision rounding of the same sum
    r_ref = oracle.residual(r, gpu["y"].astype(np.float32).astype(np.float64))
    assert np.abs(r_ref.astype(np.int32) - gpu["residual_out"].astype(np.int32)).max() <= 1
    say(f"  rel err {err:.2e}, near ties {ties}")


@pytest.mark.timeout(600)
def test_prefill_chunk_full(mb):
    """Config 4 at full size (2048 tokens, the launch configuration the
    benchmark times), every token checked against the oracle (threaded on
    the host cores)."""
    import parity_util as pu
    shape = synth.CONFIGS[4]
    say("prefill cfg4 T=2048, all tokens")
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    gpu = pu.run_layer(dl, pu.dev_u16(x), shape.tokens)
    ids = gpu["ids"]
    assert ids.min() >= 0 and ids.max() < shape.n_experts
    assert all(len(set(r.tolist())) == shape.top_k for r in ids)
    assert np.all(np.abs(gpu["w"].sum(axis=1) - 1.0) <= 1e-6)
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    say(f"cfg4 all tokens: rel err {err:.2e}, near ties {ties}")


@pytest.mark.timeout(900)
def test_stack_teacher_forced(mb):
    """Config 3: 16 tokens through 40 distinct layers.  The residual stream
    r takes r + y (bf16) after every layer and the next layer reads its RMS
    normalisation; each layer is checked against the oracle fed the GPU's
    input, and the epilogue against the oracle's rounding of the GPU's y."""
    import parity_util as pu
    import oracle
    shape = synth.CONFIGS[3]
    x = synth.make_x(shape)  # the first layer's input, also the initial residual
    r = x.copy()
    worst = 0.0
    for l in range(shape.layers):
        say(f"stack cfg3 layer {l}")
        layer = synth.make_layer(shape, layer=l)
        dl = mb.layer_to_device(layer)
        gpu = pu.run_layer(dl, pu.dev_u16(x), shape.tokens, residual=pu.dev_u16(r))
        err, ties = pu.check_layer_against_oracle(layer, x, gpu)
        worst = max(worst, err)
        assert np.array_equal(gpu["residual_out"], pu.residual_expected(r, gpu["y"])), \
            "residual_out is not bf16_rne(float32(r) + y)"
        r_ref = oracle.residual(r, gpu["y"].astype(np.float32).astype(np.float64))
        assert np.abs(r_ref.astype(np.int32) - gpu["residual_out"].astype(np.int32)).max() <= 1
        n_ref = oracle.rmsnorm(gpu["residual_out"])
        d_n = np.abs(n_ref.astype(np.int32) - gpu["normed_out"].astype(np.int32))
        assert d_n.max() <= 1, "normed_out differs from bf16(rmsnorm(r)) by more than one bf16 step"
        say(f"  layer {l}: rel err {err:.2e}, near ties {ties}, max|r| {np.abs(pu.bf16_to_f64(r)).max():.2f}")
        r = gpu["residual_out"]
        x = gpu["normed_out"]
        del dl
    say(f"stack worst rel err {worst:.2e}")


def test_run_to_run_bit_identical(mb):
    import parity_util as pu
    import torch
    shape = synth.CONFIGS[3]
    layer = synth.make_layer(shape, layer=0)
    dl = mb.layer_to_device(layer)
    x = pu.dev_u16(synth.make_x(shape))
    say("determinism cfg3 layer0")
    a = pu.run_layer(dl, x, shape.tokens)
    b = pu.run_layer(dl, x, shape.tokens)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["ids"], b["ids"])
    del torch


def test_decode_batch_invariance(mb):
    """A token's decode output has the same bits alone and inside a batch."""
    import parity_util as pu
    shape = synth.CONFIGS[3]
    layer = synth.make_layer(shape, layer=1)
    dl = mb.layer_to_device(layer)
    x = synth.make_x(shape)
    say("batch invariance cfg3 layer1")
    full = pu.run_layer(dl, pu.dev_u16(x), shape.tokens)
    for t in (0, 5, 15):
        solo = pu.run_layer(dl, pu.dev_u16(x[t:t + 1]), 1)
        assert np.array_equal(solo["y"][0], full["y"][t]), f"token {t} changes with its company"


def test_zero_tokens_is_a_noop(mb):
    import torch
    shape = synth.CONFIGS[0]
    dl = mb.layer_to_device(synth.make_layer(shape))
    ws = mb.make_workspace(dl, 4)
    x = torch.zeros((0, shape.hidden), dtype=torch.int16, device="cuda")
    y = torch.zeros((0, shape.hidden), dtype=torch.float32, device="cuda")
    mb.layer_forward(dl, x, y, ws)
    torch.cuda.synchronize()


def test_workspace_too_small_is_rejected(mb):
    import torch
    shape = synth.CONFIGS[0]
    dl = mb.layer_to_device(synth.make_layer(shape))
    need = mb.workspace_bytes(dl, 4)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    x = torch.zeros((4, shape.hidden), dtype=torch.int16, device="cuda")
    y = torch.empty((4, shape.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(mb.MoeError) as ei:
        mb.layer_forward(dl, x, y, ws)
    assert ei.value.status == mb.MOE_ERR_WORKSPACE
