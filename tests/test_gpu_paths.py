"""GPU tests of the kernel families and of the inputs the other parity tests
do not reach: forced decode / prefill paths and their agreement, the
environment override, an expert with more rows than one matrix tile on the
decode kernels, more than 16 slots per token, more than 256 experts on a
decode call, int8 batches above the decode size at the real shape, a
prefill call whose hot experts span several 128-row items, and the prefill
family's documented fp16 range.  Every expected value comes from the CPU
oracle or from the other kernel family on the same inputs."""
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


@pytest.mark.parametrize("T", [1, 16, 64])
def test_decode_and_prefill_paths_agree(mb, T):
    """The same layer call through the decode kernels and through the
    prefill grouped GEMMs (forced per call): both match the oracle, and they
    agree with each other within the output tolerance (the pages' practice
    of running one kernel family beside the other on the same
    activations)."""
    import parity_util as pu
    import oracle
    shape = _shape(2, tokens=T, correlated_sigma=0.0, seed=300 + T)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    out = {}
    for path in ("decode", "prefill"):
        say(f"forced {path} path, T={T}")
        out[path] = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False, opts=mb.forward_opts(path))
        err, ties = pu.check_layer_against_oracle(layer, x, out[path])
        say(f"  {path}: rel err {err:.2e}, near ties {ties}")
    # tokens away from a near tie select the same experts on both paths and
    # get the same outputs within the tolerance
    _, _, _, logits_ref = oracle.layer_forward(layer, x)
    keep = ~pu.near_tie_tokens(logits_ref, shape.top_k)
    assert np.array_equal(out["decode"]["ids"][keep], out["prefill"]["ids"][keep])
    d = pu.rel_max_err(out["prefill"]["y"][keep], out["decode"]["y"][keep])
    say(f"  decode vs prefill: {d:.2e} of max|y|")
    assert d <= pu.Y_REL


def test_force_path_environment_override(mb, monkeypatch):
    """MOE_FORCE_PATH, read at every call, forces the family of calls that
    leave the choice to the token count: a 16-token call gives the prefill
    family's bits with it set to prefill, and the default bits again once it
    is removed."""
    import parity_util as pu
    T = 16
    shape = _shape(2, tokens=T, correlated_sigma=0.0, seed=333)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    say("MOE_FORCE_PATH override, T=16")
    auto = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False)
    forced = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False, opts=mb.forward_opts("prefill"))
    monkeypatch.setenv("MOE_FORCE_PATH", "prefill")
    env = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False)
    monkeypatch.delenv("MOE_FORCE_PATH")
    back = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False)
    assert np.array_equal(env["y"], forced["y"])
    assert np.array_equal(back["y"], auto["y"])
    assert not np.array_equal(auto["y"], forced["y"])  # two families, two roundings
    pu.check_layer_against_oracle(layer, x, env)


def test_expert_ffn_unit_larger_than_a_tile(mb):
    """moe_expert_ffn with one expert owning 32 rows of a 4-token batch (rows
    repeat tokens): more rows than the decode gate/up kernel's 16-row tile,
    so the call must take kernels that handle any row count."""
    import torch
    import oracle
    shape = _shape(2, tokens=4, correlated_sigma=0.0, seed=350)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    n_rows = 32
    row_tok = (np.arange(n_rows) * 7 % 4).astype(np.int32)
    row_w = np.linspace(0.25, 1.0, n_rows).astype(np.float32)
    ex = synth.make_experts(shape.fmt, 350, 1, shape.hidden, shape.ffn)
    dex = mb.experts_to_device(ex)
    say("moe_expert_ffn: one expert, 32 rows, T=4")
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    rows_out = torch.empty((n_rows, shape.hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(mb.expert_ffn_workspace_bytes(n_rows, shape.ffn), dtype=torch.uint8, device="cuda")
    mb.expert_ffn(dex, shape.hidden, xd, n_rows, None, None, None, torch.from_numpy(row_tok).cuda(),
                  torch.from_numpy(row_w).cuda(), rows_out, ws)
    torch.cuda.synchronize()
    got = rows_out.cpu().numpy().astype(np.float64)
    offsets = np.array([0, n_rows], np.int32)
    ref = oracle.expert_rows(ex, x, offsets, row_tok, row_w)
    err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    say(f"  rel err {err:.2e}")
    assert err <= 2e-3
    del layer


def test_more_than_16_slots_per_token(mb):
    """top-20 of 64 experts on a 4-token decode call: the one-launch down +
    combine takes at most 16 slots, so this call runs the two-launch path
    and the combine kernel's loop over slots beyond its unrolled batch."""
    import parity_util as pu
    shape = _shape(0, top_k=20, seed=360)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    say("top-20 of 64, T=4")
    gpu = pu.run_layer(dl, pu.dev_u16(x), 4)
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    say(f"  rel err {err:.2e}, near ties {ties}")


def test_combine_entry_point_many_slots(mb):
    """moe_combine with K = 24 > 16 slots, some skipped (inv_pos < 0), a
    shared row and the residual epilogue, against numpy."""
    import torch
    import parity_util as pu
    rng = np.random.default_rng(5)
    T, K, H = 3, 24, 512
    rows = rng.standard_normal((T * K + 5, H)).astype(np.float32)
    inv = rng.permutation(T * K + 5)[:T * K].astype(np.int32).reshape(T, K)
    inv[1, 3] = -1
    inv[2, 20] = -1
    shared = rng.standard_normal((T, H)).astype(np.float32)
    r = synth.normal_bf16(9, 1, T * H).reshape(T, H)
    say("moe_combine K=24")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    r_out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    r_dev = pu.dev_u16(r)  # held: the descriptor keeps only its address
    res = mb.residual(r_dev, r_out)
    mb.combine(torch.from_numpy(rows).cuda(), torch.from_numpy(inv).cuda(), T, K, H,
               torch.from_numpy(shared).cuda(), y, res)
    torch.cuda.synchronize()
    ref = np.zeros((T, H), np.float32)
    for t in range(T):
        for k in range(K):  # slot order, float32, as the definition adds them
            if inv[t, k] >= 0:
                ref[t] += rows[inv[t, k]]
        ref[t] += shared[t]
    got = y.cpu().numpy()
    assert np.array_equal(got, ref), "combine is not the float32 sum in slot order"
    assert np.array_equal(pu.host_u16(r_out), pu.residual_expected(r, got))


def test_decode_with_more_than_256_experts(mb):
    """512 experts, top-8, 4 tokens: the decode call routes in a block of its
    own before the expert kernels (the in-kernel routing covers 256)."""
    import parity_util as pu
    shape = _shape(0, n_experts=512, top_k=8, seed=370)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    say("E=512 decode, T=4")
    gpu = pu.run_layer(dl, pu.dev_u16(x), 4)
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    say(f"  rel err {err:.2e}, near ties {ties}")


def test_int8_batch_above_decode_size_real_shape(mb):
    """int8 weights at the real shape (H=2048, 256 experts, top-8, F=512 +
    shared) with 40 tokens: above the decode size, on the kernels int8 calls
    of that size take."""
    import parity_util as pu
    T = 40
    shape = _shape(1, tokens=T, seed=380, jitter_scales=True)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    say("int8 real shape, T=40")
    gpu = pu.run_layer(dl, pu.dev_u16(x), T)
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    say(f"  rel err {err:.2e}, near ties {ties}")


@pytest.mark.timeout(300)
def test_prefill_skewed_routing_multi_item_experts(mb):
    """512 tokens through a config-3 layer (Zipf(1.1) router bias): the most
    popular experts get several hundred rows, so a routed expert spans
    several 128-row gate/up items and several 64-row down items; all tokens
    checked against the oracle."""
    import parity_util as pu
    T = 512
    shape = _shape(3, tokens=T, layers=1, seed=390)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    dl = mb.layer_to_device(layer)
    say("skewed prefill T=512")
    gpu = pu.run_layer(dl, pu.dev_u16(x), T)
    counts = np.bincount(gpu["ids"].ravel(), minlength=shape.n_experts)
    say(f"  rows of the three most popular experts: {sorted(counts)[-3:]}")
    assert counts.max() > 256, "the bias should give some expert more than two 128-row items"
    err, ties = pu.check_layer_against_oracle(layer, x, gpu)
    say(f"  rel err {err:.2e}, near ties {ties}")


def test_prefill_fp16_range_is_documented_behaviour(mb):
    """The prefill family multiplies in fp16: a token with |x| above 65504
    gets non-finite outputs there, while the other tokens of the call are
    unaffected and the decode family computes the same call finitely (the
    range stated in moe.h)."""
    import parity_util as pu
    T = 20
    shape = _shape(2, tokens=T, correlated_sigma=0.0, seed=400)
    layer = synth.make_layer(shape)
    x = synth.make_x(shape).copy()
    big = 3
    x[big, 17] = 0x47C3  # bf16 99840: outside fp16's range
    dl = mb.layer_to_device(layer)
    say("fp16 range: prefill vs decode with |x| = 99840 in token 3")
    pf = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False, opts=mb.forward_opts("prefill"))
    dec = pu.run_layer(dl, pu.dev_u16(x), T, with_logits=False, opts=mb.forward_opts("decode"))
    assert not np.all(np.isfinite(pf["y"][big])), "the out-of-range token should not stay finite in fp16"
    others = np.array([t for t in range(T) if t != big])
    assert np.all(np.isfinite(pf["y"][others]))
    assert np.all(np.isfinite(dec["y"]))
    pu.check_layer_against_oracle(layer, x, dec)
    # the in-range tokens of the prefill call still match the oracle
    sub = {k: v[others] for k, v in pf.items()}
    pu.check_layer_against_oracle(layer, np.ascontiguousarray(x[others]), sub)


def test_route_without_logits(mb):
    """moe_route with no logits buffer (they pass through the caller's
    workspace) gives the same ids and weights as with one."""
    import torch
    import parity_util as pu
    shape = _shape(2, tokens=40, correlated_sigma=0.0, seed=410)
    layer = synth.make_layer(shape)
    x = pu.dev_u16(synth.make_x(shape))
    dl = mb.layer_to_device(layer)
    T, K, E = 40, shape.top_k, shape.n_experts
    say("moe_route without logits, T=40")
    ids_a = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w_a = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ids_b, w_b = torch.empty_like(ids_a), torch.empty_like(w_a)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    mb.route(dl, x, ids_a, w_a, lg)
    ws = torch.empty(mb.route_workspace_bytes(dl, T), dtype=torch.uint8, device="cuda")
    mb.route(dl, x, ids_b, w_b, None, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b) and torch.equal(w_a, w_b)
