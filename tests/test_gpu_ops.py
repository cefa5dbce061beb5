"""GPU parity of the separate ABI steps: moe_route, moe_permute,
moe_expert_ffn and moe_combine, each against the oracle (integers bit-exact,
floating point within the layer's tolerances)."""
import sys

import numpy as np
import pytest

import oracle
from mixture_experts_decode_moe_amd import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mb():
    from mixture_experts_decode_moe_amd import binding
    return binding


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_route(mb, cfg):
    """moe_route alone.  It reads only the router, so the expert pointers of
    the layer descriptor are small placeholders."""
    import torch
    import parity_util as pu
    shape = synth.CONFIGS[cfg]
    say(f"route cfg{cfg}")
    seed = synth.layer_seed(shape, 0)
    E, H, K = shape.n_experts, shape.hidden, shape.top_k
    wr = synth.normal_f32(seed, synth.S_ROUTER_W, E * H, 0.0, 0.02).reshape(E, H)
    bias = synth.make_router_bias(shape, seed)
    x = synth.make_x(shape)
    T = x.shape[0]
    dummy = torch.zeros(64, dtype=torch.uint8, device="cuda")
    routed = mb.Experts(shape.fmt, E, shape.ffn, dummy, dummy, dummy, dummy, dummy, dummy)
    dl = mb.Layer(H, E, K, shape.renorm, torch.from_numpy(wr).cuda(),
                  None if bias is None else torch.from_numpy(bias).cuda(), routed, None)
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    mb.route(dl, pu.dev_u16(x), ids, w, lg)
    torch.cuda.synchronize()
    host = synth.LayerHost(H, E, K, shape.renorm, wr, bias, None)
    ref = oracle.router_logits(host, x)
    lg_h = lg.cpu().numpy().astype(np.float64)
    # float32 accumulation over H terms: |err| <= H * 2^-24 * sum|w x| (+ bias rounding)
    xf = pu.bf16_to_f64(x)
    bound = H * 2.0 ** -24 * (xf.__abs__() @ np.abs(wr.astype(np.float64)).T) + 1e-6
    assert np.all(np.abs(lg_h - ref) <= bound)
    ids_ref, w_ref = oracle.select(ref, K, shape.renorm)
    ids_h, w_h = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    tie = pu.check_selection(ids_h, ids_ref, ref, K)
    ok = ~tie
    same = np.all(ids_h == ids_ref, axis=1) & ok
    # the weights are the softmax of the GPU's own logits, and differ from
    # the oracle's by at most what the logits' float32 error allows
    pu.check_routing_self_consistent(ids_h, w_h, lg_h, K, shape.renorm)
    w_tol = pu.W_TOL + 2.0 * np.max(np.abs(lg_h - ref), axis=1)
    assert np.all(np.abs(w_h[same] - w_ref[same]) <= w_tol[same][:, None])
    assert np.all(np.abs(w_h.sum(axis=1) - 1.0) <= 1e-6)
    say(f"route cfg{cfg}: near ties {int(tie.sum())} of {T}")


@pytest.mark.parametrize("T", [1, 4, 16, 40])
def test_route_exact_ties(mb, T):
    """Equal logits: every router row appears eight times (experts e, e + 32,
    ..., e + 224 share one row, so equal logits sit both in one lane and in
    different lanes of the top-k wave).  The selection must be the lowest
    indices among equal logits, round by round: exactly the oracle's
    selection run on the GPU's own logits (T <= 16: the decode routing; T >
    16: the top-k kernel), and each token's experts are the eight copies of
    one row, ascending, with equal weights."""
    import torch
    import parity_util as pu
    E, H, K = 256, 1024, 8
    base = synth.normal_f32(7, synth.S_ROUTER_W, 32 * H, 0.0, 0.02).reshape(32, H)
    wr = np.ascontiguousarray(base[np.arange(E) % 32])
    x = synth.normal_bf16(8, synth.S_X, T * H).reshape(T, H)
    say(f"route exact ties T={T}")
    dummy = torch.zeros(64, dtype=torch.uint8, device="cuda")
    routed = mb.Experts(synth.FMT_INT4_B32, E, 512, dummy, dummy, dummy, dummy, dummy, dummy)
    dl = mb.Layer(H, E, K, 1, torch.from_numpy(wr).cuda(), None, routed, None)
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    mb.route(dl, pu.dev_u16(x), ids, w, lg)
    torch.cuda.synchronize()
    ids_h, w_h, lg_h = ids.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy().astype(np.float64)
    # duplicate rows give bit-equal logits
    assert np.array_equal(lg_h, lg_h[:, np.arange(E) % 32])
    exp_ids, _ = oracle.select(lg_h, K, 1)
    assert np.array_equal(ids_h, exp_ids)
    best = np.argmax(lg_h[:, :32], axis=1)
    assert np.array_equal(ids_h, best[:, None] + 32 * np.arange(K)[None, :])
    assert np.allclose(w_h, 1.0 / K, rtol=0, atol=1e-7)


@pytest.mark.parametrize("T,K,E,mode", [(1, 8, 256, "rand"), (16, 8, 256, "rand"), (2048, 8, 256, "rand"),
                                        (700, 4, 64, "rand"), (300, 8, 256, "one"), (5, 2, 1024, "rand"),
                                        (3000, 1, 16, "skew")])
def test_permute_exact(mb, T, K, E, mode):
    import torch
    say(f"permute T={T} K={K} E={E} {mode}")
    rng = np.random.default_rng(T * 7 + K)
    if mode == "one":
        ids = np.stack([np.r_[[3], rng.choice(np.setdiff1d(np.arange(E), [3]), K - 1, replace=False)]
                        for _ in range(T)]).astype(np.int32)
    elif mode == "skew":
        ids = rng.choice(4, size=(T, K)).astype(np.int32)
    else:
        ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(size=(T, K)).astype(np.float32)
    ref = oracle.permute(ids, w, E)
    TK = T * K
    out = dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
               offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
               row_tok=torch.empty(TK, dtype=torch.int32, device="cuda"),
               row_w=torch.empty(TK, dtype=torch.float32, device="cuda"),
               inv_pos=torch.empty((T, K), dtype=torch.int32, device="cuda"),
               active=torch.full((E,), -1, dtype=torch.int32, device="cuda"),
               n_active=torch.empty(1, dtype=torch.int32, device="cuda"))
    ws = torch.empty(mb.permute_workspace_bytes(T, K, E), dtype=torch.uint8, device="cuda")
    mb.permute(torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), E, out, ws)
    torch.cuda.synchronize()
    for k in ("counts", "offsets", "row_tok", "row_w", "inv_pos"):
        assert np.array_equal(out[k].cpu().numpy(), ref[k]), k
    na = int(out["n_active"].cpu().numpy()[0])
    assert na == ref["n_active"]
    assert np.array_equal(out["active"].cpu().numpy()[:na], ref["active"])


@pytest.mark.parametrize("cfg,tokens", [(0, None), (2, None), (4, 48)])
def test_expert_ffn_and_combine(mb, cfg, tokens):
    """moe_expert_ffn on the oracle's permutation, then moe_combine, each
    compared with the oracle's rows and layer output.  The 48-token case of
    the prefill layer runs the grouped GEMMs on x as given (bf16; the layer
    call hands them x already in fp16)."""
    import torch
    import parity_util as pu
    shape = synth.CONFIGS[cfg]
    say(f"expert_ffn+combine cfg{cfg} tokens {tokens}")
    layer = synth.make_layer(shape)
    x = synth.make_x(shape, tokens=tokens)
    T, K, E, H = x.shape[0], shape.top_k, shape.n_experts, shape.hidden
    y_ref, ids, w, _ = oracle.layer_forward(layer, x)
    p = oracle.permute(ids, w.astype(np.float32), E)
    rows_ref = oracle.expert_rows(layer.routed, x, p["offsets"], p["row_tok"], p["row_w"])
    dl = mb.layer_to_device(layer)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    TK = T * K
    rows = torch.empty((TK, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(mb.expert_ffn_workspace_bytes(TK, shape.ffn), dtype=torch.uint8, device="cuda")
    xd = pu.dev_u16(x)
    mb.expert_ffn(dl.routed, H, xd, TK, cu(p["offsets"]), cu(p["active"]), cu(np.array([p["n_active"]], np.int32)),
                  cu(p["row_tok"]), cu(p["row_w"]), rows, ws)
    shared = None
    if dl.shared is not None:
        shared = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ws2 = torch.empty(mb.expert_ffn_workspace_bytes(T, shape.shared_ffn), dtype=torch.uint8, device="cuda")
        mb.expert_ffn(dl.shared, H, xd, T, None, None, None, None, None, shared, ws2)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    r_out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    normed = torch.empty((T, H), dtype=torch.int16, device="cuda")
    mb.combine(rows, cu(p["inv_pos"]), T, K, H, shared, y, mb.residual(xd, r_out, normed))
    torch.cuda.synchronize()
    rows_h = rows.cpu().numpy().astype(np.float64)
    assert pu.rel_max_err(rows_h, rows_ref) <= pu.Y_REL
    assert pu.rel_max_err(y.cpu().numpy().astype(np.float64), y_ref) <= pu.Y_REL
    r_ref = oracle.residual(x, y.cpu().numpy().astype(np.float64))
    assert np.abs(r_ref.astype(np.int32) - pu.host_u16(r_out).astype(np.int32)).max() <= 1
    n_ref = oracle.rmsnorm(pu.host_u16(r_out))
    assert np.abs(n_ref.astype(np.int32) - pu.host_u16(normed).astype(np.int32)).max() <= 1


def test_calibration_helpers(mb):
    """The ceilings the roofline figures are compared with: the matrix-core
    issue kernel and the read-stream kernel run, and their rates sit below
    the data-sheet peaks (2516.6 TFLOP/s fp16, 5033 TOP/s int8, 8000 GB/s)
    and above a tenth of them."""
    import torch
    for kind, peak in ((0, 2516.6), (1, 2516.6), (2, 5033.2)):
        ms, ops = mb.calib_mfma(kind, 2000)
        rate = ops / (ms * 1e-3) / 1e12
        say(f"matrix cores kind {kind}: {rate:.0f} of {peak}")
        assert 0.1 * peak < rate <= 1.02 * peak
    # 1 GiB filled, then its first 512 MiB read (the 256 MB last-level
    # cache holds at most the end of the fill)
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    torch.cuda.synchronize()
    ms = mb.calib_read(buf, 512 << 20)
    gbs = (512 << 20) / (ms * 1e-3) / 1e9
    say(f"read 512 MiB: {gbs:.0f} GB/s")
    assert 800 < gbs <= 8000 * 1.02
