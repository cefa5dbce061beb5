"""The entry point that allocates nothing (moe_layer_forward_noalloc): its
workspace is the library's per-device scratch array.  Called through the C
ABI, it must give the bits of moe_layer_forward on the same inputs (same
kernels), and match the oracle, on two calls in a row where the second is
smaller (the array keeps the first call's contents); a call that needs more
than the array holds is refused before anything is launched."""
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


def _run(mb, dl, x_host, T, noalloc, residual=None):
    import torch
    import parity_util as pu
    H, K = dl.hidden, dl.top_k
    x = pu.dev_u16(x_host[:T])
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((T, K), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, K), float("nan"), dtype=torch.float32, device="cuda")
    res, held = None, []
    if residual is not None:
        r_in = pu.dev_u16(residual[:T])
        r_out = torch.empty((T, H), dtype=torch.int16, device="cuda")
        n_out = torch.empty((T, H), dtype=torch.int16, device="cuda")
        held = [r_in, r_out, n_out]  # the descriptor keeps only addresses
        res = mb.residual(r_in, r_out, n_out)
    if noalloc:
        mb.layer_forward_noalloc(dl, x, y, res=res, topk_ids=ids, topk_w=w)
    else:
        ws = mb.make_workspace(dl, T)
        mb.layer_forward(dl, x, y, ws, res=res, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    out = {"y": y.cpu().numpy().astype(np.float64), "ids": ids.cpu().numpy(),
           "w": w.cpu().numpy().astype(np.float64)}
    if held:
        out["residual_out"] = pu.host_u16(held[1])
        out["normed_out"] = pu.host_u16(held[2])
    return out


@pytest.mark.parametrize("sizes", [(16, 3), (64, 37)])
def test_noalloc_matches_workspace_entry_point(mb, sizes):
    """Decode-sized (16 then 3 tokens, with the residual epilogue) and
    prefill-sized (64 then 37 tokens) calls of a config-3 layer."""
    import parity_util as pu
    big = max(sizes)
    shape = synth.Shape(**{**synth.CONFIGS[3].__dict__, "tokens": big, "layers": 1, "seed": 500 + big})
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    r = synth.make_x(shape, seed=600 + big)
    dl = mb.layer_to_device(layer)
    with_res = big <= 16
    for T in sizes:  # the second call is the smaller one
        say(f"noalloc vs workspace entry point, T={T}")
        a = _run(mb, dl, x, T, noalloc=True, residual=r if with_res else None)
        b = _run(mb, dl, x, T, noalloc=False, residual=r if with_res else None)
        for key in a:
            assert np.array_equal(a[key], b[key]), f"T={T}: {key} differs between the two entry points"
        err, ties = pu.check_layer_against_oracle(layer, np.ascontiguousarray(x[:T]), a)
        say(f"  T={T}: identical bits; rel err vs oracle {err:.2e}, near ties {ties}")


def test_noalloc_refuses_calls_beyond_the_array(mb):
    """A 2048-token prefill chunk needs more workspace than the array holds:
    MOE_ERR_UNSUPPORTED, and the output buffer is left untouched."""
    import torch
    shape = synth.CONFIGS[4]
    dl = mb.layer_to_device(synth.make_layer(shape))
    T = shape.tokens
    assert mb.workspace_bytes(dl, T) > 16 << 20
    x = torch.zeros((T, shape.hidden), dtype=torch.int16, device="cuda")
    y = torch.full((T, shape.hidden), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(mb.MoeError) as ei:
        mb.layer_forward_noalloc(dl, x, y)
    assert ei.value.status == mb.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
