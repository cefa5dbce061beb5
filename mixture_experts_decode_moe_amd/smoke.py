"""One small layer call on cuda:0, checked against the CPU oracle (the tiny
int8 configuration: 4 tokens, 64 experts, top-4)."""
from __future__ import annotations

import numpy as np


def run() -> None:
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("smoke needs a GPU")
    import oracle
    from mixture_experts_decode_moe_amd import binding as mb
    from mixture_experts_decode_moe_amd import synth

    shape = synth.CONFIGS[0]
    layer = synth.make_layer(shape)
    x = synth.make_x(shape)
    T, H, K = x.shape[0], shape.hidden, shape.top_k
    with torch.cuda.device(0):
        dl = mb.layer_to_device(layer, "cuda:0")
        xd = torch.from_numpy(x.view(np.int16)).to("cuda:0")
        ws = mb.make_workspace(dl, T, "cuda:0")
        y = torch.empty((T, H), dtype=torch.float32, device="cuda:0")
        ids = torch.empty((T, K), dtype=torch.int32, device="cuda:0")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda:0")
        mb.layer_forward(dl, xd, y, ws, topk_ids=ids, topk_w=w)
        torch.cuda.synchronize()
    y_ref, ids_ref, w_ref, logits = oracle.layer_forward(layer, x)
    ids_g = ids.cpu().numpy()
    if not np.array_equal(ids_g, ids_ref):
        raise AssertionError(f"selection differs: {ids_g} vs {ids_ref}")
    if np.max(np.abs(w.cpu().numpy() - w_ref)) > 1e-6:
        raise AssertionError("routing weights differ by more than 1e-6")
    err = np.max(np.abs(y.cpu().numpy() - y_ref)) / np.max(np.abs(y_ref))
    if err > 2e-3:
        raise AssertionError(f"layer output error {err:.3e} > 2e-3 of max|ref|")
    print(f"smoke ok: T={T} H={H} E={shape.n_experts} K={K} rel err {err:.2e}")


if __name__ == "__main__":
    run()
