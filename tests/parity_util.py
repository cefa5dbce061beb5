"""Shared helpers of the GPU parity tests: upload synthetic inputs, run the
HIP path through the C ABI, and compare with the CPU oracle under the
acceptance rules (selection exact except near ties, weights within 1e-6,
outputs within 2e-3 of the largest reference magnitude)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from mixture_experts_decode_moe_amd import synth

TIE_EPS = 1e-4  # |l_(K) - l_(K+1)| below this: either selection is correct
W_TOL = 1e-6  # routing weights, absolute
Y_REL = 2e-3  # max|y_gpu - y_ref| <= Y_REL * max|y_ref| over a layer call


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def near_tie_tokens(logits: np.ndarray, K: int) -> np.ndarray:
    """Tokens whose K-th and (K+1)-th oracle logits are within TIE_EPS."""
    s = -np.sort(-logits, axis=1)
    if logits.shape[1] <= K:
        return np.zeros(logits.shape[0], bool)
    return (s[:, K - 1] - s[:, K]) < TIE_EPS


def check_selection(ids_gpu, ids_ref, logits_ref, K):
    """Selected sets equal for every token not at a near tie, and the order
    equal wherever adjacent selected logits differ by at least TIE_EPS."""
    tie = near_tie_tokens(logits_ref, K)
    for t in range(ids_ref.shape[0]):
        if tie[t]:
            g = ids_gpu[t]
            assert len(set(g.tolist())) == K and g.min() >= 0 and g.max() < logits_ref.shape[1]
            continue
        assert set(ids_gpu[t].tolist()) == set(ids_ref[t].tolist()), f"token {t}: {ids_gpu[t]} vs {ids_ref[t]}"
        lv = logits_ref[t, ids_ref[t]]
        for k in range(K):
            if ids_gpu[t, k] != ids_ref[t, k]:
                lo, hi = max(k - 1, 0), min(k + 1, K - 1)
                gaps = [abs(lv[k] - lv[i]) for i in (lo, hi) if i != k]
                assert min(gaps) < TIE_EPS, f"token {t} slot {k}: order differs away from a tie"
    return tie


def rel_max_err(y, ref):
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-30))


def run_layer(dlayer, x_dev, T, ws=None, residual=None, with_logits=True, normed=True, opts=None):
    """Runs moe_layer_forward (moe_layer_forward_ex with `opts`); also runs
    moe_route on the same input (same kernels) to read the GPU's fp32
    logits, unless with_logits is False."""
    from mixture_experts_decode_moe_amd import binding as mb
    H, K, E = dlayer.hidden, dlayer.top_k, dlayer.n_experts
    if ws is None:
        ws = mb.make_workspace(dlayer, T)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    res = None
    if residual is not None:
        # residual: the bf16 residual stream entering the layer (device)
        r_out = torch.empty((T, H), dtype=torch.int16, device="cuda")
        n_out = torch.empty((T, H), dtype=torch.int16, device="cuda") if normed else None
        res = mb.residual(residual, r_out, n_out)
    mb.layer_forward(dlayer, x_dev, y, ws, res=res, topk_ids=ids, topk_w=w, opts=opts)
    out = {}
    if with_logits:
        lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
        ids2 = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w2 = torch.empty((T, K), dtype=torch.float32, device="cuda")
        mb.route(dlayer, x_dev, ids2, w2, lg)
    torch.cuda.synchronize()
    out.update(y=y.cpu().numpy().astype(np.float64), ids=ids.cpu().numpy(), w=w.cpu().numpy().astype(np.float64))
    if with_logits:
        out["logits"] = lg.cpu().numpy().astype(np.float64)
        # the layer's routing is the router kernels' routing, bit for bit
        assert np.array_equal(ids2.cpu().numpy(), out["ids"])
        assert np.array_equal(w2.cpu().numpy().astype(np.float64), out["w"])
    if residual is not None:
        out["residual_out"] = host_u16(r_out)
        if normed:
            out["normed_out"] = host_u16(n_out)
    return out


def bf16_rne_f32(v: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def residual_expected(r_bf16: np.ndarray, y_f32: np.ndarray) -> np.ndarray:
    """The residual epilogue's exact result: bf16_rne(float32(r) + y) with
    one float32 addition."""
    rf = (np.asarray(r_bf16, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return bf16_rne_f32(rf + np.asarray(y_f32, np.float32))


def logit_error_bound(layer_host, x_host):
    """Rigorous bound of float32 dot-product + bias rounding:
    (H + 2) * 2^-24 * (sum_h |Wr[e][h] x[h]| + |b_e|)."""
    xf = bf16_to_f64(x_host)
    s = np.abs(xf) @ np.abs(layer_host.router_w.astype(np.float64)).T
    if layer_host.router_bias is not None:
        s = s + np.abs(layer_host.router_bias.astype(np.float64))[None, :]
    return (layer_host.hidden + 2) * 2.0 ** -24 * s


def check_routing_self_consistent(ids_g, w_g, logits_g, K, renorm=1):
    """The GPU's selection is exactly the top-K of its own float32 logits
    (descending, lower index on ties) and its weights are their softmax
    within float32 rounding."""
    T, E = logits_g.shape
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits_g[t]))[:K]
        assert np.array_equal(ids_g[t], order), f"token {t}: GPU selection is not the top-K of its own logits"
        l = logits_g[t, ids_g[t]]
        if renorm:
            p = np.exp(l - l[0])
            ref = p / p.sum()
        else:
            pe = np.exp(logits_g[t] - logits_g[t].max())
            ref = pe[ids_g[t]] / pe.sum()
        assert np.max(np.abs(w_g[t] - ref)) <= W_TOL, f"token {t}: weights are not the softmax of the logits"


def check_layer_against_oracle(layer_host, x_host, gpu, sample=None, nthreads=0):
    """Compare one layer call.  `sample`: token indices to check (all if
    None).  Near-tie tokens are re-evaluated by the oracle with the GPU's
    selection.  Without the GPU's logits in `gpu`, the routing weights are
    held to W_TOL plus twice the rigorous float32 bound of any logit's
    error (logit_error_bound): what a softmax of logits summed in any order
    can differ by.  Returns (relative error, number of near-tie tokens)."""
    K = layer_host.top_k
    idx = np.arange(x_host.shape[0]) if sample is None else np.asarray(sample)
    xs = np.ascontiguousarray(x_host[idx])
    y_ref, ids_ref, w_ref, logits_ref = oracle.layer_forward(layer_host, xs, nthreads=nthreads)
    ids_g, w_g, y_g = gpu["ids"][idx], gpu["w"][idx], gpu["y"][idx]
    tie = check_selection(ids_g, ids_ref, logits_ref, K)
    if tie.any():
        y_tie, _, w_tie, _ = oracle.layer_forward(layer_host, xs, ids=ids_g, nthreads=nthreads)
        y_ref = np.where(tie[:, None], y_tie, y_ref)
        w_ref = np.where(tie[:, None], w_tie, w_ref)
    ids_cmp = np.where(tie[:, None], ids_g, ids_ref)
    if "logits" in gpu:
        lg = gpu["logits"][idx]
        bound = logit_error_bound(layer_host, xs)
        assert np.all(np.abs(lg - logits_ref) <= bound), "GPU logits outside the float32 error bound"
        check_routing_self_consistent(ids_g, w_g, lg, K, layer_host.renorm)
        # w_k = softmax(l)_k: |dw_k| <= 2 max_j |dl_j|; plus float32 rounding
        dl = np.max(np.abs(lg - logits_ref), axis=1)
        w_tol = W_TOL + 2.0 * dl
    else:
        w_tol = W_TOL + 2.0 * np.max(logit_error_bound(layer_host, xs), axis=1)
    for t in range(len(idx)):
        by_expert = {int(e): wv for e, wv in zip(ids_cmp[t], w_ref[t])}
        for k in range(K):
            d = abs(w_g[t, k] - by_expert[int(ids_g[t, k])])
            assert d <= w_tol[t], f"token {idx[t]} slot {k}: |dw| = {d:.3e} > {w_tol[t]:.3e}"
    err = rel_max_err(y_g, y_ref)
    assert err <= Y_REL, f"max|y_gpu - y_ref| / max|y_ref| = {err:.3e}"
    return err, int(tie.sum())
