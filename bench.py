#!/usr/bin/env python3
"""Benchmark of the MoE layer on one MI355X.

A step is one pass of the whole layer (router, top-k, permutation, routed
experts, shared expert, combine) over one batch of synthetic input already
resident in HBM.  Default workload: the real-shape decode layer (1 token,
H=2048, 256 experts, top-8, F=512 + shared expert, int8 per-row weights),
run over a ring of 40 distinct layer instances so that no call finds its
weights in the 256 MB last-level cache.  Other workloads: --workload
mtp-verify-int4 | batch16-stack-int4 | prefill-int4 | tiny-int8.

The timed region is K steps launched on one stream behind a bounded spin
kernel long enough for the host to enqueue them all first, so the GPU runs
them back to back; it is bracketed by synchronisation and HIP events.
Inside it the library's profiling hook records HIP events around the
gate/up and down kernels of every layer call of the last steps, on the
stream the kernels run on; the slower of the two is the dominant kernel and
its mean duration gives the roofline figure.  (Event nodes inside captured
HIP graphs did not bracket the kernels on this stack, so no graph is used.)
The CPU oracle is timed on a bounded sample of the same workload on the host
cores.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA

WORKLOADS = {
    "decode-int8": 1,
    "mtp-verify-int4": 2,
    "batch16-stack-int4": 3,
    "prefill-int4": 4,
    "tiny-int8": 0,
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(workload, kernel):
    """HBM bytes per launch of a kernel from the committed counter runs
    (profiles/hbm_traffic.json: FETCH_SIZE and WRITE_SIZE scaled by a plain
    copy of known size), or None when there is no such run or a source file
    the kernel is built from has changed since it was taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
            rec = json.load(f)["kernels"][kernel]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sha256"]:
            return None
        return rec["bytes_per_launch"].get(workload)
    except (OSError, ValueError, KeyError):
        return None


def expert_bytes(fmt, H, F):
    """Bytes of one expert's gate+up and down weights and scales."""
    if fmt == 1:
        gu = 2 * F * H + 2 * F * 4
        dn = H * F + H * 4
    else:
        gu = 2 * F * H // 2 + 2 * F * (H // 32) * 2
        dn = H * F // 2 + H * (F // 32) * 2
    return gu, dn


_HIP = None


def hip_elapsed_ms(start, stop) -> float:
    """hipEventElapsedTime on two torch events recorded by the library (torch
    does not know they were recorded, so its own elapsed_time refuses)."""
    global _HIP
    import ctypes
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _HIP.hipEventElapsedTime.restype = ctypes.c_int
    ms = ctypes.c_float(0.0)
    rc = _HIP.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(start.cuda_event),
                                  ctypes.c_void_p(stop.cuda_event))
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
    return float(ms.value)


def build_ring(shape, n_inst, synth, mb, torch):
    """n_inst distinct layer instances (weights and inputs) in HBM."""
    import dataclasses
    ring = []
    host0 = None
    for i in range(n_inst):
        shp = dataclasses.replace(shape, seed=shape.seed if i == 0 else 100_000 + 97 * i)
        layer = synth.make_layer(shp)
        x = synth.make_x(shp)
        dl = mb.layer_to_device(layer)
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        ring.append((dl, xd))
        if i == 0:
            host0 = (layer, x, shp)
        del layer
    return ring, host0


def build_stack(shape, synth, mb, torch):
    ring = []
    host0 = None
    for l in range(shape.layers):
        layer = synth.make_layer(shape, layer=l)
        ring.append(mb.layer_to_device(layer))
        if l == 0:
            host0 = layer
        del layer
        if (l + 1) % 10 == 0:
            log(f"  stack: {l + 1}/{shape.layers} layers resident")
    x = synth.make_x(shape)
    return ring, host0, x


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode-int8")
    ap.add_argument("--ring", type=int, default=40, help="distinct layer instances (decode workloads)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (20 times), the known-size reference for "
                         "the HBM byte counters, and exit")
    args = ap.parse_args()

    if args.calibrate_copy_mib:
        import torch
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 20}), flush=True)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs on one GPU (expert-parallel sharding is a "
              "design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_decode_moe_amd import binding as mb
    from mixture_experts_decode_moe_amd import synth

    torch.cuda.set_device(0)
    cfg = WORKLOADS[args.workload]
    shape = synth.CONFIGS[cfg]
    H, E, K, F, T = shape.hidden, shape.n_experts, shape.top_k, shape.ffn, shape.tokens
    log(f"workload {args.workload}: {synth.CONFIG_NAMES[cfg]}")

    t0 = time.time()
    stack = cfg == 3
    if stack:
        layers, host_layer0, x_host = build_stack(shape, synth, mb, torch)
        x0 = torch.from_numpy(x_host.view(np.int16)).cuda()
        n_calls_per_step = shape.layers
        ring = None
    else:
        n_inst = 2 if cfg == 4 else (1 if cfg == 0 else args.ring)
        ring, (host_layer0, x_host, shp0) = build_ring(shape, n_inst, synth, mb, torch)
        n_calls_per_step = 1
    torch.cuda.synchronize()
    log(f"inputs resident in {time.time() - t0:.1f} s")

    dev_layers = layers if stack else [r[0] for r in ring]
    c_layers = [dl.c() for dl in dev_layers]
    ws = mb.make_workspace(dev_layers[0], T)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids_buf = torch.empty((T, K), dtype=torch.int32, device="cuda")
    if stack:
        # residual stream r and the next layer's RMS-normalised input xin,
        # both updated in place by the layers' combine epilogue; layer 0
        # reads the step's initial input x0 (also the initial residual)
        r_buf = torch.empty((T, H), dtype=torch.int16, device="cuda")
        xin = torch.empty((T, H), dtype=torch.int16, device="cuda")
        res0 = mb.residual(x0, r_buf, xin)
        res_l = mb.residual(r_buf, r_buf, xin)

    def stack_layer(l, ids_out=None):
        mb.layer_forward(dev_layers[l], x0 if l == 0 else xin, y, ws, res=res0 if l == 0 else res_l,
                         topk_ids=ids_out, c_layer=c_layers[l])

    def one_step(i, ids_out=None):
        if stack:
            for l in range(shape.layers):
                stack_layer(l, ids_out[l] if ids_out is not None else None)
        else:
            j = i % len(ring)
            mb.layer_forward(ring[j][0], ring[j][1], y, ws, topk_ids=ids_out, c_layer=c_layers[j])

    # warm-up (also the first launch of every kernel), timing the host side
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(args.warmup):
        one_step(i)
    host_ms = (time.perf_counter() - h0) * 1e3 / max(args.warmup, 1)
    torch.cuda.synchronize()

    # Timed region: K steps launched eagerly behind a bounded spin kernel long
    # enough for the host to enqueue every step first, so the GPU runs them
    # back to back.  The profiling hook records events around the gate/up
    # and down stages of every layer call of the last steps.
    K_steps = args.steps
    prof_steps = min(K_steps, 20)
    n_prof_calls = prof_steps * n_calls_per_step
    ev = {st: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_prof_calls)] for st in ("gateup", "down")}
    for st in ev:  # torch creates the HIP event at its first record
        for a_, b_ in ev[st]:
            a_.record(stream)
            b_.record(stream)
    torch.cuda.synchronize()
    sleep_ms = 1.5 * host_ms * K_steps + 10.0
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(sleep_ms * 1e-3 * 2.4e9))
    t_start.record(stream)
    call = 0
    for i in range(K_steps):
        prof = i >= K_steps - prof_steps
        if stack:
            for l in range(shape.layers):
                if prof:
                    for st in ev:
                        mb.profile_events(st, *ev[st][call])
                    call += 1
                stack_layer(l)
        else:
            if prof:
                for st in ev:
                    mb.profile_events(st, *ev[st][call])
                call += 1
            one_step(i)
    mb.profile_events(None)
    t_stop.record(stream)
    host_enqueue_ms = (time.perf_counter() - h0)
    torch.cuda.synchronize()
    elapsed_ms = t_start.elapsed_time(t_stop)
    ms_per_step = elapsed_ms / K_steps
    stage_us = {st: float(np.mean([hip_elapsed_ms(a_, b_) for a_, b_ in ev[st]])) * 1e3 for st in ev}
    log(f"host enqueue {host_ms:.3f} ms/step, spin {sleep_ms:.1f} ms; stage means: "
        + ", ".join(f"{k} {v:.2f} us" for k, v in stage_us.items()))

    # unique experts per call (units of the gate/up kernel), from the routing
    fmt = shape.fmt
    gu_bytes, dn_bytes = expert_bytes(fmt, H, F)
    sh_gu, sh_dn = expert_bytes(fmt, H, shape.shared_ffn) if shape.shared_ffn else (0, 0)
    if stack:
        ids_all = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(shape.layers)]
        one_step(0, ids_out=ids_all)
        torch.cuda.synchronize()
        uniq = [len(np.unique(t.cpu().numpy())) for t in ids_all]
    else:
        uniq = []
        for j in range(len(ring)):
            mb.layer_forward(ring[j][0], ring[j][1], y, ws, topk_ids=ids_buf, c_layer=c_layers[j])
            torch.cuda.synchronize()
            uniq.append(len(np.unique(ids_buf.cpu().numpy())))
    U = float(np.mean(uniq))
    # algorithmic bytes per launch of the two expert kernels: the unique
    # experts' (+ shared expert's) weights and scales, the activations read
    # and the results written
    Fs = shape.shared_ffn
    # decode calls of up to eight tokens without the normalised residual copy
    # take the one-launch down projection + combine (it writes y, not the
    # expert rows)
    fused_down = T <= 8 and not stack
    prefill = T > 16
    # the SwiGLU rows between the two kernels: bf16 hi + lo (4 bytes an
    # element) for decode calls, one fp16 plane (2 bytes) for prefill
    act_b = 2 if prefill else 4
    gateup_bytes = U * gu_bytes + sh_gu + T * H * 2 + (T * K * F + T * Fs) * act_b
    down_out = T * H * 4 if fused_down else (T * K + (T if Fs else 0)) * H * 4
    down_bytes = U * dn_bytes + sh_dn + (T * K * F + T * Fs) * act_b + down_out
    kern = {"gateup": (gateup_bytes, stage_us["gateup"]), "down": (down_bytes, stage_us["down"])}
    dom = max(kern, key=lambda k: kern[k][1])
    dom_bytes, dom_us = kern[dom]
    achieved_gbs = dom_bytes / (dom_us * 1e-6) / 1e9
    kernel_name = {("gateup", False): "gateup_mfma_kernel",
                   ("down", False): "down_combine_kernel" if fused_down else "down_mfma_kernel",
                   ("gateup", True): "gateup_gemm128_kernel", ("down", True): "down_gemm_kernel"}[(dom, prefill)]
    if prefill:
        # useful matrix-core work of the dominant grouped GEMM: every routed
        # and shared row through gate+up (2 H F each, 2 flops a product) or
        # down (H F), padding not counted
        rows = T * K + (T if shape.shared_ffn else 0)
        flops = {"gateup": 2.0 * rows * 2 * H * F, "down": 2.0 * rows * H * F}[dom]
        achieved_tf = flops / (dom_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved_tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved_tf / BF16_PEAK_TFLOPS, "traffic": measured_traffic(args.workload, kernel_name),
                    "kernel": kernel_name, "kernel_us": dom_us, "kernel_flops": flops, "kernel_bytes": dom_bytes,
                    "stage_us": stage_us}
    else:
        roofline = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload, kernel_name),
                    "kernel": kernel_name, "kernel_us": dom_us, "kernel_bytes": dom_bytes, "stage_us": stage_us}
    # whole-layer algorithmic bytes (router + unique experts + shared + x + y)
    layer_bytes = E * H * 4 + U * (gu_bytes + dn_bytes) + sh_gu + sh_dn + T * H * 2 + T * H * 4
    tokens_per_s = T * n_calls_per_step / (ms_per_step * 1e-3)
    log(f"ms/step {ms_per_step:.4f}; U={U:.1f}; gate/up {stage_us['gateup']:.2f} us -> "
        f"{gateup_bytes / (stage_us['gateup'] * 1e-6) / 1e9:.0f} GB/s; down {stage_us['down']:.2f} us -> "
        f"{down_bytes / (stage_us['down'] * 1e-6) / 1e9:.0f} GB/s; layer {layer_bytes / 1e6:.2f} MB -> "
        f"{layer_bytes / (ms_per_step / n_calls_per_step * 1e-3) / 1e9:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        # bounded sample: fresh tokens of the same workload through layer 0
        probe_T = threads
        xs = synth.make_x(synth.Shape(**{**shape.__dict__, "tokens": probe_T, "correlated_sigma": 0.0}),
                          seed=777)
        t1 = time.time()
        oracle.layer_forward(host_layer0, xs, nthreads=threads)
        dt = time.time() - t1
        reps = max(1, int(args.cpu_seconds / max(dt, 1e-3)))
        n_tok = min(probe_T * reps, 4096)
        xs = synth.make_x(synth.Shape(**{**shape.__dict__, "tokens": n_tok, "correlated_sigma": 0.0}), seed=778)
        t1 = time.time()
        oracle.layer_forward(host_layer0, xs, nthreads=threads)
        dt = time.time() - t1
        cpu = {"value": n_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n_tok} tokens, each through the first layer instance of this workload "
                         f"(double precision, {dt:.1f} s)"}
        log(f"oracle: {n_tok} tokens in {dt:.1f} s on {threads} threads")

    out = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA % (prefill), 1 GPU",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4-weights/bf16-act/f32-acc" if fmt == 2 else "int8-weights/bf16-act/f32-acc",
        "data": "synthetic (seeded generator, random-init weights of the layer's shapes)",
        "config": {"workload": synth.CONFIG_NAMES[cfg], "tokens": T, "hidden": H, "experts": E, "top_k": K,
                   "ffn": F, "shared_ffn": shape.shared_ffn, "layers_per_step": n_calls_per_step,
                   "distinct_layer_instances": len(dev_layers),
                   "unique_experts_per_call": U, "layer_GBps": layer_bytes / (ms_per_step / n_calls_per_step * 1e-3) / 1e9},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
