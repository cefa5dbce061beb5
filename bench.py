#!/usr/bin/env python3
"""Benchmark of the MoE layer on one MI355X.

A step is one pass of the whole hot path (router, top-k, permutation, routed
experts, shared expert, combine) over one batch of synthetic input already
resident in HBM.  Default workload: the 16-request decode batch through a
stack of 40 distinct int4 layers with the residual epilogue between layers
(16 tokens, H=2048, 256 experts, top-8, F=512 + a shared expert, Zipf(1.1)
expert popularity; 18.3 GB of weights resident), the largest single-GPU
workload, run as one moe_stack_forward call a step.  The same line carries
the 2048-token int4 prefill chunk as a
nested object ("prefill") with its own roofline against the matrix-core
peak, and the same chunk in the W8A8 variant (int8 weights, int8
activations: "prefill_w8a8") against the HBM peak.  Other primary workloads:
--workload decode-int8 | mtp-verify-int4 | prefill-int4 | prefill-int8-w8a8
| tiny-int8 (decode workloads rotate over a ring of 40 layer instances so
that no call finds its weights in the 256 MB last-level cache).  Each HBM
roofline also carries the rate a plain device copy of the same traffic
reaches in one launch (copy_ceiling_gbs) and the rate of a plain read-only
launch of the same bytes (read_ceiling_gbs); the prefill roofline also
carries the rate of a pure matrix-core kernel (mfma_achievable_tflops).

Timing: W warm-up steps, then R repetitions (default 5) of K steps each,
every repetition launched on one stream behind a bounded spin kernel long
enough for the host to enqueue all K steps first (so the GPU runs them back
to back), bracketed by synchronisation and HIP events; ms_per_step is the
median repetition.  No profiling happens inside the timed repetitions.
Afterwards a separate pass of a few steps (the stack as separate
moe_layer_forward calls) asks the library (per-call options) for HIP events
at the start and end of the gate/up and down kernels; the slower of the two is the dominant kernel, and its mean
duration over that pass gives the roofline figure.  The CPU oracle is timed
on a bounded sample of the same workload on the host cores.  Prints one JSON
line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA

WORKLOADS = {
    "decode-int8": 1,
    "mtp-verify-int4": 2,
    "batch16-stack-int4": 3,
    "prefill-int4": 4,
    "tiny-int8": 0,
    "prefill-int8-w8a8": 4,  # the prefill chunk with int8 row-scaled weights and int8 activations
}
# per-workload changes of the configuration's shape and per-call options
WORKLOAD_SHAPE = {"prefill-int8-w8a8": {"fmt": 1}}
WORKLOAD_OPTS = {"prefill-int8-w8a8": {"act_quant": 1}}
INT8_PEAK_TOPS = 5033.2  # MI355X dense int8 MFMA
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA % (prefill), 1 GPU"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(workload, kernel):
    """HBM bytes per launch of a kernel from the committed counter runs
    (profiles/hbm_traffic.json: FETCH_SIZE and WRITE_SIZE scaled by a plain
    copy of known size), or None when there is no such run or a source file
    the kernel is built from has changed since it was taken."""
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


def copy_ceiling_gbs(torch, traffic_bytes, n_copies=60):
    """HBM rate (GB/s of traffic) of the runtime's plain device copy moving
    the given number of bytes in one launch (half read, half written): the
    streaming rate one launch of that size reaches, the practical ceiling
    beside the 8 TB/s peak for a kernel of the same traffic.  The copies
    rotate over a pool of buffers so that none starts from data the
    256 MB last-level cache still holds: the sources together hold at least
    1 GiB, and one comes round again only after all the others."""
    half = max(int(traffic_bytes) // 2 // 256 * 256, 256)
    n_src = max(2, min(512, (1 << 30) // half + 1))
    srcs = [torch.empty(half, dtype=torch.uint8, device="cuda").fill_(i & 0xFF) for i in range(n_src)]
    dsts = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for i in range(4):
        dsts[i % 2].copy_(srcs[i % n_src])
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e-3 * 2.4e9))
    a.record()
    for i in range(n_copies):
        dsts[i % 2].copy_(srcs[(i + 4) % n_src])
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n_copies
    del srcs, dsts
    torch.cuda.empty_cache()
    return 2 * half / (us * 1e-6) / 1e9


def read_ceiling_gbs(torch, mb, nbytes, n_reads=40):
    """Read rate (GB/s) of the library's plain read-stream kernel
    (moe_calib_read) reading the given number of bytes in one launch: the
    achievable rate of a kernel that only streams that many bytes, beside
    the 8 TB/s peak.  The sources rotate over at least 1 GiB so that none is
    still in the 256 MB last-level cache; median of n_reads launches."""
    n = max(int(nbytes) // 256 * 256, 256)
    n_src = max(2, min(512, (1 << 30) // n + 1))
    srcs = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i & 0xFF) for i in range(n_src)]
    torch.cuda.synchronize()
    for i in range(3):
        mb.calib_read(srcs[i % n_src], n)
    ms = sorted(mb.calib_read(srcs[(i + 3) % n_src], n) for i in range(n_reads))
    del srcs
    torch.cuda.empty_cache()
    return n / (ms[len(ms) // 2] * 1e-3) / 1e9


def mfma_achievable_tflops(mb, kind):
    """Issue rate (TFLOP/s, or TOP/s for int8) of the library's pure matrix-core
    kernel (moe_calib_mfma): kind 0 fp16 32x32x16, 2 int8 32x32x32; the best
    of three launches of about a millisecond."""
    best = 0.0
    for _ in range(3):
        ms, ops = mb.calib_mfma(kind, 10000)
        best = max(best, ops / (ms * 1e-3) / 1e12)
    return best


class Workload:
    """Device-resident inputs of one workload and its step function."""

    def __init__(self, name, ring_size, torch, mb, synth):
        import dataclasses
        self.name = name
        self.cfg = WORKLOADS[name]
        self.shape = dataclasses.replace(synth.CONFIGS[self.cfg], **WORKLOAD_SHAPE.get(name, {}))
        self.opts_kw = WORKLOAD_OPTS.get(name, {})
        self.opts = mb.forward_opts(**self.opts_kw) if self.opts_kw else None
        self.torch, self.mb, self.synth = torch, mb, synth
        shp = self.shape
        self.T, self.H, self.E, self.K, self.F = shp.tokens, shp.hidden, shp.n_experts, shp.top_k, shp.ffn
        self.stack = self.cfg == 3
        self.label = synth.CONFIG_NAMES[self.cfg]
        if self.opts_kw.get("act_quant"):
            self.label = self.label.replace("int4", "W8A8 (int8 row-scaled weights, int8 activations)")
        log(f"workload {name}: {self.label}")
        t0 = time.time()
        if self.stack:
            self.layers = []
            for l in range(shp.layers):
                host = synth.make_layer(shp, layer=l)
                self.layers.append(mb.layer_to_device(host))
                if l == 0:
                    self.host_layer0 = host
                del host
                if (l + 1) % 10 == 0:
                    log(f"  stack: {l + 1}/{shp.layers} layers resident")
            self.x_host = synth.make_x(shp)
            self.x0 = torch.from_numpy(self.x_host.view(np.int16)).cuda()
            self.xs = None
            self.calls_per_step = shp.layers
        else:
            import dataclasses
            n_inst = 2 if self.cfg == 4 else (1 if self.cfg == 0 else ring_size)
            self.layers, self.xs = [], []
            for i in range(n_inst):
                s_i = dataclasses.replace(shp, seed=shp.seed if i == 0 else 100_000 + 97 * i)
                host = synth.make_layer(s_i)
                x = synth.make_x(s_i)
                self.layers.append(mb.layer_to_device(host))
                self.xs.append(torch.from_numpy(x.view(np.int16)).cuda())
                if i == 0:
                    self.host_layer0, self.x_host = host, x
                del host
            self.calls_per_step = 1
        torch.cuda.synchronize()
        log(f"  inputs resident in {time.time() - t0:.1f} s")
        self.c_layers = [dl.c() for dl in self.layers]
        self.c_stack = mb.stack_arrays(self.c_layers) if self.stack else None
        self.ws = mb.make_workspace(self.layers[0], self.T)
        self.y = torch.empty((self.T, self.H), dtype=torch.float32, device="cuda")
        if self.stack:
            # residual stream r and the next layer's RMS-normalised input xin,
            # both updated in place by the layers' combine epilogue; layer 0
            # reads the step's initial input x0 (also the initial residual)
            self.r_buf = torch.empty((self.T, self.H), dtype=torch.int16, device="cuda")
            self.xin = torch.empty((self.T, self.H), dtype=torch.int16, device="cuda")
            self.res0 = mb.residual(self.x0, self.r_buf, self.xin)
            self.res_l = mb.residual(self.r_buf, self.r_buf, self.xin)

    def call(self, i, l, ids_out=None, opts=None):
        """Layer call l of step i."""
        mb = self.mb
        opts = self.opts if opts is None else opts
        if self.stack:
            mb.layer_forward(self.layers[l], self.x0 if l == 0 else self.xin, self.y, self.ws,
                             res=self.res0 if l == 0 else self.res_l, topk_ids=ids_out, c_layer=self.c_layers[l],
                             opts=opts)
        else:
            j = i % len(self.layers)
            mb.layer_forward(self.layers[j], self.xs[j], self.y, self.ws, topk_ids=ids_out, c_layer=self.c_layers[j],
                             opts=opts)

    def step(self, i):
        if self.stack:
            # one moe_stack_forward call: the 40 layers chained by the
            # residual stream, each layer's combine also forming the next
            # layer's router product
            self.mb.stack_forward(self.c_stack, self.x0, self.x0, self.r_buf, self.xin, self.y, self.ws)
            return
        for l in range(self.calls_per_step):
            self.call(i, l)

    def unique_experts(self):
        """Unique experts each layer call of one step actually routed to."""
        torch = self.torch
        uniq = []
        ids = torch.empty((self.T, self.K), dtype=torch.int32, device="cuda")
        n_calls = self.calls_per_step if self.stack else len(self.layers)
        for c in range(n_calls):
            if self.stack:
                self.call(0, c, ids_out=ids)
            else:
                self.call(c, 0, ids_out=ids)
            torch.cuda.synchronize()
            uniq.append(len(np.unique(ids.cpu().numpy())))
        return float(np.mean(uniq))


def time_steps(wl, K_steps, reps, host_ms):
    """R repetitions of K back-to-back steps; returns the per-step times (ms)."""
    torch = wl.torch
    stream = torch.cuda.current_stream()
    out = []
    for r in range(reps):
        sleep_ms = 1.5 * host_ms * K_steps + 10.0
        t_start = torch.cuda.Event(enable_timing=True)
        t_stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(sleep_ms * 1e-3 * 2.4e9))
        t_start.record(stream)
        for i in range(K_steps):
            wl.step(i)
        t_stop.record(stream)
        torch.cuda.synchronize()
        out.append(t_start.elapsed_time(t_stop) / K_steps)
    return out


def stage_times(wl, n_steps, host_ms):
    """Mean kernel durations (us) of the gate/up and down stages over n_steps
    profiled steps (events requested per call, outside the timed region).
    As in the timed repetitions, the calls are queued behind a spin kernel
    first, so that the GPU runs them back to back rather than each on an
    idle device."""
    torch, mb = wl.torch, wl.mb
    stream = torch.cuda.current_stream()
    n_calls = n_steps * wl.calls_per_step
    ev = {st: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_calls)] for st in ("route", "gateup", "down")}
    for st in ev:  # torch creates the HIP event at its first record
        for a_, b_ in ev[st]:
            a_.record(stream)
            b_.record(stream)
    opts = [mb.forward_opts(events={st: ev[st][c] for st in ev}, **wl.opts_kw) for c in range(n_calls)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int((1.5 * host_ms * n_steps + 10.0) * 1e-3 * 2.4e9))
    c = 0
    for i in range(n_steps):
        for l in range(wl.calls_per_step):
            wl.call(i, l, opts=opts[c])
            c += 1
    torch.cuda.synchronize()
    return {st: float(np.mean([hip_elapsed_ms(a_, b_) for a_, b_ in ev[st]])) * 1e3 for st in ev}


def measure(wl, K_steps, warmup, reps, prof_steps):
    torch, mb = wl.torch, wl.mb
    shp = wl.shape
    T, H, E, K, F = wl.T, wl.H, wl.E, wl.K, wl.F
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(warmup):
        wl.step(i)
    host_ms = (time.perf_counter() - h0) * 1e3 / max(warmup, 1)
    torch.cuda.synchronize()
    per_rep = time_steps(wl, K_steps, reps, host_ms)
    ms_per_step = float(np.median(per_rep))
    # single-call steps: at least 20 profiled calls
    stage_us = stage_times(wl, prof_steps if wl.calls_per_step > 1 else max(prof_steps, 20), host_ms)
    U = wl.unique_experts()
    log(f"  host enqueue {host_ms:.3f} ms/step; repetitions (ms/step): "
        + ", ".join(f"{v:.4f}" for v in per_rep) + "; stage means: "
        + ", ".join(f"{k} {v:.2f} us" for k, v in stage_us.items()))

    # algorithmic bytes per launch of the two expert kernels: the unique
    # experts' (+ shared expert's) weights and scales, the activations read
    # and the results written
    fmt = shp.fmt
    gu_bytes, dn_bytes = expert_bytes(fmt, H, F)
    Fs = shp.shared_ffn
    sh_gu, sh_dn = expert_bytes(fmt, H, Fs) if Fs else (0, 0)
    # decode calls of up to eight tokens without the normalised residual copy
    # take the one-launch down projection + combine (it writes y, not the
    # expert rows)
    fused_down = T <= 8 and not wl.stack
    prefill = T > 16
    w8a8 = bool(wl.opts_kw.get("act_quant"))
    rows = T * K + (T if Fs else 0)
    if w8a8:
        # int8 x rows in, fp32 SwiGLU rows out; int8 SwiGLU rows in, fp16 rows out
        gateup_bytes = U * gu_bytes + sh_gu + T * H + rows * F * 4
        down_bytes = U * dn_bytes + sh_dn + rows * F + rows * H * 2
    else:
        # the SwiGLU rows between the two kernels: bf16 hi + lo (4 bytes an
        # element) for decode calls, one fp16 plane (2 bytes) for prefill
        act_b = 2 if prefill else 4
        gateup_bytes = U * gu_bytes + sh_gu + T * H * 2 + (T * K * F + T * Fs) * act_b
        # expert output rows: fp32 from the decode kernels, fp16 from the
        # prefill GEMMs; the one-launch down + combine writes y instead
        down_out = T * H * 4 if fused_down else (T * K + (T if Fs else 0)) * H * (2 if prefill else 4)
        down_bytes = U * dn_bytes + sh_dn + (T * K * F + T * Fs) * act_b + down_out
    kern = {"gateup": (gateup_bytes, stage_us["gateup"]), "down": (down_bytes, stage_us["down"])}
    dom = max(kern, key=lambda k: kern[k][1])
    dom_bytes, dom_us = kern[dom]
    kernel_name = {("gateup", False): "gateup_mfma_kernel",
                   ("down", False): "down_combine_kernel" if fused_down else "down_mfma_kernel",
                   ("gateup", True): "gateup_gemm128_kernel", ("down", True): "down_gemm_kernel"}[(dom, prefill)]
    if w8a8:
        kernel_name = "w8a8_gemm_kernel<true>" if dom == "gateup" else "w8a8_gemm_kernel<false>"
        # int8 weights: the weight stream bounds these GEMMs (the int8 matrix
        # work is a fifth of the weight-stream time at the peaks); the
        # matrix-core fraction is reported beside it
        ops = {"gateup": 2.0 * rows * 2 * H * F, "down": 2.0 * rows * H * F}[dom]
        achieved = dom_bytes / (dom_us * 1e-6) / 1e9
        int8_ach = mfma_achievable_tflops(mb, 2)
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(wl.name, kernel_name),
                    "kernel": kernel_name, "kernel_us": dom_us, "kernel_bytes": dom_bytes, "kernel_int8_ops": ops,
                    "int8_mfma_frac": ops / (dom_us * 1e-6) / 1e12 / INT8_PEAK_TOPS,
                    "int8_achievable_tops": int8_ach,
                    "int8_frac_of_achievable": ops / (dom_us * 1e-6) / 1e12 / int8_ach, "stage_us": stage_us,
                    "copy_ceiling_gbs": copy_ceiling_gbs(torch, dom_bytes),
                    "read_ceiling_gbs": read_ceiling_gbs(torch, mb, dom_bytes)}
    elif prefill:
        # useful matrix-core work of the dominant grouped GEMM: every routed
        # and shared row through gate+up (2 H F each, 2 flops a product) or
        # down (H F), padding not counted
        rows = T * K + (T if Fs else 0)
        flops = {"gateup": 2.0 * rows * 2 * H * F, "down": 2.0 * rows * H * F}[dom]
        achieved = flops / (dom_us * 1e-6) / 1e12
        f16_ach = mfma_achievable_tflops(mb, 0)
        roofline = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / BF16_PEAK_TFLOPS, "traffic": measured_traffic(wl.name, kernel_name),
                    "kernel": kernel_name, "kernel_us": dom_us, "kernel_flops": flops, "kernel_bytes": dom_bytes,
                    "mfma_achievable_tflops": f16_ach, "frac_of_achievable": achieved / f16_ach,
                    "stage_us": stage_us}
    else:
        achieved = dom_bytes / (dom_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(wl.name, kernel_name),
                    "kernel": kernel_name, "kernel_us": dom_us, "kernel_bytes": dom_bytes, "stage_us": stage_us,
                    "copy_ceiling_gbs": copy_ceiling_gbs(torch, dom_bytes),
                    "read_ceiling_gbs": read_ceiling_gbs(torch, mb, dom_bytes)}
    # whole-layer algorithmic bytes (router + unique experts + shared + x + y)
    layer_bytes = E * H * 4 + U * (gu_bytes + dn_bytes) + sh_gu + sh_dn + T * H * 2 + T * H * 4
    layer_ms = ms_per_step / wl.calls_per_step
    tokens_per_s = T * wl.calls_per_step / (ms_per_step * 1e-3)
    log(f"  ms/step {ms_per_step:.4f} (median of {reps}); U={U:.1f}; gate/up {stage_us['gateup']:.2f} us -> "
        f"{gateup_bytes / (stage_us['gateup'] * 1e-6) / 1e9:.0f} GB/s; down {stage_us['down']:.2f} us -> "
        f"{down_bytes / (stage_us['down'] * 1e-6) / 1e9:.0f} GB/s; layer {layer_bytes / 1e6:.2f} MB -> "
        f"{layer_bytes / (layer_ms * 1e-3) / 1e9:.0f} GB/s")
    config = {"workload": wl.label, "tokens": T, "hidden": H, "experts": E, "top_k": K,
              "ffn": F, "shared_ffn": Fs, "layers_per_step": wl.calls_per_step,
              "distinct_layer_instances": len(wl.layers), "unique_experts_per_call": U,
              "layer_bytes": layer_bytes, "layer_us": layer_ms * 1e3,
              "layer_GBps": layer_bytes / (layer_ms * 1e-3) / 1e9}
    if wl.stack:
        config["stack_tokens_per_s"] = T / (ms_per_step * 1e-3)
    return {"value": tokens_per_s, "ms_per_step": ms_per_step, "ms_per_step_reps": per_rep,
            "dtype": ("int8-weights/int8-act/i32-acc" if w8a8 else
                      "int4-weights/bf16-act/f32-acc" if fmt == 2 else "int8-weights/bf16-act/f32-acc"),
            "config": config, "roofline": roofline}


def cpu_baseline(wl, seconds):
    """The oracle on the host cores, on a bounded sample of fresh tokens of
    the workload through its first layer instance (MoE-layer tokens/s, the
    unit of the GPU figure), plus a one-thread figure."""
    import oracle
    synth = wl.synth
    hw = os.cpu_count() or 1
    threads = max(1, min(16, hw))
    shape = wl.shape

    def sample(n_tok, seed):
        return synth.make_x(synth.Shape(**{**shape.__dict__, "tokens": n_tok, "correlated_sigma": 0.0}), seed=seed)

    xs = sample(threads, 777)
    t1 = time.time()
    oracle.layer_forward(wl.host_layer0, xs, nthreads=threads)
    dt = time.time() - t1
    reps = max(1, int(seconds / max(dt, 1e-3)))
    n_tok = min(threads * reps, 4096)
    xs = sample(n_tok, 778)
    t1 = time.time()
    oracle.layer_forward(wl.host_layer0, xs, nthreads=threads)
    dt = time.time() - t1
    x1 = sample(2, 779)
    t2 = time.time()
    oracle.layer_forward(wl.host_layer0, x1, nthreads=1)
    dt1 = time.time() - t2
    log(f"  oracle: {n_tok} tokens in {dt:.1f} s on {threads} threads (host has {hw}); 1 thread: 2 tokens in "
        f"{dt1:.2f} s")
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_tok} tokens, each through the first layer instance of this workload "
                      f"(double precision, {dt:.1f} s)",
            "host_cpus": hw, "value_1thread": 2 / dt1}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="steps per timed repetition")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions (the median is reported)")
    ap.add_argument("--prof-steps", type=int, default=5, help="profiled steps after the timed repetitions")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="batch16-stack-int4")
    ap.add_argument("--no-prefill", action="store_true",
                    help="leave out the nested prefill-chunk measurements (int4, and int8 W8A8) of the default line")
    ap.add_argument("--ring", type=int, default=40, help="distinct layer instances (decode workloads)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (20 times), the known-size reference for "
                         "the HBM byte counters, and exit")
    ap.add_argument("--copy-sweep", action="store_true",
                    help="only time the plain device copy and the library's read-stream kernel over a range of "
                         "sizes (the streaming rates one launch of each size reaches) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs on one GPU (expert-parallel sharding is a "
              "design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_sweep:
        import torch
        from mixture_experts_decode_moe_amd import binding as mb
        for mib in (4, 8, 16, 36, 64, 128, 256, 1024):
            g = copy_ceiling_gbs(torch, mib << 20)
            r = read_ceiling_gbs(torch, mb, mib << 20)
            print(json.dumps({"copy_traffic_mib": mib, "GBps": g, "read_GBps": r}), flush=True)
        return

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

    import torch
    from mixture_experts_decode_moe_amd import binding as mb
    from mixture_experts_decode_moe_amd import synth

    torch.cuda.set_device(0)
    wl = Workload(args.workload, args.ring, torch, mb, synth)
    res = measure(wl, args.steps, args.warmup, args.reps, args.prof_steps)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args.cpu_seconds)

    nested = {}
    if args.workload == "batch16-stack-int4" and not args.no_prefill:
        del wl  # frees the stack's 18 GB before the prefill layers are made
        torch.cuda.empty_cache()
        for key, name in (("prefill", "prefill-int4"), ("prefill_w8a8", "prefill-int8-w8a8")):
            pf = Workload(name, args.ring, torch, mb, synth)
            r = measure(pf, args.steps, args.warmup, args.reps, args.prof_steps)
            nested[key] = {"metric": METRIC, "value": r["value"], "unit": "tokens/s", "ms_per_step": r["ms_per_step"],
                           "ms_per_step_reps": r["ms_per_step_reps"], "steps": args.steps, "dtype": r["dtype"],
                           "config": r["config"], "roofline": r["roofline"]}
            del pf
            torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic (seeded generator, random-init weights of the layer's shapes)",
        "config": res["config"],
        "repetitions": args.reps,
        "ms_per_step_reps": res["ms_per_step_reps"],
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
    }
    out.update(nested)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
