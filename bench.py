#!/usr/bin/env python3
"""Benchmark of the W8A8 MoE expert layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode]

A step is one moe_w8a8_forward over one batch (route, permute, activation
quant, GEMM1 + SwiGLU + requant, GEMM2, combine) with inputs and quantised
weights resident in HBM. The headline line is the 27B-class decode step
(32 tokens, hidden 4096, 64 experts, top-8, FFN 1536): tokens/s, plus the HBM
roofline of its dominant kernel (GEMM1) timed live with HIP events on the
layer's stream. The prefill of the same layer (16384 tokens) is measured too
and reported against the dense INT8 MFMA peak. The CPU oracle is timed on the
host on a bounded sample of the decode workload.

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 MoE layer tokens/s; HBM GB/s (decode) & INT8 MFMA % of peak (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
# Steps between two steps that carry stage events (decode; prefill steps all do).
EVENT_STRIDE = 10
COLD_FLUSH_BYTES = 512 << 20  # overwritten between cold-cache forwards
STAGE_INDEX = {s: i for i, s in enumerate(
    ("route", "scan", "scatter", "act_quant", "gemm1", "requant", "gemm2", "combine", "router"))}
# Sources of the kernels whose counter-measured traffic may be reused.
KERNEL_SOURCES = {
    "gemm1_stream": ["w8a8_int8_expert_amd/csrc/gemm_stream.hip",
                     "w8a8_int8_expert_amd/csrc/layer_device.h",
                     "w8a8_int8_expert_amd/csrc/moe_internal.h"],
    "gemm1_tiled": ["w8a8_int8_expert_amd/csrc/gemm_tiled.hip",
                    "w8a8_int8_expert_amd/csrc/layer_device.h",
                    "w8a8_int8_expert_amd/csrc/moe_internal.h"],
}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls bench needs (events), via the runtime torch loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed: %d" % rc)
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), if the
    kernel's source is unchanged since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("%s/%s" % (kernel, workload))
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec


class GpuLayer:
    def __init__(self, wl, layer, torch, fp8=False):
        import w8a8_int8_expert_amd as m
        self.m, self.torch, self.wl = m, torch, wl
        dev = torch.device("cuda")
        self.g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k, fp8=fp8)
        cx = torch.from_numpy(layer.calib_x.view("int16")).to(dev).view(torch.bfloat16)
        wg = torch.from_numpy(layer.w_gate).to(dev)
        wu = torch.from_numpy(layer.w_up).to(dev)
        wd = torch.from_numpy(layer.w_down).to(dev)
        self.g.calibrate(cx, wg, wu, wd, wl.alpha)
        torch.cuda.synchronize()
        del wg, wu, wd, cx
        torch.cuda.empty_cache()


def time_workload(gl: GpuLayer, wl, inputs, steps, warmup, hip, timed_stages, stride):
    torch, m = gl.torch, gl.m
    dev = torch.device("cuda")
    T = inputs.x.shape[0]
    x = torch.from_numpy(inputs.x.view("int16")).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(inputs.logits).to(dev) if inputs.logits is not None else None
    ids = torch.from_numpy(inputs.ids).to(dev) if inputs.ids is not None else None
    w = torch.from_numpy(inputs.w).to(dev) if inputs.w is not None else None
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device=dev)
    gl.g.workspace(T)
    # one untimed call to read back the per-expert row counts
    counts = torch.empty(wl.E, dtype=torch.int32, device=dev)
    dbg = m.moe_w8a8_debug()
    dbg.expert_counts = counts.data_ptr()
    gl.g.forward(x, logits, ids, w, wl.capacity_factor, out=out, debug=dbg)
    torch.cuda.synchronize()
    counts_h = counts.cpu().numpy()

    ev_arr = (ctypes.c_void_p * 18)()
    tdbg = m.moe_w8a8_debug()
    tdbg.stage_events = ctypes.cast(ev_arr, ctypes.POINTER(ctypes.c_void_p))
    for _ in range(warmup):
        gl.g.forward(x, logits, ids, w, wl.capacity_factor, out=out)
    torch.cuda.synchronize()
    # Stage events are stamped on every stride-th step of the timed loop only:
    # the event-carrying dispatches cost a few microseconds each, which would
    # otherwise be charged to every step of a ~0.2 ms decode step.
    sampled = list(range(0, steps, stride))
    pairs = {s: [(hip.event(), hip.event()) for _ in sampled] for s in timed_stages}
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % stride == 0:
            j = i // stride
            for s in timed_stages:
                ev_arr[2 * STAGE_INDEX[s]] = pairs[s][j][0]
                ev_arr[2 * STAGE_INDEX[s] + 1] = pairs[s][j][1]
            gl.g.forward(x, logits, ids, w, wl.capacity_factor, out=out, debug=tdbg)
        else:
            gl.g.forward(x, logits, ids, w, wl.capacity_factor, out=out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage_ms = {}
    for s in timed_stages:
        ms = [hip.elapsed_ms(a, b) for a, b in pairs[s]]
        stage_ms[s] = sum(ms) / len(ms)
        for a, b in pairs[s]:
            hip.destroy(a)
            hip.destroy(b)
    return dict(seconds=t1 - t0, stage_ms=stage_ms, counts=counts_h, out=out)


def time_cold(gl: GpuLayer, wl, inputs, steps, warmup):
    """Each forward timed alone by a pair of events on the layer's stream,
    with a 512 MiB buffer overwritten between forwards (outside the events),
    so that no weight is served from the 256 MB last-level cache: the case of
    a layer whose weights were evicted by the rest of a model. Returns the
    median and the minimum ms per forward."""
    torch = gl.torch
    dev = torch.device("cuda")
    T = inputs.x.shape[0]
    x = torch.from_numpy(inputs.x.view("int16")).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(inputs.logits).to(dev) if inputs.logits is not None else None
    ids = torch.from_numpy(inputs.ids).to(dev) if inputs.ids is not None else None
    w = torch.from_numpy(inputs.w).to(dev) if inputs.w is not None else None
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device=dev)
    gl.g.workspace(T)
    scratch = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device=dev)
    pairs = []
    for i in range(warmup + steps):
        scratch.fill_(i & 0x7F)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        gl.g.forward(x, logits, ids, w, wl.capacity_factor, out=out)
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in pairs[warmup:])
    del scratch
    return ms[len(ms) // 2], ms[0]


def time_router(gl: GpuLayer, wl, inputs, w_router, steps, warmup):
    """Router-projection mode: the whole layer routed from x and the bf16
    router matrix (ms per step), and the projection entry point alone."""
    torch = gl.torch
    dev = torch.device("cuda")
    x = torch.from_numpy(inputs.x.view("int16")).to(dev).view(torch.bfloat16)
    out = torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=dev)
    lg = torch.empty(wl.T, wl.E, dtype=torch.float32, device=dev)
    gl.g.set_router(torch.from_numpy(w_router.view("int16")).to(dev).view(torch.bfloat16))
    gl.g.workspace(wl.T)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    fwd_s = timed(lambda: gl.g.forward(x, None, None, None, wl.capacity_factor, out=out))
    lg_s = timed(lambda: gl.g.router_logits(x, out=lg))
    gl.g.set_router(None)
    flops = 2.0 * wl.T * wl.E * wl.H
    return {"forward_ms_per_step": round(fwd_s * 1e3, 5),
            "forward_tokens_per_s": round(wl.T / fwd_s, 1),
            "logits_us": round(lg_s * 1e6, 2),
            "logits_TFLOPs": round(flops / lg_s / 1e12, 2)}


def fp64_layer(layer, x_f32, ids, w):
    """The unquantised layer in fp64 from the fp32 weights (the reference the
    quantisation error is measured against): out[t] = sum_j w[t][j] *
    W_down[e] (silu(W_gate[e] x) * (W_up[e] x)), e = ids[t][j]."""
    T, k = ids.shape
    out = np.zeros((T, layer.w_down.shape[1]))
    x64 = x_f32.astype(np.float64)
    for e in np.unique(ids):
        t, j = np.nonzero(ids == e)
        xe = x64[t]
        g = xe @ layer.w_gate[e].astype(np.float64).T
        u = xe @ layer.w_up[e].astype(np.float64).T
        h = g / (1.0 + np.exp(-g)) * u
        y = h @ layer.w_down[e].astype(np.float64).T
        np.add.at(out, t, w[t, j][:, None].astype(np.float64) * y)
    return out


def alpha_sweep(gl: GpuLayer, layer, T, alphas, percentile):
    """Quantisation error of the whole layer against fp64_layer for each
    SmoothQuant alpha, without clipping, with the static percentile clip of
    the calibration and with dynamic per-token saturation at the same
    percentile: relative RMS error over T tokens of the decode layer."""
    import synth
    import w8a8_int8_expert_amd as m
    torch = gl.torch
    dev = torch.device("cuda")
    wl = synth.workload("decode", T=T)
    inputs = synth.make_inputs(wl, layer)
    x = torch.from_numpy(inputs.x.view("int16")).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(inputs.logits).to(dev)
    ids_t = torch.empty(T * wl.k, dtype=torch.int32, device=dev)
    w_t = torch.empty(T * wl.k, dtype=torch.float32, device=dev)
    dbg = m.moe_w8a8_debug()
    dbg.topk_ids, dbg.topk_w = ids_t.data_ptr(), w_t.data_ptr()
    cx = torch.from_numpy(layer.calib_x.view("int16")).to(dev).view(torch.bfloat16)
    wg = torch.from_numpy(layer.w_gate).to(dev)
    wu = torch.from_numpy(layer.w_up).to(dev)
    wd = torch.from_numpy(layer.w_down).to(dev)
    ref = None
    rows = []
    for a in alphas:
        gl.g.calibrate(cx, wg, wu, wd, a)
        gl.g.calibrate_clip(cx, percentile)
        for name, static, sat in (("none", False, 0.0),
                                  ("static_p%g" % percentile, True, 0.0),
                                  ("dynamic_p%g" % percentile, False, percentile)):
            gl.g.set_clip(static=static, sat_percentile=sat)
            out = gl.g.forward(x, logits, None, None, 0.0, debug=dbg)
            torch.cuda.synchronize()
            if ref is None:
                ids = ids_t.cpu().numpy().reshape(T, wl.k)
                w = w_t.cpu().numpy().reshape(T, wl.k)
                ref = fp64_layer(layer, synth.bf16_bits_to_f32(inputs.x), ids, w)
                rms = float(np.sqrt(np.mean(ref ** 2)))
            o = out.float().cpu().numpy().astype(np.float64)
            rows.append({"alpha": a, "clip": name,
                         "rel_rms_err": round(float(np.sqrt(np.mean((o - ref) ** 2))) / rms, 6)})
    gl.g.set_clip()
    del wg, wu, wd
    torch.cuda.empty_cache()
    return {"workload": "decode layer, %d tokens, logits routing" % T, "tokens": T,
            "percentile": percentile, "reference": "unquantised layer in fp64", "rows": rows}


def launched_stages(wl):
    """Stages that have a launch of their own (and so a timing pair): up to
    2048 assignments route, grouping and activation quantisation are one
    launch, timed as "route"."""
    fused = wl.T * wl.k <= 2048
    pre = ["route"] if fused else ["route", "scan", "scatter", "act_quant"]
    return pre + ["gemm1", "requant", "gemm2", "combine"]


def layer_bytes(wl, counts, T):
    touched = int((counts > 0).sum())
    b = touched * (3 * wl.H * wl.F + 4 * (2 * wl.F + wl.H)) + 4 * wl.H + 4 * T * wl.H
    b += 8 * T * wl.k if wl.pre_routed else 4 * T * wl.E
    return b, touched


def gemm1_bytes(wl, touched):
    return touched * (2 * wl.F * wl.H + 4 * 2 * wl.F)


def cpu_baseline(wl, layer, inputs, seconds):
    import oracle
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(inputs.x, cal, wl.k, logits=inputs.logits, ids=inputs.ids, w=inputs.w,
                       capacity_factor=wl.capacity_factor, want_acc1=False, want_h=False)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    T = inputs.x.shape[0]
    return {"value": round(T * reps / el, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%s workload (%d tokens, whole layer route..combine) x %d reps, %.1f s"
                      % (wl.name, T, reps, el)}


def copy_probe(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size (for scaling the HBM byte counters)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "prefill", "ep_share", "stress"])
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-router", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--alpha-sweep", action="store_true",
                    help="only the quantisation-error sweep over alpha and the clip variants")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        copy_probe(torch)
        return
    import synth
    import w8a8_int8_expert_amd as m
    m.load_library()
    hip = Hip()
    torch.cuda.set_device(0)

    wl = synth.workload(args.workload)
    layer_wl = synth.workload("decode") if wl.name == "prefill" else wl
    log("generating %s layer (H=%d F=%d E=%d)" % (layer_wl.name, wl.H, wl.F, wl.E))
    layer = synth.make_layer(layer_wl)
    gl = GpuLayer(layer_wl, layer, torch)
    if args.alpha_sweep:
        log("alpha sweep")
        print(json.dumps({"alpha_sweep": alpha_sweep(
            gl, layer, 128, [0.5, 0.55, 0.6, 0.65, 0.7], 99.9)}), flush=True)
        return
    inputs = synth.make_inputs(wl, layer)
    gl.wl = wl
    log("timing %s: %d warmup + %d steps" % (wl.name, args.warmup, args.steps))
    r = time_workload(gl, wl, inputs, args.steps, args.warmup, hip, launched_stages(wl),
                      EVENT_STRIDE if wl.name == "decode" else 1)
    T = wl.T
    sec = r["seconds"]
    ms_step = sec * 1e3 / args.steps
    tok_s = T * args.steps / sec
    lb, touched = layer_bytes(wl, r["counts"], T)
    A = int(r["counts"].sum())
    path = "stream" if T * wl.k <= 32 * wl.E else "tiled"
    gemm1_ms = r["stage_ms"]["gemm1"]
    if path == "stream":
        g1b = gemm1_bytes(wl, touched)
        achieved = g1b / (gemm1_ms * 1e-3) / 1e9
        traffic = stored_traffic("gemm1_stream", wl.name)
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic["bytes_per_launch"] if traffic else None,
                "kernel": "gemm_stream_kernel<gate/up> (GEMM1)",
                "algorithmic_bytes_per_launch": g1b, "avg_launch_us": round(gemm1_ms * 1e3, 2)}
    else:
        ops = 4 * A * wl.H * wl.F
        achieved = ops / (gemm1_ms * 1e-3) / 1e12
        traffic = stored_traffic("gemm1_tiled", wl.name)
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4),
                "traffic": traffic["bytes_per_launch"] if traffic else None,
                "kernel": "gemm_tiled_kernel<gate/up> (GEMM1)",
                "algorithmic_ops_per_launch": ops, "avg_launch_us": round(gemm1_ms * 1e3, 2)}
    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.description, "tokens": T, "hidden": wl.H, "experts": wl.E,
                   "top_k": wl.k, "ffn": wl.F, "gemm_path": path},
        "roofline": roof,
        "layer_hbm": {"algorithmic_bytes": lb, "touched_experts": touched,
                      "achieved_GBps": round(lb / sec * args.steps / 1e9, 1),
                      "frac": round(lb / sec * args.steps / 1e9 / HBM_PEAK_GBS, 4)},
        "layer_int8": {"algorithmic_ops": 6 * A * wl.H * wl.F,
                       "achieved_TOPs": round(6.0 * A * wl.H * wl.F / sec * args.steps / 1e12, 1),
                       "frac": round(6.0 * A * wl.H * wl.F / sec * args.steps / 1e12 /
                                     INT8_PEAK_TOPS, 4)},
        "stage_us": {k: round(v * 1e3, 2) for k, v in r["stage_ms"].items()},
    }
    log("timing %d forwards with the last-level cache flushed before each" % args.steps)
    cmed, cmin = time_cold(gl, wl, inputs, args.steps, args.warmup)
    res["cold_cache"] = {"flush_bytes": COLD_FLUSH_BYTES, "ms_per_step_median": round(cmed, 5),
                         "ms_per_step_min": round(cmin, 5),
                         "tokens_per_s_median": round(T / (cmed * 1e-3), 1)}
    if wl.name == "decode" and not args.no_prefill:
        pwl = synth.workload("prefill")
        log("timing prefill: 3 warmup + %d steps" % args.prefill_steps)
        pin = synth.make_inputs(pwl, layer)
        gl.wl = pwl
        pr = time_workload(gl, pwl, pin, args.prefill_steps, 3, hip, launched_stages(pwl), 1)
        pA = int(pr["counts"].sum())
        psec = pr["seconds"]
        g1ops = 4 * pA * pwl.H * pwl.F
        g2ops = 2 * pA * pwl.H * pwl.F
        g1 = g1ops / (pr["stage_ms"]["gemm1"] * 1e-3) / 1e12
        g2 = g2ops / (pr["stage_ms"]["gemm2"] * 1e-3) / 1e12
        layer_tops = (g1ops + g2ops) * args.prefill_steps / psec / 1e12
        res["prefill"] = {
            "workload": pwl.description, "tokens_per_s": round(pwl.T * args.prefill_steps / psec, 1),
            "ms_per_step": round(psec * 1e3 / args.prefill_steps, 4),
            "gemm1": {"achieved_TOPs": round(g1, 1), "frac_int8_peak": round(g1 / INT8_PEAK_TOPS, 4),
                      "avg_launch_us": round(pr["stage_ms"]["gemm1"] * 1e3, 1)},
            "gemm2": {"achieved_TOPs": round(g2, 1), "frac_int8_peak": round(g2 / INT8_PEAK_TOPS, 4),
                      "avg_launch_us": round(pr["stage_ms"]["gemm2"] * 1e3, 1)},
            "layer_frac_int8_peak": round(layer_tops / INT8_PEAK_TOPS, 4),
            "stage_us": {k: round(v * 1e3, 1) for k, v in pr["stage_ms"].items()},
        }
        del pr
    if wl.name == "decode" and not args.no_fp8:
        log("FP8 (e4m3) expert path: calibrating and timing decode")
        gf = GpuLayer(layer_wl, layer, torch, fp8=True)
        fr = time_workload(gf, wl, inputs, args.steps, args.warmup, hip, launched_stages(wl),
                           EVENT_STRIDE)
        fsec = fr["seconds"]
        g1b = gemm1_bytes(wl, touched)
        fp8 = {"decode": {
            "tokens_per_s": round(T * args.steps / fsec, 1),
            "ms_per_step": round(fsec * 1e3 / args.steps, 5),
            "gemm1_hbm_frac": round(g1b / (fr["stage_ms"]["gemm1"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "layer_hbm_frac": round(lb / fsec * args.steps / 1e9 / HBM_PEAK_GBS, 4),
            "stage_us": {k: round(v * 1e3, 2) for k, v in fr["stage_ms"].items()}}}
        if not args.no_prefill:
            log("FP8 prefill: 3 warmup + %d steps" % args.prefill_steps)
            pwl = synth.workload("prefill")
            gf.wl = pwl
            pin = synth.make_inputs(pwl, layer)
            pr = time_workload(gf, pwl, pin, args.prefill_steps, 3, hip, launched_stages(pwl), 1)
            pA = int(pr["counts"].sum())
            ops = 6.0 * pA * pwl.H * pwl.F
            fp8["prefill"] = {
                "tokens_per_s": round(pwl.T * args.prefill_steps / pr["seconds"], 1),
                "ms_per_step": round(pr["seconds"] * 1e3 / args.prefill_steps, 4),
                "layer_frac_fp8_peak": round(ops * args.prefill_steps / pr["seconds"] / 1e12 /
                                             FP8_PEAK_TFLOPS, 4),
                "gemm1_frac_fp8_peak": round(4.0 * pA * pwl.H * pwl.F /
                                             (pr["stage_ms"]["gemm1"] * 1e-3) / 1e12 /
                                             FP8_PEAK_TFLOPS, 4),
                "stage_us": {k: round(v * 1e3, 1) for k, v in pr["stage_ms"].items()}}
            del pr
        res["fp8"] = fp8
        del gf, fr
        torch.cuda.empty_cache()
    if wl.name == "decode" and not args.no_router:
        log("timing router-projection mode")
        w_router = synth.make_router(layer_wl)
        rp = {"decode": time_router(gl, wl, inputs, w_router, args.steps, args.warmup)}
        if not args.no_prefill:
            pwl = synth.workload("prefill")
            rp["prefill"] = time_router(gl, pwl, synth.make_inputs(pwl, layer), w_router,
                                        args.prefill_steps, 3)
        res["router_projection"] = rp
    res["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle for %.0f s" % args.cpu_seconds)
        res["cpu_baseline"] = cpu_baseline(wl, layer, inputs, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
