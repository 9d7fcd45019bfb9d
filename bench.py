#!/usr/bin/env python3
"""Benchmark of the W8A8 MoE expert layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one moe_w8a8_forward over one batch (route, permute, activation
quant, GEMM1 + SwiGLU + requant, GEMM2, combine) with inputs and quantised
weights resident in HBM. Each of the K timed steps is timed alone by a pair of
HIP events, with a 512 MiB buffer overwritten between steps (outside the
events), so that no weight is served from the 256 MB last-level cache; the
headline is the median (the minimum and the back-to-back mean are reported
too). The headline workload is the 27B-class decode step (32 tokens, hidden
4096, 64 experts, top-8, FFN 1536); the prefill of the same layer (16384
tokens), the tiny layer, one GPU's expert-parallel share and the outlier/skew
stress layer are measured the same way and reported under "configs", each with
its HBM and INT8 fractions of the algorithmic work, per-stage launch times
(dispatch-stamped events, averaged over max(20, K) launches) and the CPU
oracle's tokens/s on a bounded sample of the same workload.

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
    """Algorithmic HBM bytes of one forward: the touched experts' INT8 weights
    and scales, inv_s, x in and out (bf16), and the routing input (fp32 logits,
    or ids and weights when pre-routed)."""
    touched = int((counts > 0).sum())
    b = touched * (3 * wl.H * wl.F + 4 * (2 * wl.F + wl.H)) + 4 * wl.H + 4 * T * wl.H
    b += 8 * T * wl.k if wl.pre_routed else 4 * T * wl.E
    return b, touched


def gemm1_bytes(wl, touched):
    return touched * (2 * wl.F * wl.H + 4 * 2 * wl.F)


def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


# Bounded samples of each workload for the CPU oracle: (tokens, minimum seconds).
ORACLE_SAMPLE = {"tiny": (None, 2.0), "decode": (None, 10.0), "prefill": (512, 0.0),
                 "ep_share": (1024, 0.0), "stress": (256, 0.0)}


def cpu_baseline(wl, cal, inputs):
    """The oracle (as it stands) on a bounded sample of the workload: the whole
    sample repeated for at least the sample's minimum seconds (at least once)."""
    import oracle
    n, min_s = ORACLE_SAMPLE[wl.name]
    T = inputs.x.shape[0] if n is None else min(n, inputs.x.shape[0])
    sl = slice(0, T)
    kw = dict(logits=None if inputs.logits is None else inputs.logits[sl],
              ids=None if inputs.ids is None else inputs.ids[sl],
              w=None if inputs.w is None else inputs.w[sl])
    x = inputs.x[sl]
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(x, cal, wl.k, capacity_factor=wl.capacity_factor, want_acc1=False,
                       want_h=False, **kw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            break
    what = "all %d tokens" % T if n is None else "the first %d of %d tokens" % (T, wl.T)
    if n is not None and wl.capacity_factor > 0:
        what += " (capacity taken over the sample)"
    return {"value": round(T * reps / el, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%s workload, %s, whole layer route..combine, x %d, %.1f s"
                      % (wl.name, what, reps, el)}


def copy_probe(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size (for scaling the HBM byte counters)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


def dense_int8_reference(torch, steps=10):
    """The vendor library's dense INT8 GEMM (hipBLASLt through torch._int_mm,
    int32 output) on the prefill GEMMs' shapes: all 131072 rows against one
    expert's weights, with no gather, grouping or epilogue. Context for the
    grouped kernels' INT8 fractions, timed with events on the same stream."""
    dev = torch.device("cuda")
    out = {}
    for name, (M, K, N) in (("gemm1_shape", (131072, 4096, 3072)),
                            ("gemm2_shape", (131072, 1536, 4096))):
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
        b = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev).t()
        for _ in range(2):
            torch._int_mm(a, b)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for e0, e1 in ev:
            e0.record()
            torch._int_mm(a, b)
            e1.record()
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[steps // 2]
        tops = 2.0 * M * K * N / (ms * 1e-3) / 1e12
        out[name] = {"M": M, "K": K, "N": N, "ms_median": round(ms, 4), "TOPs": round(tops, 1),
                     "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
        del a, b
        torch.cuda.empty_cache()
    out["library"] = "hipBLASLt via torch._int_mm (dense, int32 output)"
    return out


def make_layer_for(name):
    """(the layer's workload, the layer): prefill runs on the decode layer."""
    import synth
    lwl = synth.workload("decode") if name == "prefill" else synth.workload(name)
    log("generating the %s layer (H=%d F=%d E=%d)" % (lwl.name, lwl.H, lwl.F, lwl.E))
    return lwl, synth.make_layer(lwl)


def measure(gl, wl, inputs, steps, warmup, hip):
    """One workload: flushed per-forward times (median and minimum, the headline
    form), the back-to-back mean, and every stage's average launch time over
    max(20, steps) dispatch-stamped launches."""
    t_mean = time_workload(gl, wl, inputs, steps, warmup, hip, [], 1)
    cmed, cmin = time_cold(gl, wl, inputs, steps, warmup)
    st = time_workload(gl, wl, inputs, max(20, steps), 2, hip, launched_stages(wl), 1)
    return dict(ms_median=cmed, ms_min=cmin, ms_b2b=t_mean["seconds"] * 1e3 / steps,
                stage_ms=st["stage_ms"], counts=t_mean["counts"], n_stage=max(20, steps))


def config_block(wl, m_):
    """Per-workload record: tokens/s at the flushed median, HBM and INT8
    fractions of the algorithmic work, stage times and the dominant kernel."""
    T = wl.T
    lb, touched = layer_bytes(wl, m_["counts"], T)
    A = int(m_["counts"].sum())
    ops = 6 * A * wl.H * wl.F
    sec = m_["ms_median"] * 1e-3
    g1, g2 = m_["stage_ms"]["gemm1"] * 1e-3, m_["stage_ms"]["gemm2"] * 1e-3
    stream = T * wl.k <= 32 * wl.E
    blk = {
        "workload": wl.description, "tokens": T, "kept_rows": A, "touched_experts": touched,
        "gemm_path": "stream" if stream else "tiled",
        "tokens_per_s": round(T / sec, 1),
        "ms_per_step_median": round(m_["ms_median"], 5), "ms_per_step_min": round(m_["ms_min"], 5),
        "ms_per_step_back_to_back": round(m_["ms_b2b"], 5),
        "hbm": {"algorithmic_bytes": lb, "GBps": round(lb / sec / 1e9, 1),
                "frac": round(lb / sec / 1e9 / HBM_PEAK_GBS, 4)},
        "int8": {"algorithmic_ops": ops, "TOPs": round(ops / sec / 1e12, 1),
                 "frac": round(ops / sec / 1e12 / INT8_PEAK_TOPS, 4)},
        "gemm1": {"avg_launch_us": round(g1 * 1e6, 2),
                  "hbm_frac": round(gemm1_bytes(wl, touched) / g1 / 1e9 / HBM_PEAK_GBS, 4),
                  "int8_frac": round(4.0 * A * wl.H * wl.F / g1 / 1e12 / INT8_PEAK_TOPS, 4)},
        "gemm2": {"avg_launch_us": round(g2 * 1e6, 2),
                  "hbm_frac": round(touched * (wl.H * wl.F + 4 * wl.H) / g2 / 1e9 / HBM_PEAK_GBS,
                                    4),
                  "int8_frac": round(2.0 * A * wl.H * wl.F / g2 / 1e12 / INT8_PEAK_TOPS, 4)},
        "stage_us": {k: round(v * 1e3, 2) for k, v in m_["stage_ms"].items()},
        "stage_launches_timed": m_["n_stage"],
        "bound": "hbm" if lb / (HBM_PEAK_GBS * 1e9) >= ops / (INT8_PEAK_TOPS * 1e12) else "mfma",
        "roofline_us": {"hbm": round(lb / (HBM_PEAK_GBS * 1e9) * 1e6, 1),
                        "int8": round(ops / (INT8_PEAK_TOPS * 1e12) * 1e6, 1)},
    }
    return blk


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    choices=["tiny", "decode", "prefill", "ep_share", "stress"],
                    help="time this workload only (it becomes the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-router", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the vendor dense INT8 GEMM reference point")
    ap.add_argument("--alpha-sweep", action="store_true",
                    help="only the quantisation-error sweep over alpha and the clip variants")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this layer has no multi-GPU path "
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

    if args.alpha_sweep:
        lwl, layer = make_layer_for("decode")
        gl = GpuLayer(lwl, layer, torch)
        log("alpha sweep")
        print(json.dumps({"alpha_sweep": alpha_sweep(
            gl, layer, 128, [0.5, 0.55, 0.6, 0.65, 0.7], 99.9)}), flush=True)
        return

    head = args.workload or "decode"
    order = [head] if args.workload else ["decode", "prefill", "tiny", "ep_share", "stress"]
    configs, extra = {}, {}
    cpu = {}
    gl = layer = lwl = None
    for name in order:
        wl = synth.workload(name)
        want_lwl = synth.workload("decode") if name == "prefill" else wl
        if lwl is None or lwl.name != want_lwl.name:
            gl = layer = None
            torch.cuda.empty_cache()
            lwl, layer = make_layer_for(name)
            gl = GpuLayer(lwl, layer, torch)
            cal = None
        inputs = synth.make_inputs(wl, layer)
        gl.wl = wl
        log("timing %s: %d warmup + %d flushed steps, %d stamped launches"
            % (name, args.warmup, args.steps, max(20, args.steps)))
        meas = measure(gl, wl, inputs, args.steps, args.warmup, hip)
        configs[name] = config_block(wl, meas)
        if name == "decode" and not args.no_fp8:
            log("FP8 (e4m3) expert path, decode")
            gf = GpuLayer(lwl, layer, torch, fp8=True)
            gf.wl = wl
            fm = measure(gf, wl, inputs, args.steps, args.warmup, hip)
            pwl = synth.workload("prefill")
            pin = synth.make_inputs(pwl, layer)
            gf.wl = pwl
            log("FP8 prefill")
            pm = measure(gf, pwl, pin, max(5, args.steps // 4), 2, hip)
            fd, fpf = config_block(wl, fm), config_block(pwl, pm)
            extra["fp8"] = {
                "decode": {"tokens_per_s": fd["tokens_per_s"],
                           "ms_per_step_median": fd["ms_per_step_median"],
                           "gemm1_hbm_frac": fd["gemm1"]["hbm_frac"], "layer_hbm_frac":
                           fd["hbm"]["frac"], "stage_us": fd["stage_us"]},
                "prefill": {"tokens_per_s": fpf["tokens_per_s"],
                            "ms_per_step_median": fpf["ms_per_step_median"],
                            "gemm1_frac_fp8_peak": fpf["gemm1"]["int8_frac"],
                            "layer_frac_fp8_peak": fpf["int8"]["frac"],
                            "stage_us": fpf["stage_us"]}}
            del gf
            torch.cuda.empty_cache()
        if name == "decode" and not args.no_router:
            log("router-projection mode")
            w_router = synth.make_router(lwl)
            rp = {"decode": time_router(gl, wl, inputs, w_router, args.steps, args.warmup)}
            pwl = synth.workload("prefill")
            rp["prefill"] = time_router(gl, pwl, synth.make_inputs(pwl, layer), w_router,
                                        max(5, args.steps // 4), 2)
            extra["router_projection"] = rp
        if not args.no_cpu_baseline:
            import oracle
            if cal is None:
                cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down,
                                       lwl.alpha)
            log("timing the CPU oracle on a sample of %s" % name)
            cpu[name] = cpu_baseline(wl, cal, inputs)
            configs[name]["oracle_tokens_per_s"] = cpu[name]["value"]
            configs[name]["oracle_sample"] = cpu[name]["sample"]

    h = configs[head]
    wl = synth.workload(head)
    if h["gemm_path"] == "stream":
        g1b = gemm1_bytes(wl, h["touched_experts"])
        g1s = h["gemm1"]["avg_launch_us"] * 1e-6
        achieved = g1b / g1s / 1e9
        traffic = stored_traffic("gemm1_stream", head)
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic["bytes_per_launch"] if traffic else None,
                "kernel": "gemm_stream_kernel<gate/up> (GEMM1)",
                "algorithmic_bytes_per_launch": g1b, "avg_launch_us": h["gemm1"]["avg_launch_us"],
                "launches_timed": h["stage_launches_timed"]}
    else:
        ops = 4 * h["kept_rows"] * wl.H * wl.F
        g1s = h["gemm1"]["avg_launch_us"] * 1e-6
        achieved = ops / g1s / 1e12
        traffic = stored_traffic("gemm1_tiled", head)
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4),
                "traffic": traffic["bytes_per_launch"] if traffic else None,
                "kernel": "gemm_tiled_kernel<gate/up> (GEMM1)",
                "algorithmic_ops_per_launch": ops, "avg_launch_us": h["gemm1"]["avg_launch_us"],
                "launches_timed": h["stage_launches_timed"]}
    res = {
        "metric": METRIC, "value": h["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": h["ms_per_step_median"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.description, "tokens": wl.T, "hidden": wl.H, "experts": wl.E,
                   "top_k": wl.k, "ffn": wl.F, "gemm_path": h["gemm_path"],
                   "timing": "median of per-forward HIP-event times, 512 MiB overwritten "
                             "between forwards"},
        "roofline": roof,
        "configs": configs,
    }
    res.update(extra)
    if not args.workload and not args.no_reference:
        log("vendor dense INT8 GEMM reference (hipBLASLt) on the prefill GEMM shapes")
        res["dense_int8_reference"] = dense_int8_reference(torch)
    res["cpu_baseline"] = None
    if head in cpu:
        res["cpu_baseline"] = dict(cpu[head], **host_info())
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
