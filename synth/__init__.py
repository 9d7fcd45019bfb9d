"""Seeded synthetic workloads for the W8A8 MoE expert layer.

This module only draws random inputs; it holds none of the layer's arithmetic
(no routing, quantisation, smoothing or GEMM). Both the HIP path and the CPU
oracle are fed from here, and nothing else is shared between them.

The pages' calibration corpora and evaluation sets are not available, so every
input is synthetic with the shapes and value distributions of the workloads the
layer is measured on (see WORKLOADS). Streams are numpy PCG64 generators spawned
from a SeedSequence: a *layer* seed draws the weights, the calibration tokens and
the outlier-channel choice; an *input* seed draws the tokens, the router logits
(or pre-routed assignments) and per-token magnitudes. Every float is drawn as
float32; token tensors are rounded to bfloat16 (ties to even) and carried as
uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens (rows) entering the layer
    H: int                 # hidden size
    E: int                 # experts held by this GPU
    k: int                 # assignments per token
    F: int                 # expert FFN width (SwiGLU gate/up/down)
    alpha: float           # SmoothQuant migration strength
    layer_seed: int
    input_seed: int
    n_calib: int = 512     # calibration tokens
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    lognormal_tokens: bool = False
    logit_step: float = 0.0          # >0: logits rounded to this step (forces ties)
    capacity_factor: float = 0.0     # <=0: no capacity limit
    pre_routed: bool = False         # ids/weights given instead of logits
    zipf_s: float = 0.0              # pre-routed expert popularity exponent
    weight_std: float = 0.02
    description: str = ""


WORKLOADS = {
    "tiny": Workload(
        "tiny", T=16, H=256, E=8, k=2, F=512, alpha=0.6, layer_seed=101, input_seed=102,
        n_calib=64,
        description="Tiny MoE layer: 16 tokens, hidden 256, 8 experts, top-2, FFN 512"),
    "decode": Workload(
        "decode", T=32, H=4096, E=64, k=8, F=1536, alpha=0.6, layer_seed=202, input_seed=203,
        outlier_frac=0.01, outlier_mult=50.0,
        description="27B-class decode step: 32 tokens, hidden 4096, 64 experts, top-8, FFN 1536"),
    "prefill": Workload(
        "prefill", T=16384, H=4096, E=64, k=8, F=1536, alpha=0.6, layer_seed=202, input_seed=303,
        outlier_frac=0.01, outlier_mult=50.0,
        description="Prefill of the decode layer: 16384 tokens (32 x 512), same weights"),
    "ep_share": Workload(
        "ep_share", T=8192, H=8192, E=32, k=1, F=2048, alpha=0.6, layer_seed=404, input_seed=405,
        pre_routed=True, zipf_s=1.1,
        description="One GPU's expert-parallel share: 8192 pre-routed rows, hidden 8192, "
                    "32 local experts of 256, FFN 2048, Zipf(1.1) popularity"),
    "stress": Workload(
        "stress", T=4096, H=4096, E=128, k=8, F=1024, alpha=0.5, layer_seed=505, input_seed=506,
        outlier_frac=0.005, outlier_mult=100.0, lognormal_tokens=True, logit_step=1.0 / 16,
        capacity_factor=1.25,
        description="Outlier/skew stress: 4096 tokens, hidden 4096, 128 experts, top-8, FFN 1024, "
                    "tied logits, capacity 1.25"),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


@dataclass
class Layer:
    """Unquantised layer parameters and calibration tokens (host arrays)."""
    w_gate: np.ndarray        # float32 [E][F][H]
    w_up: np.ndarray          # float32 [E][F][H]
    w_down: np.ndarray        # float32 [E][H][F]
    calib_x: np.ndarray       # uint16 (bf16) [n_calib][H]
    outlier_channels: np.ndarray


@dataclass
class Inputs:
    x: np.ndarray                         # uint16 (bf16) [T][H]
    logits: Optional[np.ndarray] = None   # float32 [T][E]
    ids: Optional[np.ndarray] = None      # int32 [T][k] (pre-routed)
    w: Optional[np.ndarray] = None        # float32 [T][k] (pre-routed)


def _tokens(rng_x, rng_scale, n: int, wl: Workload, channels: np.ndarray) -> np.ndarray:
    x = rng_x.standard_normal((n, wl.H), dtype=np.float32)
    if wl.lognormal_tokens:
        x *= rng_scale.lognormal(0.0, 1.0, size=(n, 1)).astype(np.float32)
    if channels.size:
        x[:, channels] *= np.float32(wl.outlier_mult)
    return f32_to_bf16_bits(x)


def make_layer(wl: Workload) -> Layer:
    r_w, r_cal, r_ch, r_cal_scale = _streams(wl.layer_seed, 4)
    n_out = int(round(wl.outlier_frac * wl.H))
    channels = np.sort(r_ch.choice(wl.H, size=n_out, replace=False)).astype(np.int64) \
        if n_out else np.zeros(0, np.int64)
    std = np.float32(wl.weight_std)
    w_gate = r_w.standard_normal((wl.E, wl.F, wl.H), dtype=np.float32)
    w_gate *= std
    w_up = r_w.standard_normal((wl.E, wl.F, wl.H), dtype=np.float32)
    w_up *= std
    w_down = r_w.standard_normal((wl.E, wl.H, wl.F), dtype=np.float32)
    w_down *= std
    calib = _tokens(r_cal, r_cal_scale, wl.n_calib, wl, channels)
    return Layer(w_gate, w_up, w_down, calib, channels)


def make_router(wl: Workload) -> np.ndarray:
    """bf16 [E][H] router matrix, N(0, 1/H) rounded to bf16, from the fifth
    stream of the layer seed (the first four make the layer)."""
    r = _streams(wl.layer_seed, 5)[4]
    w = r.standard_normal((wl.E, wl.H), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(wl.H))
    return f32_to_bf16_bits(w)


def make_inputs(wl: Workload, layer: Layer, T: Optional[int] = None) -> Inputs:
    T = wl.T if T is None else T
    r_x, r_route, r_scale = _streams(wl.input_seed, 3)
    x = _tokens(r_x, r_scale, T, wl, layer.outlier_channels)
    if not wl.pre_routed:
        logits = r_route.standard_normal((T, wl.E), dtype=np.float32)
        if wl.logit_step > 0:
            step = np.float32(wl.logit_step)
            logits = (np.round(logits / step) * step).astype(np.float32)
        return Inputs(x=x, logits=logits)
    # Pre-routed rows: each row goes to one local expert drawn from a truncated
    # Zipf(s) popularity over the local experts (rank -> expert id by a seeded
    # permutation); its gate weight is one slot of a uniform Dirichlet over the
    # k_global = 8 slots of the sending token, i.e. Beta(1, 7).
    ranks = np.arange(1, wl.E + 1, dtype=np.float64)
    p = ranks ** (-wl.zipf_s) if wl.zipf_s > 0 else np.ones(wl.E)
    p /= p.sum()
    perm = r_route.permutation(wl.E)
    ids = np.empty((T, wl.k), np.int32)
    for j in range(wl.k):
        ids[:, j] = perm[r_route.choice(wl.E, size=T, p=p)]
    w = r_route.beta(1.0, 7.0, size=(T, wl.k)).astype(np.float32)
    return Inputs(x=x, ids=ids, w=w)
