"""CPU check of the FP8 parity bounds (fp8_bounds in test_gpu_fp8): a pipeline
whose GEMM sums carry errors anywhere inside the accumulation bound, and
whose other steps round in fp32 as the kernels do, stays inside every bound
derived from the oracle's quantities. Each GEMM sum is moved by a seeded
uniform draw over the whole allowance (far more than the hardware's measured
error), the SwiGLU and the dequantisations run in fp32, the requantisation is
the oracle's own quantiser on the perturbed rows, y is rounded to int16 codes
with one scale per 16 columns as the tiled path holds it (or kept in fp32 as
the streaming path does), and the combine sums in fp32 in slot order before
its rounding to bf16."""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import bf16_step
from synth import bf16_bits_to_f32, f32_to_bf16_bits
from test_gpu_fp8 import LUT, acc_bound, fp8_bounds

def _y16(y):
    """y rows rounded as the tiled path holds them (signed normalised int16
    codes of v / group max, one scale per 16 columns)."""
    g = np.abs(y).reshape(y.shape[0], -1, 16).max(-1, keepdims=True)
    inv = np.where(g > 1e-30, np.float32(1) / np.maximum(g, np.float32(1e-30)), 0)
    q = np.clip(np.rint(y.reshape(g.shape[0], -1, 16) * inv.astype(np.float32) * 32767),
                -32767, 32767)
    sc = np.where(g > 1e-30, g / np.float32(32767), 0).astype(np.float32)
    return (q.astype(np.float32) * sc).astype(np.float32).reshape(y.shape)


CASES = {
    "tiny": dict(T=40),
    "outliers": dict(T=33, outlier_frac=0.02, outlier_mult=50.0, lognormal_tokens=True),
    "ties_capacity": dict(T=60, E=5, k=3, logit_step=0.5, capacity_factor=0.8),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("seed,y16", [(0, True), (1, False)])
def test_fp8_bounds_hold_for_perturbed_pipeline(case, seed, y16):
    wl = synth.workload("tiny", **CASES[case])
    layer = synth.make_layer(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha,
                           fmt=oracle.FMT_FP8)
    inputs = synth.make_inputs(wl, layer)
    o = oracle.forward(inputs.x, cal, wl.k, logits=inputs.logits,
                       capacity_factor=wl.capacity_factor, fmt=oracle.FMT_FP8)
    b = fp8_bounds(o, cal, wl, y16)
    rng = np.random.default_rng(seed)
    F, H, k = wl.F, wl.H, wl.k
    acc = (o["acc1"] + rng.uniform(-1, 1, o["acc1"].shape) * b["acc_tol"]).astype(np.float32)
    tok = o["sorted"] // k
    e_id = o["ids"].reshape(-1)[o["sorted"]]
    sx = o["sx"][tok].astype(np.float32)
    sw = cal["sw_gu"][e_id]
    g = (acc[:, :F] * sx[:, None]).astype(np.float32) * sw[:, :F]
    u = (acc[:, F:] * sx[:, None]).astype(np.float32) * sw[:, F:]
    h = (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float32)
    assert np.all(np.abs(h.astype(np.float64) - o["h"]) <= b["h_tol"])
    qh, sh = oracle.quant_rows_fmt(h, oracle.FMT_FP8)
    d = np.abs(LUT[qh.view(np.uint8)] - LUT[o["qh"].view(np.uint8)])
    assert np.count_nonzero(d) > 0, "the draw should flip some codes"
    assert np.all(d <= b["code_gap"])
    sh_o = o["sh"].astype(np.float64)
    assert np.all(np.abs(sh - sh_o) <= b["sh_rtol"] * sh_o)
    y = np.empty((o["kept"], H), np.float32)
    qv = LUT[qh.view(np.uint8)]
    for e in np.unique(e_id):
        rows = np.nonzero(e_id == e)[0]
        wd = LUT[cal["q_d"][e].view(np.uint8)]
        s2 = qv[rows] @ wd.T
        s2 += rng.uniform(-1, 1, s2.shape) * acc_bound(qv[rows], wd)
        y[rows] = (s2.astype(np.float32) * sh[rows, None]).astype(np.float32) * \
            cal["sw_d"][e][None, :]
    # y rows as the tiled path holds them: int16 codes, one scale per 16 columns
    if y16:
        y = _y16(y)
    out = np.zeros((wl.T, H), np.float32)
    for j in range(k):
        r = o["row_of"][:, j]
        keep = r >= 0
        out[keep] += o["w"][keep, j][:, None] * y[r[keep]]
    got = bf16_bits_to_f32(f32_to_bf16_bits(out)).astype(np.float64)
    lim = b["out_tol"] + 0.5 * bf16_step(got)
    assert np.all(np.abs(got - o["out_exact"]) <= lim)


def test_fp8_bound_catches_a_wrong_code():
    """A code moved by two e4m3 steps where the oracle's value sits far from a
    midpoint is outside the code bound."""
    wl = synth.workload("tiny", T=40)
    layer = synth.make_layer(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha,
                           fmt=oracle.FMT_FP8)
    inputs = synth.make_inputs(wl, layer)
    o = oracle.forward(inputs.x, cal, wl.k, logits=inputs.logits, fmt=oracle.FMT_FP8)
    b = fp8_bounds(o, cal, wl)
    safe = np.argwhere(b["code_gap"] == 0)
    assert safe.size
    i, f = safe[0]
    c = int(o["qh"][i, f].view(np.uint8))
    moved = LUT[(c + 2) & 0x7F | (c & 0x80)]
    assert abs(moved - LUT[c]) > b["code_gap"][i, f]
