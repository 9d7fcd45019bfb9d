"""FP8 (OCP e4m3) expert path through the C ABI against the CPU oracle.

Codes are decided in fp32 by the same operation sequence on both sides, so
weight codes, scales and activation codes are bit-exact. The GEMMs
accumulate on the FP8 matrix instructions on the GPU and exactly (fp64) in
the oracle. Those instructions do not round each addition to fp32: their
error, measured on MI355X, is ~6e-7 (median) to ~8e-6 (max) of sum
|products|, where fp32 rounding would give ~1e-8. Hence, for FP8 only:
  - GEMM1 sums within 2^-14 * sum |products| (8x above the largest error
    seen, far below one missing 16-byte chunk of products);
  - requantised codes within one e4m3 step plus 2^-4 (in the 448-range code
    space) and differing in at most 1 % of entries (an h within that error of
    one of e4m3's 8-16 rounding midpoints per binade flips a code);
  - requant scales within 1e-3 relative (a row's largest |h| carries the
    sum error times sum |products| / |sum|, ~10-20 at the row maxima, from
    both gate and up);
  - the layer output within 8e-2 * RMS: a flipped code moves h by one e4m3
    step (up to 1/8 of its value), and the measured deviation (3-4.5 % of RMS
    at the largest element) stays below the format's own error against the
    unquantised layer (5-6 % RMS, pinned on the CPU); INT8 keeps 2e-2.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from moe_testlib import (check_act_quant, check_routing_and_grouping, run_gpu, unpack_tiled,
                         upload_weights)

pytestmark = pytest.mark.gpu

LUT = np.array([oracle.e4m3_value(c) for c in range(256)])
ACC_REL = 2.0 ** -14      # GEMM1 sums, relative to sum |products|
QH_FRAC = 1e-2            # requantised codes that may differ
SH_RTOL_FP8 = 1e-3
OUT_RMS_FRAC_FP8 = 8e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_int8_expert_amd as m
    m.load_library()
    return torch


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_fp8_calibrate_parity(torch_cuda, name):
    import torch
    import w8a8_int8_expert_amd as m
    from moe_testlib import bf16_tensor
    wl = synth.workload(name)
    _say("[fp8] calibrate case=%s H=%d F=%d E=%d" % (name, wl.H, wl.F, wl.E))
    layer = synth.make_layer(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha,
                           fmt=oracle.FMT_FP8)
    dev = torch.device("cuda")
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k, fp8=True)
    wg = torch.from_numpy(layer.w_gate).to(dev)
    wu = torch.from_numpy(layer.w_up).to(dev)
    wd = torch.from_numpy(layer.w_down).to(dev)
    g.calibrate(bf16_tensor(layer.calib_x, dev), wg, wu, wd, wl.alpha)
    torch.cuda.synchronize()
    del wg, wu, wd
    assert np.array_equal(g.s_gate_up.cpu().numpy().view(np.uint32), cal["sw_gu"].view(np.uint32))
    assert np.array_equal(g.s_down.cpu().numpy().view(np.uint32), cal["sw_d"].view(np.uint32))
    q_gu = unpack_tiled(g.w_gate_up.cpu().numpy(), wl.E, 2 * wl.F, wl.H)
    assert np.array_equal(q_gu, cal["q_gu"])
    q_d = unpack_tiled(g.w_down.cpu().numpy(), wl.E, wl.H, wl.F)
    assert np.array_equal(q_d, cal["q_d"])


CASES = {
    "tiny": dict(T=40),
    "mid_tiled": dict(T=1000, E=4, k=2, H=512, F=384),
    # partial last N tiles in both GEMMs, 5 N tiles each, capacity drops
    "mid_odd_nt": dict(T=600, E=3, k=1, H=1792, F=896, capacity_factor=0.9),
    "decode": None,
}


@pytest.mark.parametrize("gemm_path", [1, 2])
@pytest.mark.parametrize("case", sorted(CASES))
def test_fp8_forward_parity(torch_cuda, case, gemm_path):
    wl = synth.workload("decode") if CASES[case] is None else synth.workload("tiny", **CASES[case])
    _say("[fp8] forward case=%s path=%d T=%d H=%d F=%d E=%d k=%d" % (
        case, gemm_path, wl.T, wl.H, wl.F, wl.E, wl.k))
    fp8_full_parity(wl, gemm_path)


def fp8_full_parity(wl, gemm_path):
    """Every stage of the FP8 layer on workload wl against the oracle, to the FP8 bars."""
    import w8a8_int8_expert_amd as m
    layer = synth.make_layer(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha,
                           fmt=oracle.FMT_FP8)
    inputs = synth.make_inputs(wl, layer)
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k, fp8=True)
    upload_weights(g, cal)
    res = run_gpu(g, inputs, wl.k, wl.capacity_factor, gemm_path)
    o = oracle.forward(inputs.x, cal, wl.k, logits=inputs.logits, ids=inputs.ids, w=inputs.w,
                       capacity_factor=wl.capacity_factor, fmt=oracle.FMT_FP8)
    check_routing_and_grouping(res, o)
    check_act_quant(res, o["qx"], o["sx"])
    kept = o["kept"]
    if kept == 0:
        return
    # GEMM1: fp32 sums against the exact ones, within the accumulation bound
    acc1 = res["gpu_tensors"]["acc1"].view(-1, 2 * wl.F)[:kept].cpu().numpy().view(np.float32)
    tok = o["sorted"] // wl.k
    exp_id = o["ids"].reshape(-1)[o["sorted"]]
    absx = np.abs(LUT[o["qx"].view(np.uint8)])
    bound = np.empty((kept, 2 * wl.F))
    for e in np.unique(exp_id):
        rows = np.nonzero(exp_id == e)[0]
        absw = np.abs(LUT[cal["q_gu"][e].view(np.uint8)])
        bound[rows] = absx[tok[rows]] @ absw.T
    err = np.abs(acc1.astype(np.float64) - o["acc1"])
    rel = err / np.maximum(bound, 1e-300)
    _say("[fp8] GEMM1 error / sum|products|: median %.3g, 99.9%% %.3g, max %.3g" % (
        np.median(rel), np.quantile(rel, 0.999), rel.max()))
    assert np.all(err <= ACC_REL * bound + 1e-30), "max %.3g of sum|products|" % rel.max()
    # Requantised codes, compared by value in the code space (v * 448/max):
    # at most one e4m3 step at their magnitude plus 2^-4 absolute. The
    # absolute part covers h near zero, where e4m3 steps (2^-9) are finer
    # than the accumulation error that reaches h when the gate or up sum
    # cancels; 2^-4 is 1/7168 of the row's range.
    qh = res["gpu_tensors"]["qh"].view(-1, wl.F)[:kept].cpu().numpy()
    tg, to = LUT[qh.view(np.uint8)], LUT[o["qh"].view(np.uint8)]
    mag = np.maximum(np.abs(tg), np.abs(to))
    step = np.where(mag < 2.0 ** -6, 2.0 ** -9,
                    2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3))
    dist = np.abs(tg - to)
    assert np.all(dist <= step + 2.0 ** -4), "max excess %.4g" % np.max(dist - step)
    frac = np.count_nonzero(dist) / dist.size
    _say("[fp8] requantised codes differing: %.4f %%" % (100 * frac))
    assert frac <= QH_FRAC
    sh = res["gpu_tensors"]["sh"][:kept].cpu().numpy()
    np.testing.assert_allclose(sh, o["sh"], rtol=SH_RTOL_FP8, atol=0)
    from synth import bf16_bits_to_f32
    got = bf16_bits_to_f32(res["out"]).astype(np.float64)
    want = bf16_bits_to_f32(o["out"]).astype(np.float64)
    rms = np.sqrt(np.mean(want ** 2))
    err = np.max(np.abs(got - want))
    _say("[fp8] output max error %.4g of RMS" % (err / rms))
    assert err <= OUT_RMS_FRAC_FP8 * rms


def test_fp8_format_validated(torch_cuda):
    """A format outside {INT8, FP8} is refused before anything runs."""
    import torch
    import w8a8_int8_expert_amd as m
    wl = synth.workload("tiny")
    _say("[fp8] format validation")
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    g.weights.format = 2
    x = torch.zeros(4, wl.H, dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros(4, wl.E, dtype=torch.float32, device="cuda")
    with pytest.raises(m.MoEW8A8Error):
        g.forward(x, router_logits=lg)
