"""Activation clipping variants through the C ABI against the CPU oracle:
the static threshold of the calibration (bit-exact), and the forward with a
static clip, with dynamic per-token saturation, and with both."""
import sys

import numpy as np
import pytest

import oracle
import synth
from moe_testlib import (bf16_tensor, check_act_quant, check_out, check_requant,
                         check_routing_and_grouping, flip_allowance, layer_of, run_gpu,
                         upload_weights)

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("name", ["decode", "stress", "tiny"])
def test_clip_threshold_parity(torch_cuda, name):
    import torch
    import w8a8_int8_expert_amd as m
    wl = synth.workload(name)
    _say("[clip] threshold case=%s n_calib=%d H=%d" % (name, wl.n_calib, wl.H))
    layer = layer_of(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha)
    dev = torch.device("cuda")
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    upload_weights(g, cal)
    cx = bf16_tensor(layer.calib_x, dev)
    for p in (99.9, 99.0, 100.0, 50.0):
        g.calibrate_clip(cx, p)
        torch.cuda.synchronize()
        got = g.act_clip.cpu().numpy()[0]
        want = oracle.clip_threshold(layer.calib_x, cal["inv_s"], p)
        assert got.view(np.uint32) == want.view(np.uint32), (p, got, want)


CASES = {
    # name: (workload overrides or None for decode, static clip, saturation percentile)
    "tiny_static": (dict(T=40), True, 0.0),
    "tiny_sat": (dict(T=40), False, 99.0),           # H 256: m = 3
    "tiny_both": (dict(T=40), True, 98.0),           # m = 6
    "mid_sat": (dict(T=700, E=8, k=4, H=1024, F=256), False, 99.5),   # large-A path, m = 6
    "decode_both": (None, True, 99.9),               # H 4096: m = 5
}


@pytest.mark.parametrize("gemm_path", [1, 2])
@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_clip_parity(torch_cuda, case, gemm_path):
    import torch
    over, static, sat_p = CASES[case]
    wl = synth.workload("decode") if over is None else synth.workload("tiny", **over)
    _say("[clip] forward case=%s path=%d T=%d H=%d static=%s sat=%g" % (
        case, gemm_path, wl.T, wl.H, static, sat_p))
    clip_full_parity(torch, wl, gemm_path, static, sat_p)


def clip_full_parity(torch, wl, gemm_path, static, sat_p):
    """The layer with the static clip (at the calibration tokens' 99th percentile)
    and/or dynamic saturation at percentile sat_p, every stage against the oracle."""
    import w8a8_int8_expert_amd as m
    layer = layer_of(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha)
    inputs = synth.make_inputs(wl, layer)
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    upload_weights(g, cal)
    clip = 0.0
    if static:
        # a low percentile so that the clip bites on many tokens
        g.calibrate_clip(bf16_tensor(layer.calib_x, torch.device("cuda")), 99.0)
        clip = oracle.clip_threshold(layer.calib_x, cal["inv_s"], 99.0)
    g.set_clip(static=static, sat_percentile=sat_p)
    res = run_gpu(g, inputs, wl.k, wl.capacity_factor, gemm_path)
    o = oracle.forward(inputs.x, cal, wl.k, logits=inputs.logits, ids=inputs.ids, w=inputs.w,
                       capacity_factor=wl.capacity_factor, clip=clip, sat_percentile=sat_p)
    plain_sx = oracle.act_quant(inputs.x, cal["inv_s"])[1]
    assert np.any(o["sx"] < plain_sx), "the clip changes no token"
    check_routing_and_grouping(res, o)
    check_act_quant(res, o["qx"], o["sx"])
    kept = o["kept"]
    if kept:
        acc1 = res["gpu_tensors"]["acc1"].view(-1, 2 * wl.F)[:kept].cpu().numpy()
        assert np.array_equal(acc1, o["acc1"]), "GEMM1 accumulators differ"
        qh = res["gpu_tensors"]["qh"].view(-1, wl.F)[:kept].cpu().numpy()
        sh = res["gpu_tensors"]["sh"][:kept].cpu().numpy()
        check_requant(qh, sh, o["qh"], o["sh"])
    check_out(res["out"], o["out_exact"], allow=flip_allowance(o, cal, wl.k))


def test_saturation_rank_limit(torch_cuda):
    """A percentile whose rank leaves more than 16 values above is refused
    before anything runs."""
    import torch
    import w8a8_int8_expert_amd as m
    wl = synth.workload("tiny")
    _say("[clip] saturation rank limit")
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    g.set_clip(sat_percentile=90.0)   # H 256: m = 26 > 16
    x = torch.zeros(4, wl.H, dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros(4, wl.E, dtype=torch.float32, device="cuda")
    with pytest.raises(m.MoEW8A8Error):
        g.forward(x, router_logits=lg)


def fp8_clip_full_parity(torch, wl, gemm_path, static, sat_p):
    """FP8 experts with the static clip and/or dynamic saturation: activation
    codes and scales bit-exact against the oracle in the FP8 format, every
    later stage to the FP8 bars (test_gpu_fp8.fp8_check)."""
    import w8a8_int8_expert_amd as m
    from test_gpu_fp8 import fp8_check, tiled_path
    dev = torch.device("cuda")
    layer = layer_of(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha,
                           fmt=oracle.FMT_FP8)
    inputs = synth.make_inputs(wl, layer)
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k, fp8=True)
    upload_weights(g, cal)
    clip = 0.0
    if static:
        g.calibrate_clip(bf16_tensor(layer.calib_x, dev), 99.0)
        clip = oracle.clip_threshold(layer.calib_x, cal["inv_s"], 99.0)
    g.set_clip(static=static, sat_percentile=sat_p)
    res = run_gpu(g, inputs, wl.k, wl.capacity_factor, gemm_path)
    o = oracle.forward(inputs.x, cal, wl.k, logits=inputs.logits, ids=inputs.ids, w=inputs.w,
                       capacity_factor=wl.capacity_factor, clip=clip, sat_percentile=sat_p,
                       fmt=oracle.FMT_FP8)
    plain_sx = oracle.act_quant(inputs.x, cal["inv_s"], fmt=oracle.FMT_FP8)[1]
    assert np.any(o["sx"] < plain_sx), "the clip changes no token"
    check_routing_and_grouping(res, o)
    check_act_quant(res, o["qx"], o["sx"])
    kept = o["kept"]
    if kept:
        t = res["gpu_tensors"]
        gpu = dict(acc1=t["acc1"].view(-1, 2 * wl.F)[:kept].cpu().numpy().view(np.float32),
                   h=t["h"].view(-1, wl.F)[:kept].cpu().numpy(),
                   qh=t["qh"].view(-1, wl.F)[:kept].cpu().numpy(),
                   sh=t["sh"][:kept].cpu().numpy(), out=res["out"])
        fp8_check(gpu, o, cal, wl, tiled_path(wl, gemm_path))
