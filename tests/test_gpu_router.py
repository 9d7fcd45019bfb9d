"""Router projection (logits = x . W_r^T, bf16 inputs, fp32 accumulation)
through the C ABI against the CPU oracle.

The logits are compared with the oracle's fp64 dot products within the
fp32 accumulation bound: |gpu - exact| <= H * 2^-24 * sum_j |x_j w_j| (each of
at most H additions rounds once; the bf16 products are exact). The routing
decision is taken in the kernel's precision: the oracle routes from the
logits the GPU used, and its ids must then match bit for bit; against the
exact logits the chosen experts may differ only where the k-th and (k+1)-th
exact logits are closer than twice the bound.
"""
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


def _bound(x_bits, w_bits):
    xf = synth.bf16_bits_to_f32(x_bits).astype(np.float64)
    wf = synth.bf16_bits_to_f32(w_bits).astype(np.float64)
    H = xf.shape[1]
    return H * 2.0 ** -24 * (np.abs(xf) @ np.abs(wf).T)


def _gpu_logits(torch, wl, x_bits, w_bits):
    import w8a8_int8_expert_amd as m
    dev = torch.device("cuda")
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    g.set_router(bf16_tensor(w_bits, dev))
    out = g.router_logits(bf16_tensor(x_bits, dev))
    torch.cuda.synchronize()
    return out.cpu().numpy()


ROUTER_CASES = {
    "tiny": dict(),                                   # H 256: one part
    "E5_T33": dict(E=5, k=3, T=33, H=512),            # ragged token and expert tiles
    "E256": dict(E=256, k=8, H=768, F=128, T=130),    # 2 parts, the last one short
    "decode": None,                                   # H 4096: 8 parts
}


@pytest.mark.parametrize("case", sorted(ROUTER_CASES))
def test_router_logits_parity(torch_cuda, case):
    wl = synth.workload("decode") if ROUTER_CASES[case] is None else \
        synth.workload("tiny", **ROUTER_CASES[case])
    _say("[router] logits case=%s T=%d H=%d E=%d" % (case, wl.T, wl.H, wl.E))
    layer = layer_of(wl)
    x = synth.make_inputs(wl, layer).x
    w = synth.make_router(wl)
    got = _gpu_logits(torch_cuda, wl, x, w)
    exact = oracle.router_logits(x, w)
    err = np.abs(got.astype(np.float64) - exact)
    assert np.all(err <= _bound(x, w)), "max excess %.3g" % np.max(err - _bound(x, w))


def test_router_logits_independent_of_batch(torch_cuda):
    """A token's logits do not depend on the batch it comes in."""
    wl = synth.workload("decode", T=1000)
    _say("[router] batch independence T=1000 vs 1 and 37")
    layer = layer_of(synth.workload("decode"))
    x = synth.make_inputs(wl, layer).x
    w = synth.make_router(wl)
    full = _gpu_logits(torch_cuda, wl, x, w)
    one = _gpu_logits(torch_cuda, wl, x[5:6], w)
    part = _gpu_logits(torch_cuda, wl, x[100:137], w)
    assert np.array_equal(full[5:6].view(np.uint32), one.view(np.uint32))
    assert np.array_equal(full[100:137].view(np.uint32), part.view(np.uint32))


def _near_tie_ok(ids_gpu, exact, bound, k):
    """GPU ids vs the top-k of the exact logits: equal, or the k-th and
    (k+1)-th exact logits are closer than twice the bound."""
    T, E = exact.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -exact), axis=1)
    want = order[:, :k]
    bad = np.any(np.sort(want, axis=1) != np.sort(ids_gpu, axis=1), axis=1)
    if k < E:
        rows = np.arange(T)
        gap = exact[rows, order[:, k - 1]] - exact[rows, order[:, k]]
        slack = 2.0 * np.maximum(bound[rows, order[:, k - 1]], bound[rows, order[:, k]])
        bad &= gap > slack
    return not np.any(bad)


FORWARD_CASES = {
    "tiny": dict(),                                          # fused small-batch routing
    "mid_route_hist": dict(T=1000, E=8, k=4, H=1024, F=256),  # block routing, 2 parts
    "decode": None,
    # the largest hidden size (128 partial-sum planes of 512 channels)
    "max_hidden": dict(H=65536, F=128, E=8, k=2, T=300),
    # 1024 experts (sixteen per router lane), top-32, block routing
    "E1024_k32": dict(E=1024, k=32, H=1024, F=128, T=700),
}


@pytest.mark.parametrize("gemm_path", [1, 2])
@pytest.mark.parametrize("case", sorted(FORWARD_CASES))
def test_forward_router_mode_parity(torch_cuda, case, gemm_path):
    import torch
    wl = synth.workload("decode") if FORWARD_CASES[case] is None else \
        synth.workload("tiny", **FORWARD_CASES[case])
    _say("[router] forward case=%s path=%d T=%d H=%d E=%d k=%d" % (case, gemm_path, wl.T, wl.H,
                                                                   wl.E, wl.k))
    router_full_parity(torch, wl, gemm_path)


def router_full_parity(torch, wl, gemm_path):
    """The layer routed by its router projection: logits within the fp32 bound of the
    exact ones, the routing decision bit-exact on the GPU's logits, every later stage
    against the oracle routed from them."""
    import w8a8_int8_expert_amd as m
    layer = layer_of(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha)
    inputs = synth.make_inputs(wl, layer)
    w = synth.make_router(wl)
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    upload_weights(g, cal)
    g.set_router(bf16_tensor(w, torch.device("cuda")))
    res = run_gpu(g, inputs, wl.k, wl.capacity_factor, gemm_path, project=True)
    lg = res["router_logits"]
    # the forward's logits are the entry point's logits, bit for bit
    alone = g.router_logits(bf16_tensor(inputs.x, torch.device("cuda"))).cpu().numpy()
    assert np.array_equal(lg.view(np.uint32), alone.view(np.uint32))
    exact = oracle.router_logits(inputs.x, w)
    bound = _bound(inputs.x, w)
    assert np.all(np.abs(lg.astype(np.float64) - exact) <= bound)
    assert _near_tie_ok(res["ids"], exact, bound, wl.k)
    # the rest of the layer against the oracle routed from the GPU's logits
    o = oracle.forward(inputs.x, cal, wl.k, logits=lg, capacity_factor=wl.capacity_factor)
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
