"""moe_w8a8_forward_noalloc (the forward whose workspace is the library's
static device scratch) through the C ABI, against moe_w8a8_forward on the same
inputs: two calls in a row, the second with a smaller batch (and, after them,
another layer shape), each output bit-identical to the allocating entry
point's (same kernels, same order of every sum). A batch too large for the
scratch is refused with nothing written."""
import sys

import numpy as np
import pytest

import oracle
import synth
from moe_testlib import bf16_tensor, tensor_bits, upload_weights, layer_of

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


def _layer(wl):
    import w8a8_int8_expert_amd as m
    layer = layer_of(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha)
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    upload_weights(g, cal)
    return g, layer


def _both(torch, g, wl, inputs, T):
    import w8a8_int8_expert_amd as m
    dev = g.device
    x = bf16_tensor(inputs.x[:T], dev)
    lg = torch.from_numpy(np.ascontiguousarray(inputs.logits[:T])).to(dev)
    ref = g.forward(x, router_logits=lg, capacity_factor=wl.capacity_factor)
    out = torch.full((T, wl.H), 7, dtype=torch.int16, device=dev).view(torch.bfloat16)
    rc = m.moe_w8a8_forward_noalloc(g.d, g.weights, x, T, lg, None, None, wl.capacity_factor,
                                    out)
    assert rc == m.MOE_W8A8_OK, m.moe_w8a8_strerror(rc)
    torch.cuda.synchronize()
    return tensor_bits(ref), tensor_bits(out)


def test_noalloc_matches_forward(torch_cuda):
    torch = torch_cuda
    import w8a8_int8_expert_amd as m
    wl = synth.workload("decode")
    _say("[noalloc] decode layer: T=%d then T=5" % wl.T)
    g, layer = _layer(wl)
    inputs = synth.make_inputs(wl, layer)
    for T in (wl.T, 5):
        a, b = _both(torch, g, wl, inputs, T)
        assert np.array_equal(a, b), "T=%d: outputs differ" % T
    # a batch whose workspace exceeds the scratch is refused, out untouched
    big = 512
    assert m.moe_w8a8_workspace_size(g.d, big) > m.MOE_W8A8_SCRATCH_BYTES
    x = torch.zeros(big, wl.H, dtype=torch.bfloat16, device=g.device)
    lg = torch.zeros(big, wl.E, dtype=torch.float32, device=g.device)
    out = torch.full((big, wl.H), 3, dtype=torch.int16, device=g.device)
    rc = m.moe_w8a8_forward_noalloc(g.d, g.weights, x, big, lg, None, None, 0.0, out)
    assert rc == m.MOE_W8A8_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3).all())
    # another layer shape on the same scratch, with capacity drops
    wt = synth.workload("tiny", T=40, capacity_factor=0.75)
    _say("[noalloc] tiny layer with capacity: T=40 then T=7")
    gt, lt = _layer(wt)
    it = synth.make_inputs(wt, lt)
    for T in (40, 7):
        a, b = _both(torch, gt, wt, it, T)
        assert np.array_equal(a, b), "tiny T=%d: outputs differ" % T
