"""moe_w8a8_pack through the C ABI: row-major codes in, the fragment-tiled
layout the header defines out, bit for bit (checked against the layout's
definition written out in numpy, pack_tiled). Every parity test loads its
weights through the same entry point (upload_weights)."""
import sys

import numpy as np
import pytest

from moe_testlib import layer_of, pack_tiled, unpack_tiled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_int8_expert_amd as m
    m.load_library()
    return torch


@pytest.mark.parametrize("count,N,K", [(1, 16, 64), (3, 48, 192), (2, 4096, 1536),
                                       (5, 272, 4160), (1, 16, 65536)])
def test_pack_matches_layout(torch_cuda, count, N, K):
    torch = torch_cuda
    import w8a8_int8_expert_amd as m
    print("[pack] count=%d N=%d K=%d" % (count, N, K), flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(count * 100003 + N * 7 + K)
    src = rng.integers(-128, 128, size=(count, N, K), dtype=np.int8)
    s = torch.from_numpy(src).cuda()
    d = torch.full((count * N * K,), 0x55, dtype=torch.int8, device="cuda")
    assert m.moe_w8a8_pack(count, N, K, s, d) == m.MOE_W8A8_OK
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    assert np.array_equal(got, pack_tiled(src))
    assert np.array_equal(unpack_tiled(got, count, N, K), src)


def test_stale_hip_error_not_reported(torch_cuda):
    """An error that another HIP user in the process left pending (here a
    hipSetDevice to a device that does not exist, which changes nothing else)
    is not reported as the failure of the library's next launch: the pack and
    a whole forward after it still succeed and give their results."""
    import ctypes
    torch = torch_cuda
    import synth
    import w8a8_int8_expert_amd as m
    hip = ctypes.CDLL("libamdhip64.so")
    dev = torch.device("cuda")
    src = torch.randint(-127, 128, (2, 32, 128), dtype=torch.int8, device=dev)
    dst = torch.empty(2 * 32 * 128, dtype=torch.int8, device=dev)
    torch.cuda.synchronize()
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    assert m.moe_w8a8_pack(2, 32, 128, src, dst) == m.MOE_W8A8_OK
    torch.cuda.synchronize()
    want = pack_tiled(src.cpu().numpy())
    assert np.array_equal(dst.cpu().numpy(), want)
    # a forward of the tiny layer after another pending error
    wl = synth.workload("tiny")
    layer = layer_of(wl)
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    g.calibrate(torch.from_numpy(layer.calib_x.view("int16")).to(dev).view(torch.bfloat16),
                torch.from_numpy(layer.w_gate).to(dev), torch.from_numpy(layer.w_up).to(dev),
                torch.from_numpy(layer.w_down).to(dev), wl.alpha)
    inputs = synth.make_inputs(wl, layer)
    x = torch.from_numpy(inputs.x.view("int16")).to(dev).view(torch.bfloat16)
    lg = torch.from_numpy(inputs.logits).to(dev)
    ref = g.forward(x, lg).clone()
    torch.cuda.synchronize()
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    out = g.forward(x, lg)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
