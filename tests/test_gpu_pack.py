"""moe_w8a8_pack through the C ABI: row-major codes in, the fragment-tiled
layout the header defines out, bit for bit (checked against the layout's
definition written out in numpy, pack_tiled). Every parity test loads its
weights through the same entry point (upload_weights)."""
import sys

import numpy as np
import pytest

from moe_testlib import pack_tiled, unpack_tiled

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
