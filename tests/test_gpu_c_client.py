"""The library used from C alone (tests/c_client.c: hipMalloc'd buffers, a
stream of its own, moe_w8a8_calibrate then moe_w8a8_forward), with no Python
or torch in that process: it compiles as C99 against the header and the HIP
runtime (CPU), and on the GPU its output equals, bit for bit, the same layer
calibrated and run through the Python binding, and meets the output bar
against the oracle."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synth
from moe_testlib import check_out, flip_allowance, layer_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    import w8a8_int8_expert_amd as m
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("no gcc or ROCm headers")
    libdir = os.path.dirname(m.LIB_PATH)
    exe = tmp_path / "c_client"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "c_client.c"),
                    "-L", libdir, "-lmoe_w8a8", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + libdir, "-Wl,-rpath," + os.path.join(ROCM, "lib"),
                    "-o", str(exe)], check=True, timeout=120)
    return exe


def test_c_client_builds(tmp_path):
    assert os.path.exists(_build(tmp_path))


@pytest.mark.gpu
@pytest.mark.parametrize("over", [dict(T=16), dict(T=100, E=64, k=8, H=512, F=256)],
                         ids=["tiny", "E64_k8"])
def test_c_client_matches_binding(tmp_path, over):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_int8_expert_amd as m
    exe = _build(tmp_path)
    wl = synth.workload("tiny", **over)
    print("[c client] %s" % over, flush=True)
    sys.stdout.flush()
    layer = layer_of(wl)
    inputs = synth.make_inputs(wl, layer)
    d = tmp_path / "io"
    d.mkdir()
    for name, a in (("calib_x", layer.calib_x), ("w_gate", layer.w_gate), ("w_up", layer.w_up),
                    ("w_down", layer.w_down), ("x", inputs.x), ("logits", inputs.logits)):
        np.ascontiguousarray(a).tofile(str(d / (name + ".bin")))
    r = subprocess.run([str(exe), str(d), str(wl.H), str(wl.F), str(wl.E), str(wl.k), str(wl.T),
                        str(layer.calib_x.shape[0]), repr(float(wl.alpha))],
                       capture_output=True, text=True, timeout=300)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0
    c_out = np.fromfile(str(d / "out.bin"), dtype=np.uint16).reshape(wl.T, wl.H)
    # the same layer through the binding (torch's memory and stream)
    dev = torch.device("cuda")
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    g.calibrate(torch.from_numpy(layer.calib_x.view("int16")).to(dev).view(torch.bfloat16),
                torch.from_numpy(layer.w_gate).to(dev), torch.from_numpy(layer.w_up).to(dev),
                torch.from_numpy(layer.w_down).to(dev), wl.alpha)
    x = torch.from_numpy(inputs.x.view("int16")).to(dev).view(torch.bfloat16)
    out = g.forward(x, torch.from_numpy(inputs.logits).to(dev))
    torch.cuda.synchronize()
    py_out = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(c_out, py_out), "C client and binding outputs differ"
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha)
    o = oracle.forward(inputs.x, cal, wl.k, logits=inputs.logits)
    check_out(c_out, o["out_exact"], "c client", allow=flip_allowance(o, cal, wl.k))
