"""The GPU path on inputs that every quantiser represents exactly: the
construction of tests/test_oracle_exact_layer.py at the kernels' sizes
(hidden 256, FFN 128, 8 routed experts and one that only carries the weight
ranges, top-2; hidden 512, FFN 256, 64 routed experts, top-8), with the layer
calibrated on the GPU from the unquantised weights ("MiniMax-M3 W8A8
inference on K100AI" §3.2).

On these inputs nothing in the quantised path may round, so the checks are
exact where the path is integer and tight where it is not:
  - smoothing factors, weight codes and weight scales equal the planted ones;
  - token codes and scales, the GEMM1 INT32 sums, the requantised codes (not
    one may flip) and their scales equal the planted values;
  - each dequantised expert row y differs from the exact fp64 row by at most
    the GPU's fp32 roundings, 2^-22 |y|, plus on the tiled path y's int16
    step: half the 16-column group's largest |y| / 32767, plus 2^-20 of it;
  - the output differs from the dense fp64 MoE FFN by at most those errors
    weighted by |w|, the fp32 combine (2^-22 of sum |w y|) and half a bf16
    step at the output.
A fifth mode adds a static activation clip that the construction keeps
exact (static_clip in the CPU test): the reference then takes the clipped
tokens. A sixth routes by the router projection on the GPU ("超大规模模型推理
的Day0适配实践" §四): the router matrix reads each expert's logit from a
channel of its own, so the projected logits are exact and must equal the
planted ones, with the chosen experts tied.
The reference is the dense FFN of the CPU test, with routing (ties to the
lower index, "超大规模模型推理的Day0适配实践" §四) and capacity (§二.2) by
their definitions; it takes nothing from the oracle or the GPU.

The FP8 layer (same page, §二.1) runs the same checks with 448 in place of
127. Its matrix instructions align the products of each 8 consecutive k to
the group's largest and keep 13 bits below that one's leading bit (the
behaviour tests/test_gpu_fp8_accumulation.py measures). Every product in
the GEMMs here is an integer, so nothing is cut where the largest product is
below 2^14: the gate and up sums. For the down projection the requantised
values and the down codes are multiples of 4, so every product is a multiple
of 16 = 2^(17 - 13) and none loses a bit either. The GEMM sums are then
exact for FP8 too, and the checks are the same.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from moe_testlib import bf16_step, bf16_tensor, run_gpu, unpack_tiled
from test_oracle_exact_layer import (ALPHA, _code_values, build, reference_keep,
                                     reference_route, reference_y, static_clip)

pytestmark = pytest.mark.gpu

SHAPES = {"E9_k2": dict(H=256, F=128, E=9, K=2),
          "E65_k8": dict(H=512, F=256, E=65, K=8),
          # the decode layer: hidden 4096, FFN 1536, 64 routed experts, top-8
          "decode": dict(H=4096, F=1536, E=65, K=8)}
Y_GROUP = 16
Y_CODE_MAX = 32767


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_int8_expert_amd as m
    m.load_library()
    return torch


FORMATS = {"int8": (oracle.FMT_INT8, 127, 1), "fp8": (oracle.FMT_FP8, 448, 4)}


@functools.lru_cache(maxsize=1)
def _case(T, fmt_name, shape):
    _, qmax, step = FORMATS[fmt_name]
    if fmt_name == "fp8" and SHAPES[shape]["F"] > 256:
        # FFN 1536: GEMM2 partial sums reach 2^28, so every product is made a
        # multiple of 256 (values multiples of 16) to keep them within fp32
        step = 16
    return build(7, qmax, T=T, down_step=step, **SHAPES[shape])


@functools.lru_cache(maxsize=1)
def _gpu_layer(T, fmt_name, shape):
    """The case's layer, calibrated on the GPU, after checking that the
    calibration reproduces the planted smoothing, codes and scales."""
    import torch
    import w8a8_int8_expert_amd as m
    fmt = FORMATS[fmt_name][0]
    c = _case(T, fmt_name, shape)
    H, F, E, K = c["H"], c["F"], c["E"], c["K"]
    dev = torch.device("cuda")
    g = m.MoEW8A8(H, F, E, K, fp8=fmt == oracle.FMT_FP8)
    g.calibrate(bf16_tensor(c["calib_bits"], dev), torch.from_numpy(c["wg"]).to(dev),
                torch.from_numpy(c["wu"]).to(dev), torch.from_numpy(c["wd"]).to(dev), ALPHA)
    torch.cuda.synchronize()
    assert np.array_equal(g.smooth.cpu().numpy().astype(np.float64), c["s"])
    assert np.array_equal(g.inv_smooth.cpu().numpy().astype(np.float64), 1.0 / c["s"])
    q_gu = unpack_tiled(g.w_gate_up.cpu().numpy(), E, 2 * F, H)
    q_d = unpack_tiled(g.w_down.cpu().numpy(), E, H, F)
    s_gu, s_d = g.s_gate_up.cpu().numpy(), g.s_down.cpu().numpy()
    for e, p in c["plan"].items():
        assert np.array_equal(_code_values(q_gu[e, :F], fmt), np.tile(p["cg"], (F, 1)))
        assert np.array_equal(_code_values(q_gu[e, F:], fmt), p["cu"])
        assert np.array_equal(_code_values(q_d[e], fmt), p["cd"])
        assert np.all(s_gu[e, :F] == 2.0 ** p["pg"]) and np.all(s_gu[e, F:] == 2.0 ** p["pu"])
        assert np.all(s_d[e] == 2.0 ** p["pr"])
    return g


def _y_error_bound(y, tiled):
    """Per-element bound on |y_gpu - y| for exact rows y [n][H]."""
    b = 2.0 ** -22 * np.abs(y)
    if tiled:
        G = np.abs(y).reshape(y.shape[0], -1, Y_GROUP).max(axis=2)
        b = b + np.repeat(G, Y_GROUP, axis=1) * (0.5 / Y_CODE_MAX + 2.0 ** -20)
    return b


@pytest.mark.parametrize("gemm_path", [1, 2])
@pytest.mark.parametrize("mode", ["logits", "capacity", "pre_routed", "repeated", "clip",
                                  "router"])
@pytest.mark.parametrize("shape,T", [("E9_k2", 40), ("E9_k2", 3000), ("E65_k8", 200),
                                     ("E65_k8", 3000), ("decode", 32)])
@pytest.mark.parametrize("fmt_name", ["int8", "fp8"])
def test_exact_grid_layer(torch_cuda, fmt_name, shape, T, mode, gemm_path):
    fmt, qmax, _ = FORMATS[fmt_name]
    c = _case(T, fmt_name, shape)
    H, F, E, K = c["H"], c["F"], c["E"], c["K"]
    _say("[exact grid] %s T=%d H=%d F=%d E=%d k=%d mode=%s path=%d"
         % (fmt_name, T, H, F, E, K, mode, gemm_path))
    g = _gpu_layer(T, fmt_name, shape)
    cf = 0.75 if mode in ("capacity", "repeated") else 0.0
    level, d, m, x = 0.0, c["d"], c["m"], c["x"]
    if mode == "clip":     # a static activation clip the construction keeps exact
        level, d, m, x = static_clip(c)
    if mode in ("pre_routed", "repeated"):
        # repeated: every slot of about a third of the tokens names one expert
        ids = c["pre_ids"] if mode == "pre_routed" else c["rep_ids"]
        w = c["pre_w"].astype(np.float64)
        inputs = synth.Inputs(x=c["x_bits"], ids=ids, w=c["pre_w"])
    elif mode == "router":  # logits projected on the GPU from x and the router matrix
        ids, w = reference_route(c["router_logits"], K)
        inputs = synth.Inputs(x=c["x_bits"])
    else:
        ids, w = reference_route(c["logits"], K)
        inputs = synth.Inputs(x=c["x_bits"], logits=c["logits"])
    g.act_clip.fill_(level)
    g.set_clip(static=mode == "clip")
    if mode == "router":
        g.set_router(bf16_tensor(c["w_router_bits"], g.device))
    try:
        r = run_gpu(g, inputs, K, cf, gemm_path, project=mode == "router")
    finally:
        g.set_clip(static=False)
        g.set_router(None)
    if mode == "router":
        assert np.array_equal(r["router_logits"].astype(np.float64), c["router_logits"])
    if mode in ("logits", "capacity", "clip", "router"):
        assert np.array_equal(r["ids"], ids) and np.all(r["w"] == 1.0 / K)
    keep = reference_keep(ids, cf, E)
    assert np.array_equal(r["row_of"] >= 0, keep)
    if mode == "capacity":
        assert not keep.all()
    assert np.array_equal(_code_values(r["qx"], fmt), d)
    assert np.array_equal(r["sx"].astype(np.float64), 2.0 ** m)

    kept = r["kept"]
    a = r["sorted"].astype(np.int64)
    t_of, j_of = a // K, a % K
    acc1 = r["gpu_tensors"]["acc1"].view(-1, 2 * F)[:kept].cpu().numpy()
    if fmt == oracle.FMT_FP8:      # the fp32 sums, held as their bits
        acc1 = acc1.view(np.float32).astype(np.float64)
    qh = r["gpu_tensors"]["qh"].view(-1, F)[:kept].cpu().numpy()
    sh = r["gpu_tensors"]["sh"][:kept].cpu().numpy()
    y_gpu = r["gpu_tensors"]["y"].view(-1, H)[:kept].cpu().numpy().astype(np.float64)
    # the planted values of every kept row, gathered by its token and expert
    e_of = ids[t_of, j_of]
    plan = c["plan"]
    cg = np.stack([plan[e]["cg"] for e in range(E - 1)])
    n = np.stack([plan[e]["n"] for e in range(E - 1)])
    pgu = np.array([plan[e]["pg"] + plan[e]["pu"] for e in range(E - 1)])
    acc_g = np.einsum("rh,rh->r", d[t_of], cg[e_of])
    assert np.all(acc1[:, :F] == acc_g[:, None]), "GEMM1 gate sums differ"
    assert np.array_equal(acc1[:, F:], qmax * n[e_of]), "GEMM1 up sums differ"
    moved = np.nonzero(np.any(_code_values(qh, fmt) != n[e_of], axis=1))[0]
    assert moved.size == 0, "rows %s: a requantised code moved" % moved[:5]
    expo = 2 * m[t_of] + pgu[e_of]
    assert np.array_equal(sh.astype(np.float64), acc_g * qmax * 2.0 ** expo)

    y = reference_y(x, c["wg"], c["wu"], c["wd"], ids, keep)       # [T][K][H]
    tiled = gemm_path == 2
    y_rows = y[t_of, j_of]
    y_err = np.abs(y_gpu - y_rows)
    y_bound = _y_error_bound(y_rows, tiled)
    y_ratio = (y_err / np.maximum(y_bound, 1e-300)).max()
    assert np.all(y_err <= y_bound), "y: %g of its bound" % y_ratio

    ref = np.einsum("tk,tkh->th", w * keep, y)
    out = synth.bf16_bits_to_f32(r["out"]).reshape(T, H).astype(np.float64)
    absw = np.abs(w * keep)
    bound = np.zeros((T, H))
    for j in range(K):
        y_j = y[:, j]
        bound += absw[:, j, None] * (_y_error_bound(y_j, tiled) + 2.0 ** -22 * np.abs(y_j))
    bound += 0.5 * bf16_step(out)
    err = np.abs(out - ref)
    _say("[exact grid] y: max error %.3g of its bound; out: max error %.3g of its bound, "
         "%.3g x RMS" % (y_ratio, (err / np.maximum(bound, 1e-300)).max(),
                          err.max() / np.sqrt(np.mean(ref ** 2))))
    assert np.all(err <= bound)
