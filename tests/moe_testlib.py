"""Shared helpers of the tests: layout (un)packing, running the HIP path with
every debug output, and the parity comparisons.

Parity bar (what the benchmark spec of the layer fixes):
  - routing ids, grouping (counts, offsets, sorted, row_of), activation codes
    and scales, and the GEMM1 int32 accumulators: bit-exact;
  - routing weights: |diff| <= 1e-6;
  - requantised hidden codes: |diff| <= 1 everywhere and diff != 0 in at most
    0.1 % of entries; their scales: relative diff <= 1e-5;
  - layer output (bf16): |diff| <= 2e-2 * RMS(oracle output) element by element, plus
    one bf16 step at the element's magnitude. Both sides round the final sum to bf16,
    the kernels from fp32 and the oracle from fp64, so an element whose exact value
    lies within that difference of a rounding midpoint rounds one step apart; that
    step (up to 2^-7 of the value) exceeds 2e-2 * RMS wherever the output is more
    than 2.56x its RMS.
"""
from __future__ import annotations

import numpy as np

QH_MISMATCH_FRAC = 1e-3
SH_RTOL = 1e-5
W_ATOL = 1e-6
OUT_RMS_FRAC = 2e-2


def pack_tiled(w: np.ndarray) -> np.ndarray:
    """[E][N][K] int8 row-major -> fragment-tiled bytes (the ABI's layout)."""
    E, N, K = w.shape
    t = w.reshape(E, N // 16, 16, K // 64, 4, 16).transpose(0, 1, 3, 4, 2, 5)
    return np.ascontiguousarray(t).reshape(-1)


def unpack_tiled(b: np.ndarray, E: int, N: int, K: int) -> np.ndarray:
    """Fragment-tiled bytes -> [E][N][K] int8 row-major."""
    t = b.reshape(E, N // 16, K // 64, 4, 16, 16).transpose(0, 1, 4, 2, 3, 5)
    return np.ascontiguousarray(t).reshape(E, N, K)


def upload_weights(layer_gpu, cal):
    """Copy oracle-calibrated weights (row-major) into a MoEW8A8's buffers."""
    import torch
    dev = layer_gpu.device
    layer_gpu.w_gate_up.copy_(torch.from_numpy(pack_tiled(cal["q_gu"])).to(dev))
    layer_gpu.w_down.copy_(torch.from_numpy(pack_tiled(cal["q_d"])).to(dev))
    layer_gpu.s_gate_up.copy_(torch.from_numpy(cal["sw_gu"]).to(dev))
    layer_gpu.s_down.copy_(torch.from_numpy(cal["sw_d"]).to(dev))
    layer_gpu.smooth.copy_(torch.from_numpy(cal["s"]).to(dev))
    layer_gpu.inv_smooth.copy_(torch.from_numpy(cal["inv_s"]).to(dev))


def bf16_tensor(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def tensor_bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_gpu(layer_gpu, inputs, k, capacity_factor=0.0, gemm_path=0, project=False):
    """Run moe_w8a8_forward with every debug buffer; returns host arrays.
    project=True routes by the layer's router matrix (set_router) instead of
    the inputs' logits; the logits it used come back as "router_logits"."""
    import torch
    import w8a8_int8_expert_amd as m
    dev = layer_gpu.device
    T = inputs.x.shape[0]
    H, F, E = layer_gpu.d.hidden, layer_gpu.d.ffn, layer_gpu.d.num_experts
    A = max(T * k, 1)
    x = bf16_tensor(inputs.x, dev)
    logits = torch.from_numpy(inputs.logits).to(dev) \
        if inputs.logits is not None and not project else None
    ids = torch.from_numpy(inputs.ids).to(dev) if inputs.ids is not None else None
    w = torch.from_numpy(inputs.w).to(dev) if inputs.w is not None else None
    dbgt = dict(
        topk_ids=torch.empty(A, dtype=torch.int32, device=dev),
        topk_w=torch.empty(A, dtype=torch.float32, device=dev),
        expert_counts=torch.empty(E, dtype=torch.int32, device=dev),
        expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        sorted_assign=torch.empty(A, dtype=torch.int32, device=dev),
        row_of=torch.empty(A, dtype=torch.int32, device=dev),
        qx=torch.empty(max(T, 1) * H, dtype=torch.int8, device=dev),
        sx=torch.empty(max(T, 1), dtype=torch.float32, device=dev),
        acc1=torch.empty(A * 2 * F, dtype=torch.int32, device=dev),
        h=torch.empty(A * F, dtype=torch.float32, device=dev),
        qh=torch.empty(A * F, dtype=torch.int8, device=dev),
        sh=torch.empty(A, dtype=torch.float32, device=dev),
        y=torch.empty(A * H, dtype=torch.float32, device=dev),
        router_logits=torch.empty(max(T, 1) * E, dtype=torch.float32, device=dev))
    dbg = m.moe_w8a8_debug()
    for name, t in dbgt.items():
        setattr(dbg, name, t.data_ptr())
    dbg.gemm_path = gemm_path
    out = layer_gpu.forward(x, router_logits=logits, topk_ids=ids, topk_w=w,
                            capacity_factor=capacity_factor, debug=dbg)
    torch.cuda.synchronize()
    res = dict(out=tensor_bits(out), gpu_tensors=dbgt)
    offs = dbgt["expert_offsets"].cpu().numpy()
    kept = int(offs[-1])
    res.update(
        ids=dbgt["topk_ids"].cpu().numpy()[: T * k].reshape(T, k),
        w=dbgt["topk_w"].cpu().numpy()[: T * k].reshape(T, k),
        counts=dbgt["expert_counts"].cpu().numpy(), offsets=offs, kept=kept,
        sorted=dbgt["sorted_assign"].cpu().numpy()[:kept],
        row_of=dbgt["row_of"].cpu().numpy()[: T * k].reshape(T, k),
        qx=dbgt["qx"].cpu().numpy()[: T * H].reshape(T, H), sx=dbgt["sx"].cpu().numpy()[:T],
        router_logits=dbgt["router_logits"].cpu().numpy()[: T * E].reshape(T, E))
    return res


def rows_of(res, rows, name, width):
    """Fetch permuted rows `rows` of a [A][width] debug tensor from the GPU."""
    import torch
    t = res["gpu_tensors"][name].view(-1, width)
    idx = torch.as_tensor(np.asarray(rows, np.int64), device=t.device)
    return t.index_select(0, idx).cpu().numpy()


def check_routing_and_grouping(g, o):
    assert np.array_equal(g["ids"], o["ids"]), "routing ids differ"
    assert np.max(np.abs(g["w"].astype(np.float64) - o["w"]), initial=0.0) <= W_ATOL
    assert np.array_equal(g["counts"], o["counts"])
    assert np.array_equal(g["offsets"], o["offsets"])
    assert np.array_equal(g["sorted"], o["sorted"])
    assert np.array_equal(g["row_of"], o["row_of"])


def check_act_quant(g, qx, sx):
    assert np.array_equal(g["qx"], qx), "activation codes differ"
    assert np.array_equal(g["sx"].view(np.uint32), sx.view(np.uint32)), "activation scales differ"


def check_requant(qh_g, sh_g, qh_o, sh_o):
    d = qh_g.astype(np.int32) - qh_o.astype(np.int32)
    assert np.abs(d).max(initial=0) <= 1, "requant codes differ by more than 1"
    frac = np.count_nonzero(d) / max(d.size, 1)
    assert frac <= QH_MISMATCH_FRAC, "requant mismatch fraction %.3g" % frac
    np.testing.assert_allclose(sh_g, sh_o, rtol=SH_RTOL, atol=0)
    return frac


def bf16_step(v: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |v| (8 significant bits); 0 for v = 0."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 0.0)


def check_out(out_g_bits, out_o_bits):
    from synth import bf16_bits_to_f32
    g = bf16_bits_to_f32(out_g_bits).astype(np.float64)
    o = bf16_bits_to_f32(out_o_bits).astype(np.float64)
    rms = np.sqrt(np.mean(o ** 2)) if o.size else 0.0
    diff = np.abs(g - o)
    lim = OUT_RMS_FRAC * rms + bf16_step(np.maximum(np.abs(g), np.abs(o))) + 1e-30
    worst = np.max(diff - lim, initial=-1.0)
    err = np.max(diff, initial=0.0)
    assert worst <= 0, "output err %.4g over the bar (max err %.4g, 2e-2 x rms %.4g)" % (
        worst, err, OUT_RMS_FRAC * rms)
    return err / rms if rms else 0.0
