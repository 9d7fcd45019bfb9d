"""Shared helpers of the tests: layout (un)packing, running the HIP path with
every debug output, and the parity comparisons.

Parity bar of the layer:
  - routing ids, grouping (counts, offsets, sorted, row_of), activation codes
    and scales, and the GEMM1 int32 accumulators: bit-exact;
  - routing weights: |diff| <= 1e-6;
  - requantised hidden codes: |diff| <= 1 everywhere and diff != 0 in at most
    0.1 % of entries; their scales: relative diff <= 1e-5;
  - layer output (bf16), element by element against the oracle's exact fp64
    sum before its rounding: |gpu - exact| <= 2e-2 * RMS(exact) + half a bf16
    step at |gpu|. The half step is the GPU's own final rounding to bf16, the
    one part of the difference that no implementation can avoid; everything
    else (requantisation flips, fp32 sums) must fit in 2e-2 * RMS. How many
    elements needed the half step, and the largest error over RMS without it,
    are reported.
"""
from __future__ import annotations

import functools

import numpy as np

QH_MISMATCH_FRAC = 1e-3
SH_RTOL = 1e-5
W_ATOL = 1e-6
OUT_RMS_FRAC = 2e-2


@functools.lru_cache(maxsize=2)
def layer_of(wl):
    """synth.make_layer(wl), kept for the next test that draws the same seeded
    layer (the full-size layers take ~15 s to draw). Callers only read it."""
    import synth
    return synth.make_layer(wl)


def pack_tiled(w: np.ndarray) -> np.ndarray:
    """[E][N][K] int8 row-major -> fragment-tiled bytes, the layout as the
    header defines it (the reference the library's moe_w8a8_pack is checked
    against)."""
    E, N, K = w.shape
    t = w.reshape(E, N // 16, 16, K // 64, 4, 16).transpose(0, 1, 3, 4, 2, 5)
    return np.ascontiguousarray(t).reshape(-1)


def unpack_tiled(b: np.ndarray, E: int, N: int, K: int) -> np.ndarray:
    """Fragment-tiled bytes -> [E][N][K] int8 row-major."""
    t = b.reshape(E, N // 16, K // 64, 4, 16, 16).transpose(0, 1, 4, 2, 3, 5)
    return np.ascontiguousarray(t).reshape(E, N, K)


def upload_weights(layer_gpu, cal):
    """Load oracle-calibrated weights (row-major codes) into a MoEW8A8 through
    the library's own packing (moe_w8a8_pack)."""
    import torch
    dev = layer_gpu.device
    t = {k: torch.from_numpy(np.ascontiguousarray(cal[k])).to(dev)
         for k in ("q_gu", "sw_gu", "q_d", "sw_d", "s", "inv_s")}
    layer_gpu.load_quantized(t["q_gu"], t["sw_gu"], t["q_d"], t["sw_d"], t["s"], t["inv_s"])
    torch.cuda.synchronize()


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


class OutCheck:
    """Output bar over one or more chunks of tokens: |gpu - exact| <=
    2e-2 * RMS(exact over every chunk) + half a bf16 step at |gpu|."""

    def __init__(self):
        self.sumsq = 0.0
        self.n = 0
        self.diff = []     # |gpu - exact| per element, by chunk
        self.half = []     # half a bf16 step at |gpu|

    def add(self, out_g_bits, exact):
        from synth import bf16_bits_to_f32
        g = bf16_bits_to_f32(out_g_bits).astype(np.float64).ravel()
        x = np.asarray(exact, np.float64).ravel()
        assert g.shape == x.shape
        self.sumsq += float(np.sum(x * x))
        self.n += x.size
        self.diff.append(np.abs(g - x))
        self.half.append(0.5 * bf16_step(g))

    def finish(self, label="", allow=None):
        """allow (one chunk only): a function of flat element indices giving
        the largest output change that requantised codes which may flip can
        cause there (flip_allowance); it is added for elements over the bar."""
        rms = np.sqrt(self.sumsq / self.n) if self.n else 0.0
        diff = np.concatenate(self.diff) if self.diff else np.zeros(0)
        half = np.concatenate(self.half) if self.half else np.zeros(0)
        bar = OUT_RMS_FRAC * rms
        excess = diff - (bar + half + 1e-30)
        n_flip = 0
        if allow is not None:
            over = np.nonzero(excess > 0)[0]
            if over.size:
                excess[over] -= allow(over)
                n_flip = int(over.size)
        worst = float(np.max(excess, initial=-1.0))
        err = float(np.max(diff, initial=0.0))
        n_step = int(np.count_nonzero(diff > bar))
        rel = err / rms if rms else 0.0
        past = float(np.max(diff - half, initial=0.0)) / rms if rms else 0.0
        print("[out] %s %d elements: max |gpu - exact| = %.4g x RMS, %.4g x RMS beyond half a "
              "bf16 step at |gpu| (bar %.3g x RMS); %d elements past 2e-2 x RMS, within half a "
              "bf16 step; %d within the effect of codes that may flip"
              % (label, diff.size, rel, past, OUT_RMS_FRAC, n_step, n_flip), flush=True)
        assert worst <= 0, ("output over the bar by %.4g (max err %.4g, 2e-2 x rms %.4g)"
                            % (worst, err, bar))
        return rel


def check_out(out_g_bits, exact, label="", allow=None):
    """The output bar on one batch: exact is the oracle's fp64 sum (out_exact)."""
    c = OutCheck()
    c.add(out_g_bits, exact)
    return c.finish(label, allow)


def may_flip(o, cal, k, r):
    """Mask over the F requantised codes of kept row r of an INT8 oracle
    forward o (with acc1 and h): the codes that an fp32 SwiGLU may round
    differently from the oracle.

    The GPU's h differs from the oracle's fl32 of the fp64 value by at most
    2^-20 + |g| * 2^-21 relative (g the gate pre-activation: the exponential's
    argument carries its relative rounding into exp), and its row maximum by
    the largest such bound. The code-space value c = fl32(h * fl32(127 /
    max|h|)) then moves by at most |c| * (eps_h + eps_max + 2^-22) + 2^-24, and
    a code can flip only where c lies that close to a rounding midpoint."""
    F = cal["q_d"].shape[2]
    a = int(o["sorted"][r])
    t, e = a // k, int(o["ids"].reshape(-1)[a])
    g = o["acc1"][r, :F].astype(np.float64) * float(o["sx"][t]) * \
        cal["sw_gu"][e, :F].astype(np.float64)
    eps_h = 2.0 ** -20 + np.abs(g) * 2.0 ** -21
    h = o["h"][r].astype(np.float32)
    amax = np.float32(np.max(np.abs(h)))
    if amax == 0:
        return np.zeros(F, bool)
    rr = np.float32(127.0) / amax
    c = np.abs((h * rr).astype(np.float32).astype(np.float64))
    dc = c * (eps_h + eps_h.max() + 2.0 ** -22) + 2.0 ** -24
    return np.abs(c - np.floor(c) - 0.5) <= dc


def flip_allowance(o, cal, k):
    """For an INT8 oracle forward o (with acc1 and h): a function of flat
    output indices t*H + n giving the sum over the token's kept slots of |w|
    times the largest change of y[row][n] that the row's codes which may flip
    (may_flip) can cause, sh * sw_d[e][n] * sum over those codes of
    |q_d[e][n][f]|, plus the scale's tolerance SH_RTOL * |y[row][n]|."""
    H = cal["q_d"].shape[1]
    ids = o["ids"].reshape(-1)
    cache = {}

    def row_effect(r):
        if r in cache:
            return cache[r]
        e = int(ids[int(o["sorted"][r])])
        may = may_flip(o, cal, k, r)
        qd = np.abs(cal["q_d"][e][:, may].astype(np.float64)).sum(axis=1)
        eff = float(o["sh"][r]) * cal["sw_d"][e].astype(np.float64) * qd
        eff = eff + SH_RTOL * np.abs(o["y"][r])
        cache[r] = eff
        return eff

    def allow(flat):
        out = np.zeros(flat.size)
        for i, f in enumerate(flat):
            t, n = divmod(int(f), H)
            for j in range(k):
                r = int(o["row_of"][t, j])
                if r >= 0:
                    out[i] += abs(float(o["w"][t, j])) * row_effect(r)[n]
        return out

    return allow
