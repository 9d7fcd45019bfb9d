"""End-to-end pin of the oracle: on inputs that every quantiser of the layer
represents exactly, the W8A8 layer must equal the plain dense MoE FFN in fp64,
to the last bit of its fp64 sum and of its bf16 output.

The inputs are built so that no step of the quantised path loses anything:
  - SmoothQuant ("MiniMax-M3 W8A8 inference on K100AI" §3.2, alpha = 0.5):
    per-channel activation and weight ranges are powers of 4, so every s_j is
    an exact power of 2 and smoothing only moves exponents;
  - the per-token and per-output-channel quantisers ("... K100AI" §1.2,
    §3.2): every row's largest magnitude is 127 * 2^p, so 127/amax and the
    scale are exact and the row's codes are its integer values;
  - SwiGLU: every gate value is at least 40, where 1 + exp(-g) rounds to 1
    in fp64 and silu(g) = g exactly;
  - the requantisation of h ("... K100AI" §4.3): the up projection of each
    expert reads the token through one anchor channel that is 127 in every
    token, so h_f = g * 127 * n_f * 2^e with integer n_f and some |n_f| = 127:
    the row maximum is 127 * (g * 127 * 2^e) and the codes are the n_f;
  - every product and sum stays within 24 (fp32) and 53 (fp64) significant
    bits.
The last two channels are zero in every token and carry the 127 of the gate
and up rows, so those rows have their maximum where it does not touch the
sums. The last expert is never routed; it holds each channel's weight range,
which fixes s. The helpers take any size; tests/test_gpu_exact_grid.py builds
the same construction at the GPU kernels' sizes.

The reference uses nothing of the oracle: top-k by (logit descending, index
ascending) with softmax weights renormalised over the chosen experts
("超大规模模型推理的Day0适配实践" §四), the first C = ceil(cf*T*k/E)
assignments of each expert in (token, slot) order (§二.2), and
out[t] = sum_j w[t][j] * W_down[e] (silu(W_gate[e] x_t) * (W_up[e] x_t)) in
fp64 from the unquantised tensors. A wrong scale, a weight on the wrong slot,
a transposed operand, gate and up swapped, a lost capacity drop or a wrong
permutation changes the result. The planted codes (qx, q_gu, q_d, qh) and the
exact scales are checked stage by stage as well.

The FP8 experts ("超大规模模型推理的Day0适配实践" §二.1, §四) are pinned the
same way with 448 in place of 127: every planted value is an integer that
e4m3 represents (at most 4 significant bits), so codes and scales are again
exact and the FP8 layer must equal the same dense FFN. The e4m3 bytes are
decoded here from their bit fields (sign, 4 exponent bits with bias 7, 3
mantissa bits), independently of the oracle's decoder.
"""
import math

import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits
from test_oracle_pins import _bf16_nearest_bruteforce

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

FORMATS = {"int8": (oracle.FMT_INT8, 127), "fp8": (oracle.FMT_FP8, 448)}
# k is a power of 2, so that the weights of k tied experts (1/k) are exact
SHAPES = {"E5_k2": dict(H=8, F=4, E=5, K=2, T=6), "E7_k4": dict(H=16, F=4, E=7, K=4, T=8)}
ALPHA = 0.5


def _pow2(e):
    return float(2.0 ** e)


def _e4m3_byte_value(c):
    """Value of an OCP e4m3 byte from its bit fields (NaN for 0x7f, 0xff)."""
    sign = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    if e == 15 and m == 7:
        return math.nan
    return sign * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


_E4M3 = np.array([_e4m3_byte_value(c) for c in range(256)])


def _code_values(codes, fmt):
    codes = np.asarray(codes)
    if fmt == oracle.FMT_INT8:
        return codes.astype(np.float64)
    return _E4M3[codes.view(np.uint8)]


def _grid(qmax):
    """Signed integers the format represents exactly, up to qmax: all of
    [-127, 127] for INT8; for e4m3 the integers with at most 4 significant
    bits (1..15, then steps of 2 to 30, 4 to 60, 8 to 120, 16 to 240, 32 to
    448)."""
    if qmax == 127:
        return np.arange(-127, 128)
    pos = [v for v in range(1, 449)
           if v < 16 or (v >> (v.bit_length() - 4)) << (v.bit_length() - 4) == v]
    return np.array(sorted([-v for v in pos] + [0] + pos))


def reference_route(logits, k):
    """Top-k with ties to the lower index; softmax renormalised over the k."""
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        ids[t] = order
        ex = np.array([math.exp(float(logits[t, e]) - float(logits[t, order[0]]))
                       for e in order])
        w[t] = ex / ex.sum()
    return ids, w


def reference_keep(ids, cf, E):
    """The first C assignments of each expert in (token, slot) order."""
    T, k = ids.shape
    keep = np.ones((T, k), bool)
    if cf <= 0:
        return keep
    C = math.ceil(cf * T * k / E)
    seen = np.zeros(E, int)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            keep[t, j] = seen[e] < C
            seen[e] += 1
    return keep


def reference_y(x, wg, wu, wd, ids, keep, swap_gate_up=False):
    """Each kept assignment's expert output W_down[e] (silu(W_gate[e] x) *
    (W_up[e] x)) in fp64 on the unquantised tensors: [T][k][H], 0 if dropped.
    On the inputs built here every product and partial sum is a dyadic value
    within 53 bits, so the order of the matrix products' sums is immaterial."""
    T, k = ids.shape
    y = np.zeros((T, k, wd.shape[1]))
    for e in np.unique(ids[keep]):
        t, j = np.nonzero((ids == e) & keep)
        g = x[t] @ wg[e].astype(np.float64).T
        u = x[t] @ wu[e].astype(np.float64).T
        if swap_gate_up:
            g, u = u, g
        y[t, j] = (g / (1.0 + np.exp(-g)) * u) @ wd[e].astype(np.float64).T
    return y


def reference_layer(x, wg, wu, wd, ids, w, keep, swap_slots=False, swap_gate_up=False):
    """Dense MoE FFN in fp64: sum over the kept slots of w * y, slot order."""
    y = reference_y(x, wg, wu, wd, ids, keep, swap_gate_up)
    k = ids.shape[1]
    out = np.zeros((x.shape[0], wd.shape[1]))
    for j in range(k):
        wj = w[:, k - 1 - j] if swap_slots else w[:, j]
        out += wj.astype(np.float64)[:, None] * y[:, j]
    return out


def build(seed, qmax=127, H=8, F=4, E=5, K=2, T=6, down_step=1):
    """One lossless case: tensors, the planted codes and exponents, logits.
    Experts 0..E-2 are routed; expert E-1 only carries the weight ranges.
    Channel 0 is the anchor (qmax in every token); channels H-2 and H-1 are
    zero in every token and hold the qmax of the gate and the up rows.
    down_step: the requantised values n and the down codes are drawn from the
    multiples of down_step on the grid.
    Router projection: channel 1 + e is routed expert e's routing channel
    (s = 1 there); the router matrix reads expert e's logit from it
    (w_router[e] = one-hot at 1 + e; the carrier reads expert 0's channel, so
    it ties expert 0 whenever that one is chosen, and must lose). Each token
    holds one value v on the channels of its K chosen experts and smaller
    ones on the others, so the projected logits d * 2^m are exact and tie at
    the top (weights exactly 1/K)."""
    rng = np.random.default_rng([4242, seed, qmax, H, T, down_step])
    grid = _grid(qmax)
    grid_down = grid[grid % down_step == 0]
    routed, anchor, gate_pad, up_pad = E - 1, 0, H - 2, H - 1
    assert routed + 3 <= H, "no room for a routing channel per expert"
    b = rng.integers(-1, 3, size=H)                 # s_j = 2^b_j
    b[1:1 + routed] = 0
    a = rng.integers(5, 7, size=H) + (qmax > 127)   # weight range aw_j = 4^a_j
    aw = np.array([4.0 ** int(v) for v in a])
    ax = np.array([4.0 ** int(a[j] + b[j]) for j in range(H)])
    calib = np.stack([ax * rng.choice([-1, 1], size=H), ax / 2 * rng.choice([-1, 1], size=H)])
    s = np.array([_pow2(int(v)) for v in b])

    # tokens: codes d on the grid with d[anchor] = qmax, zero padding channels
    m = rng.integers(-1, 2, size=T)
    d = rng.choice(grid, size=(T, H))
    d[:, anchor] = qmax
    d[:, gate_pad] = 0
    d[:, up_pad] = 0
    router_top = np.stack([np.sort(rng.choice(routed, size=K, replace=False)) for _ in range(T)])
    for t in range(T):
        i = int(rng.integers(5, grid.size))
        lower = grid[i - rng.integers(1, 6, size=routed)]
        d[t, 1:1 + routed] = lower
        d[t, 1 + router_top[t]] = grid[i]
    x = (d * np.array([_pow2(int(v)) for v in m])[:, None]) * s[None, :]
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)
    x_bits = f32_to_bf16_bits(x32)
    assert np.array_equal(x_bits.astype(np.uint32) << 16, x32.view(np.uint32)), "x not bf16"

    # routing: K routed experts tied at the top of every token (weights
    # exactly 1/K); the carrier expert sometimes ties too and must lose
    logits = np.zeros((T, E), np.float32)
    for t in range(T):
        top = rng.choice(routed, size=K, replace=False)
        L = np.float32(rng.integers(-8, 9) / 4)
        logits[t] = L - np.float32(1 + rng.integers(0, 4, size=E))
        logits[t, top] = L
        if rng.random() < 0.5:
            logits[t, routed] = L
    pre_ids = np.stack([rng.permutation(routed)[:K] for _ in range(T)]).astype(np.int32)
    pre_w = (rng.integers(1, 9, size=(T, K)) / 8).astype(np.float32)
    # the same with every slot of about a third of the tokens on one expert
    rep_ids = pre_ids.copy()
    rep = rng.choice(T, size=max(1, T // 3), replace=False)
    rep_ids[rep] = rep_ids[rep, :1]
    w_router = np.zeros((E, H), np.float32)
    w_router[np.arange(routed), 1 + np.arange(routed)] = 1.0
    w_router[routed, 1] = 1.0
    router_logits = x @ w_router.astype(np.float64).T
    assert np.array_equal(router_logits[:, :routed], d[:, 1:1 + routed] * 2.0 ** m[:, None])
    r_ids, _ = reference_route(logits, K)
    p_ids, _ = reference_route(router_logits, K)
    assert np.array_equal(p_ids, router_top)
    pairs = {(t, int(e)) for t in range(T) for e in r_ids[t]} | \
            {(t, int(e)) for t in range(T) for e in pre_ids[t]} | \
            {(t, int(e)) for t in range(T) for e in p_ids[t]}

    wg = np.zeros((E, F, H), np.float32)
    wu = np.zeros((E, F, H), np.float32)
    wd = np.zeros((E, H, F), np.float32)
    plan = {}
    for e in range(routed):
        pu, pr = (int(v) for v in rng.integers(-1, 2, size=2))
        # gate anchor code 3 and two live +-1: acc_g >= 3*qmax - 2*qmax = qmax,
        # and with 2^(m + pg) >= 1/2 every gate value is at least qmax/2 >= 40
        pg = int(rng.integers(0, 2))
        cg = np.zeros(H, np.int64)
        cg[anchor] = 3
        live = rng.choice(np.arange(1, gate_pad), size=2, replace=False)
        cg[live] = rng.choice([-1, 1], size=2)
        cg[gate_pad] = qmax
        acc_g = {t: int(d[t] @ cg) for t in range(T) if (t, e) in pairs}
        assert all(v * _pow2(int(m[t]) + pg) >= 40 for t, v in acc_g.items())
        n = rng.choice(grid_down, size=F)
        n[rng.integers(F)] = qmax * rng.choice([-1, 1])
        cu = np.zeros((F, H), np.int64)
        cu[:, anchor] = n
        cu[:, up_pad] = qmax
        cd = rng.choice(grid_down, size=(H, F))
        cd[np.arange(H), rng.integers(0, F, size=H)] = qmax * rng.choice([-1, 1], size=H)
        # smoothed rows are 2^p * codes; the stored weights divide by s
        wg[e] = (_pow2(pg) * cg[None, :] / s[None, :]).astype(np.float32)
        wu[e] = (_pow2(pu) * cu / s[None, :]).astype(np.float32)
        wd[e] = (_pow2(pr) * cd).astype(np.float32)
        plan[e] = dict(pg=pg, pu=pu, pr=pr, cg=cg, n=n, cu=cu, cd=cd, acc_g=acc_g)
    # the never-routed expert attains each channel's weight range
    wg[routed, 0] = (aw * rng.choice([-1, 1], size=H)).astype(np.float32)
    wu[routed] = rng.uniform(-1, 1, size=(F, H)).astype(np.float32)
    wd[routed] = rng.uniform(-1, 1, size=(H, F)).astype(np.float32)
    assert np.array_equal(np.maximum(np.abs(wg).max(axis=(0, 1)), np.abs(wu).max(axis=(0, 1))),
                          aw)
    assert np.array_equal(np.abs(calib).max(axis=0), ax)
    calib_bits = f32_to_bf16_bits(calib.astype(np.float32))
    return dict(H=H, F=F, E=E, K=K, T=T, qmax=qmax, x=x, x_bits=x_bits, d=d, m=m, s=s,
                calib_bits=calib_bits, wg=wg, wu=wu, wd=wd, plan=plan, logits=logits,
                pre_ids=pre_ids, pre_w=pre_w, rep_ids=rep_ids,
                w_router_bits=f32_to_bf16_bits(w_router), router_logits=router_logits)


def static_clip(c):
    """A static activation clip that the construction keeps exact: the level
    qmax * 2^q, q the smallest token exponent, so every token with a larger
    exponent is clipped ("一晚上完成MoE模型推理优化…" §3.2: activations beyond
    the calibrated level are cut off). Smoothed values beyond the level become
    +-level and the others d * 2^(m - q), integers (e4m3 ones for FP8), so the
    codes stay exact; the anchor code stays qmax. Returns the level, the codes
    and exponents the tokens quantise to, and the clipped tokens
    clamp(x * inv_s, +-level) * s that the dense reference takes."""
    qmax = c["qmax"]
    q = int(c["m"].min())
    level = qmax * _pow2(q)
    d = np.clip(c["d"] * 2.0 ** (c["m"] - q)[:, None], -qmax, qmax)
    m = np.full_like(c["m"], q)
    x = np.clip(c["x"] / c["s"][None, :], -level, level) * c["s"][None, :]
    assert np.array_equal(x, d * _pow2(q) * c["s"][None, :])
    return level, d, m, x


# pre_routed: given ids and unequal weights; repeated: given ids naming one
# expert in every slot of some tokens (one row per slot), with capacity;
# clip: logits routing with a static activation clip; router: logits from the
# router projection of the tokens
MODES = ["logits", "capacity", "pre_routed", "repeated", "clip", "router"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("fmt_name", sorted(FORMATS))
def test_lossless_layer_equals_dense_ffn(fmt_name, shape, seed, mode):
    fmt, qmax = FORMATS[fmt_name]
    c = build(seed, qmax, **SHAPES[shape])
    F, E, K = c["F"], c["E"], c["K"]
    cal = oracle.calibrate(c["calib_bits"], c["wg"], c["wu"], c["wd"], ALPHA, fmt=fmt)
    # calibration: exact s, the planted codes and power-of-2 scales
    assert np.array_equal(cal["s"].astype(np.float64), c["s"])
    assert np.array_equal(cal["inv_s"].astype(np.float64), 1.0 / c["s"])
    for e, p in c["plan"].items():
        assert np.array_equal(_code_values(cal["q_gu"][e, :F], fmt), np.tile(p["cg"], (F, 1)))
        assert np.array_equal(_code_values(cal["q_gu"][e, F:], fmt), p["cu"])
        assert np.array_equal(_code_values(cal["q_d"][e], fmt), p["cd"])
        assert np.all(cal["sw_gu"][e, :F] == _pow2(p["pg"]))
        assert np.all(cal["sw_gu"][e, F:] == _pow2(p["pu"]))
        assert np.all(cal["sw_d"][e] == _pow2(p["pr"]))

    cf = 0.75 if mode in ("capacity", "repeated") else 0.0   # C = 2 (E5_k2), 4 (E7_k4)
    level, d, m, x = 0.0, c["d"], c["m"], c["x"]
    if mode == "clip":
        level, d, m, x = static_clip(c)
        assert np.any(c["m"] > m), "no token is clipped"
    if mode in ("pre_routed", "repeated"):
        ids = c["pre_ids"] if mode == "pre_routed" else c["rep_ids"]
        w = c["pre_w"].astype(np.float64)
        o = oracle.forward(c["x_bits"], cal, K, ids=ids, w=c["pre_w"], capacity_factor=cf,
                           fmt=fmt)
    elif mode == "router":
        lg = oracle.router_logits(c["x_bits"], c["w_router_bits"])
        assert np.array_equal(lg, c["router_logits"])
        ids, w = reference_route(c["router_logits"], K)
        o = oracle.forward(c["x_bits"], cal, K, logits=lg.astype(np.float32), fmt=fmt)
        assert np.array_equal(o["ids"], ids) and np.all(w == 1.0 / K) and np.all(ids < E - 1)
    else:
        ids, w = reference_route(c["logits"], K)
        o = oracle.forward(c["x_bits"], cal, K, logits=c["logits"], capacity_factor=cf,
                           clip=level, fmt=fmt)
        assert np.array_equal(o["ids"], ids)
        assert np.array_equal(o["w"].astype(np.float64), w)     # ties: exactly 1/2
        assert np.all(w == 1.0 / K) and np.all(ids < E - 1)
    keep = reference_keep(ids, cf, E)
    assert np.array_equal(o["row_of"] >= 0, keep)
    if mode == "capacity":
        assert not keep.all()

    # token codes and scales are the planted ones
    assert np.array_equal(_code_values(o["qx"], fmt), d)
    assert np.array_equal(o["sx"].astype(np.float64), [_pow2(int(v)) for v in m])
    # every kept row requantises to its expert's n_f, with the exact scale
    for i in range(o["kept"]):
        a = int(o["sorted"][i])
        t, e = a // K, int(o["ids"].reshape(-1)[a])
        p = c["plan"][e]
        assert np.array_equal(_code_values(o["qh"][i], fmt), p["n"])
        expo = 2 * int(m[t]) + p["pg"] + p["pu"]
        assert float(o["sh"][i]) == float(d[t] @ p["cg"]) * qmax * _pow2(expo)

    args = (x, c["wg"], c["wu"], c["wd"], ids, w)
    ref = reference_layer(*args, keep)
    assert np.array_equal(o["out_exact"], ref), np.abs(o["out_exact"] - ref).max()
    want = np.array([[_bf16_nearest_bruteforce(float(v)) for v in row] for row in ref], np.uint16)
    assert np.array_equal(o["out"], want)

    # the pin has power: plausible slips in the layer change the result
    assert not np.array_equal(ref, reference_layer(*args, keep, swap_gate_up=True))
    if mode == "pre_routed":
        assert not np.array_equal(ref, reference_layer(*args, keep, swap_slots=True))
    if mode == "repeated":
        assert np.any(ids[:, 0] == ids[:, 1])
        # where a repeated slot survives the capacity, keeping one row per
        # token and expert instead of one per slot gives another result
        dup = np.zeros_like(keep)
        dup[:, 1:] = ids[:, 1:] == ids[:, :1]
        if (keep & dup).any():
            assert not np.array_equal(ref, reference_layer(*args, keep & ~dup))
    if mode == "capacity":
        assert not np.array_equal(ref, reference_layer(*args, np.ones_like(keep)))
    if mode == "clip":
        assert not np.array_equal(ref, reference_layer(c["x"], *args[1:], keep))
