"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a
hand-derived fixture, a closed form, an invariant, brute force, or an
independent fp64 evaluation of the unquantised layer. They are chosen so that a
plausible slip in the oracle (a swapped exponent, a transposed operand, the
wrong tie rule, truncation instead of rounding, a dropped term) fails at least
one of them. No GPU is needed.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from synth import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _f(v):
    return float(v) if not isinstance(v, str) else float(v)


# --------------------------------------------------------------- bfloat16

def _bf16_nearest_bruteforce(v: float) -> int:
    """Nearest bfloat16 to v by exact rational comparison of the two
    bracketing candidates (ties to the even bit pattern)."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    f32 = np.float32(v)  # any bracketing start; walk to the true neighbours
    b = int(np.array([f32], np.float32).view(np.uint32)[0] >> 16)
    exact = Fraction(v)
    def val(bits):
        return Fraction(float(np.array([bits << 16], np.uint32).view(np.float32)[0]))
    # candidates: b-1, b, b+1 within the same sign half
    cands = [c for c in (b - 1, b, b + 1, b + 2) if (c & 0x8000) == (b & 0x8000) and (c & 0x7F80) != 0x7F80]
    best = min(cands, key=lambda c: (abs(val(c) - exact), c & 1))
    return best


def test_bf16_rounding_bruteforce():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    # exact midpoints between adjacent bfloat16 values (ties must go to even)
    for bits in rng.integers(0x0080, 0x7F00, 400):
        lo = Fraction(float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0]))
        hi = Fraction(float(np.array([(int(bits) + 1) << 16], np.uint32).view(np.float32)[0]))
        vals.append(float((lo + hi) / 2))
        vals.append(-float((lo + hi) / 2))
    vals += [1e-40, -3e-42, 2.0 ** -133, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9]
    for v in vals:
        assert oracle.f64_to_bf16(v) == _bf16_nearest_bruteforce(v), v
    assert oracle.f64_to_bf16(-0.0) == 0x8000
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80        # tie -> even (1.0)
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82    # tie -> even (1+2^-6)
    assert oracle.f64_to_bf16(1e39) == 0x7F80


# ---------------------------------------------------------------- quantiser

def test_quant_golden_rne(golden_dir):
    g = _load(golden_dir, "quant_rne.json")
    v = np.array([r["v"] for r in g["rows"]], np.float32)
    q, s = oracle.quant_rows(v)
    for i, r in enumerate(g["rows"]):
        assert q[i].tolist() == r["q"]
        assert s[i] == np.float32(r["scale"])


@pytest.mark.parametrize("dist", ["normal", "outlier", "lognormal", "tiny"])
def test_quant_roundtrip_bound(dist):
    """Round trip |v - q*scale| <= scale*(0.5 + 1e-4); codes in [-127,127];
    the largest magnitude maps to +-127. The 1e-4 slack covers the fp32
    rounding of the reciprocal, the scale and the product."""
    rng = np.random.default_rng({"normal": 1, "outlier": 2, "lognormal": 3, "tiny": 4}[dist])
    v = rng.standard_normal((64, 1536)).astype(np.float32)
    if dist == "outlier":
        v[:, rng.choice(1536, 15, replace=False)] *= 100
    elif dist == "lognormal":
        v *= rng.lognormal(0, 1, (64, 1)).astype(np.float32)
    elif dist == "tiny":
        v *= np.float32(1e-30)
    q, s = oracle.quant_rows(v)
    assert q.min() >= -127 and q.max() <= 127
    err = np.abs(v.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-4))
    amax = np.abs(v).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(127)).astype(np.float32))
    imax = np.abs(v).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(64), imax]) == 127)
    # rounding is to nearest: every code is within 0.5 of v/scale (up to fp32 slack)
    ratio = v.astype(np.float64) / s[:, None].astype(np.float64)
    assert np.all(np.abs(ratio - q) <= 0.5 + 1e-4)


def test_quant_zero_row():
    q, s = oracle.quant_rows(np.zeros((2, 64), np.float32))
    assert not q.any() and not s.any()


# ------------------------------------------------------------------ routing

def test_routing_golden_ties(golden_dir):
    g = _load(golden_dir, "routing_ties.json")
    for c in g["cases"]:
        lg = np.array([[_f(v) for v in c["logits"]]], np.float32)
        ids, w = oracle.route(lg, c["k"])
        assert ids[0].tolist() == c["ids"], c
        if c["w"] is not None:
            np.testing.assert_allclose(w[0], np.array(c["w"]), rtol=0, atol=1e-7)


def _route_bruteforce(lg, k):
    T, E = lg.shape
    ids = np.empty((T, k), np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))
        ids[t] = order[:k]
    return ids


@pytest.mark.parametrize("E,k,step", [(8, 2, 0.0), (64, 8, 0.0), (128, 8, 1 / 16), (33, 5, 0.5), (256, 8, 0.0)])
def test_routing_bruteforce_and_invariants(E, k, step):
    rng = np.random.default_rng(E * 100 + k)
    lg = rng.standard_normal((300, E)).astype(np.float32)
    if step:
        lg = (np.round(lg / step) * step).astype(np.float32)   # ties and -0.0
    ids, w = oracle.route(lg, k)
    assert np.array_equal(ids, _route_bruteforce(lg, k))
    # k distinct experts per token, weights renormalise to 1
    assert all(len(set(r)) == k for r in ids.tolist())
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23)
    # weights equal the full softmax restricted to the chosen experts, renormalised
    p = np.exp(lg.astype(np.float64) - lg.astype(np.float64).max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    sel = np.take_along_axis(p, ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=0, atol=1e-7)
    # non-increasing weights in slot order
    assert np.all(np.diff(w.astype(np.float64), axis=1) <= 0)


def test_routing_all_equal():
    for E, k in [(8, 2), (64, 8), (128, 8)]:
        lg = np.full((5, E), 0.25, np.float32)
        ids, w = oracle.route(lg, k)
        assert np.array_equal(ids, np.tile(np.arange(k), (5, 1)))
        assert np.all(w == np.float32(1.0 / k))


# ------------------------------------------------------------------ permute

# ------------------------------------------------------- router projection

def test_router_logits_bruteforce():
    """fp64 dot products against Python's exact rational sum of the bf16
    products (a transposed operand or a dropped term fails)."""
    rng = np.random.default_rng(11)
    T, E, H = 3, 5, 24
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = f32_to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.1))
    xf, wf = bf16_bits_to_f32(x), bf16_bits_to_f32(w)
    got = oracle.router_logits(x, w)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(xf[t, j])) * Fraction(float(wf[e, j])) for j in range(H))
            assert abs(got[t, e] - float(exact)) <= 1e-15 * max(1.0, abs(float(exact)))


def test_router_logits_one_hot_and_sign():
    """x = unit vector j selects column j of the router matrix exactly; the
    map is odd in x."""
    rng = np.random.default_rng(12)
    E, H = 7, 64
    w = f32_to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32))
    eye = f32_to_bf16_bits(np.eye(H, dtype=np.float32))
    got = oracle.router_logits(eye, w)
    assert np.array_equal(got, bf16_bits_to_f32(w).T.astype(np.float64))
    x = f32_to_bf16_bits(rng.standard_normal((4, H), dtype=np.float32))
    neg = f32_to_bf16_bits(-bf16_bits_to_f32(x))
    assert np.array_equal(oracle.router_logits(neg, w), -oracle.router_logits(x, w))


def test_router_logits_integer_closed_form():
    """Small integers are exact in bf16 and fp64: x[t][j] = t + 1, w[e][j] =
    (j % 5) - e gives logits (t + 1) * sum_j ((j % 5) - e)."""
    T, E, H = 4, 3, 40
    xf = np.repeat(np.arange(1, T + 1, dtype=np.float32)[:, None], H, axis=1)
    wf = np.array([[(j % 5) - e for j in range(H)] for e in range(E)], np.float32)
    got = oracle.router_logits(f32_to_bf16_bits(xf), f32_to_bf16_bits(wf))
    want = np.array([[(t + 1) * sum((j % 5) - e for j in range(H)) for e in range(E)]
                     for t in range(T)], np.float64)
    assert np.array_equal(got, want)


# ------------------------------------------------------- activation clips

def test_percentile_rank_closed_forms():
    """Nearest rank ceil(p/100 * N), clamped to [1, N]."""
    assert oracle.percentile_rank(75.0, 1000) == 750
    # p is taken as its float32 value: 99.9f = 99.900001526 > 99.9, so the
    # rank among 1000 values is ceil(999.0000153) = 1000
    assert oracle.percentile_rank(99.9, 1000) == 1000
    assert oracle.percentile_rank(100.0, 4096) == 4096
    assert oracle.percentile_rank(50.0, 4) == 2
    assert oracle.percentile_rank(1e-6, 5) == 1
    # 99.9 as float32 is 99.90000152...: 0.999000015 * 4096 = 4091.90 -> 4092
    assert oracle.percentile_rank(99.9, 4096) == 4092


def test_clip_threshold_bruteforce():
    """The static threshold is the ranked value of the sorted |x * inv_s|."""
    rng = np.random.default_rng(21)
    n, H = 37, 64
    x = f32_to_bf16_bits(rng.standard_normal((n, H), dtype=np.float32) * np.float32(3.0))
    inv_s = rng.uniform(0.2, 2.0, H).astype(np.float32)
    a = np.sort(np.abs(bf16_bits_to_f32(x) * inv_s).ravel())
    for p in (99.9, 99.0, 90.0, 50.0, 100.0, 0.01):
        r = math.ceil(np.float64(np.float32(p)) / 100.0 * a.size)
        want = a[min(max(r, 1), a.size) - 1]
        assert oracle.clip_threshold(x, inv_s, p) == want
    assert oracle.clip_threshold(x, inv_s, 100.0) == a[-1]
    assert oracle.clip_threshold(x[:0], inv_s, 99.9) == 0.0


def _levels_quant(v, level):
    """Quantiser of the pages at a given level, in float32 arithmetic."""
    rr = np.float32(127.0) / np.float32(level)
    q = np.clip(np.rint((v * rr).astype(np.float32)), -127, 127).astype(np.int8)
    return q, np.float32(level) / np.float32(127.0)


def test_dynamic_saturation_hand_row():
    """A row 1..256 (inv_s = 1) plus three outliers: at p with m = 4 the level
    is the 4th largest |v|; the three outliers saturate at +-127."""
    H = 256
    vals = np.arange(1, H + 1, dtype=np.float32)
    vals[[10, 20, 30]] = [5000.0, -4000.0, 3000.0]
    x = f32_to_bf16_bits(vals[None, :])
    v = bf16_bits_to_f32(x)[0]
    inv_s = np.ones(H, np.float32)
    p = 98.5                         # ceil(0.985 * 256) = 253 -> m = 256 - 253 + 1 = 4
    assert oracle.percentile_rank(p, H) == 253
    level = np.sort(np.abs(v))[-4]
    assert level == 256.0
    qx, sx = oracle.act_quant(x, inv_s, sat_percentile=p)
    q, sc = _levels_quant(v, level)
    assert np.array_equal(qx[0], q) and sx[0] == sc
    assert qx[0, 10] == 127 and qx[0, 20] == -127 and qx[0, 30] == 127
    # p = 100 keeps the plain per-token maximum
    q0, s0 = oracle.act_quant(x, inv_s)
    q1, s1 = oracle.act_quant(x, inv_s, sat_percentile=100.0)
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


def test_static_clip_level_and_off_values():
    """Static clip: level = min(max |v|, c); c above the maximum or <= 0 leaves
    the plain quantiser; values past c saturate."""
    rng = np.random.default_rng(22)
    T, H = 9, 256
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    inv_s = rng.uniform(0.5, 1.5, H).astype(np.float32)
    v = bf16_bits_to_f32(x) * inv_s
    amax = np.abs(v).max(axis=1)
    c = np.float32(np.median(amax))
    qx, sx = oracle.act_quant(x, inv_s, clip=c)
    for t in range(T):
        q, sc = _levels_quant(v[t], min(amax[t], c))
        assert np.array_equal(qx[t], q) and sx[t] == sc
    q0, s0 = oracle.act_quant(x, inv_s)
    for off in (np.float32(1e9), np.float32(-1.0)):
        q1, s1 = oracle.act_quant(x, inv_s, clip=off)
        assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


# --------------------------------------------------------------- FP8 e4m3

def _e4m3_table():
    """Values of the 256 e4m3 codes from the bit fields, as exact Fractions
    (None for the two NaN codes)."""
    tab = []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            tab.append(None)
            continue
        v = Fraction(m, 8) * Fraction(1, 2 ** 6) if e == 0 else \
            (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))
        tab.append(-v if s else v)
    return tab


def test_e4m3_decode_table():
    tab = _e4m3_table()
    for c in range(256):
        got = oracle.e4m3_value(c)
        if tab[c] is None:
            assert math.isnan(got)
        else:
            assert got == float(tab[c]), hex(c)
            if c == 0x80:
                assert math.copysign(1.0, got) < 0
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6 and oracle.e4m3_value(0x38) == 1.0


def _e4m3_nearest(t: float) -> int:
    """Brute force: the finite code nearest to t (ties to the even code),
    with t's sign bit."""
    tab = _e4m3_table()
    a = abs(Fraction(t))
    best, bd = 0, None
    for c in range(0x7F):
        d = abs(tab[c] - a)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best | (0x80 if math.copysign(1.0, t) < 0 else 0)


def test_e4m3_encode_bruteforce():
    """Every code value, every midpoint (ties to even) and its fp32
    neighbours, signed zeros and random values in [-448, 448]."""
    tab = _e4m3_table()
    vals = [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 1e-30, -1e-30]
    for c in range(0x7F):
        vals.append(float(tab[c]))
        if c < 0x7E:
            mid = np.float32((tab[c] + tab[c + 1]) / 2)
            vals += [float(mid), float(np.nextafter(mid, np.float32(0))),
                     float(np.nextafter(mid, np.float32(1e9))), -float(mid)]
    rng = np.random.default_rng(31)
    vals += [float(v) for v in rng.uniform(-448, 448, 3000).astype(np.float32)]
    vals += [float(v) for v in (rng.standard_normal(500) * 1e-2).astype(np.float32)]
    for t in vals:
        assert oracle.e4m3_code(t) == _e4m3_nearest(float(np.float32(t))), t


def test_fp8_quantiser_roundtrip_and_max():
    """Row maximum codes to +-448; each value lands within half an e4m3
    step of v * 448 / max (fp32 rounding slack aside); zero row: scale 0."""
    rng = np.random.default_rng(32)
    v = (rng.standard_normal((20, 300)) * rng.lognormal(0, 2, (20, 1))).astype(np.float32)
    q, sc = oracle.quant_rows_fmt(v, oracle.FMT_FP8)
    for r in range(v.shape[0]):
        amax = np.max(np.abs(v[r]))
        assert sc[r] == np.float32(amax / np.float32(448.0))
        i = int(np.argmax(np.abs(v[r])))
        assert int(q[r].view(np.uint8)[i]) in (0x7E, 0xFE)
        rr = np.float32(448.0) / np.float32(amax)
        t = np.clip((v[r] * rr).astype(np.float32), -448, 448).astype(np.float64)
        dec = np.array([oracle.e4m3_value(c) for c in q[r]])
        step = np.where(np.abs(t) < 2.0 ** -6, 2.0 ** -9,
                        2.0 ** (np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** -6))) - 3))
        assert np.all(np.abs(t - dec) <= step / 2 * (1 + 1e-6))
    q0, s0 = oracle.quant_rows_fmt(np.zeros((1, 8), np.float32), oracle.FMT_FP8)
    assert s0[0] == 0.0 and np.all(q0 == 0)


def test_fp8_expert_row_exact_sums():
    """FP8 GEMM sums equal the fp64 dot products of the decoded codes, and
    GEMM2's y recovers them through sh and the weight scale."""
    rng = np.random.default_rng(33)
    H, F, E, T, k = 128, 64, 2, 5, 1
    lut = np.array([oracle.e4m3_value(c) for c in range(256)])
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    cal = dict(q_gu=rng.choice(finite, (E, 2 * F, H)).astype(np.uint8).view(np.int8),
               sw_gu=rng.uniform(1e-3, 1e-2, (E, 2 * F)).astype(np.float32),
               q_d=rng.choice(finite, (E, H, F)).astype(np.uint8).view(np.int8),
               sw_d=rng.uniform(1e-3, 1e-2, (E, H)).astype(np.float32))
    qx = rng.choice(finite, (T, H)).astype(np.uint8).view(np.int8)
    sx = rng.uniform(1e-3, 1e-2, T).astype(np.float32)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    sorted_ = np.arange(T, dtype=np.int32)
    r = oracle.expert_rows(np.arange(T, dtype=np.int32), ids, sorted_, qx, sx, cal,
                           fmt=oracle.FMT_FP8)
    for t in range(T):
        e = ids[t, 0]
        want = lut[cal["q_gu"][e].view(np.uint8)] @ lut[qx[t].view(np.uint8)]
        np.testing.assert_allclose(r["acc1"][t], want, rtol=1e-13, atol=1e-300)
        acc2 = lut[cal["q_d"][e].view(np.uint8)] @ lut[r["qh"][t].view(np.uint8)]
        np.testing.assert_allclose(r["y"][t], acc2 * np.float64(r["sh"][t]) * cal["sw_d"][e],
                                   rtol=1e-12)


def test_permute_golden(golden_dir):
    g = _load(golden_dir, "permute_capacity.json")
    ids = np.array(g["ids"], np.int32)
    for key in ("with_capacity", "no_capacity"):
        c = g[key]
        p = oracle.permute(ids, g["E"], c["capacity"])
        assert p["counts"].tolist() == c["counts"]
        assert p["offsets"].tolist() == c["offsets"]
        assert p["sorted"].tolist() == c["sorted"]
        assert p["row_of"].ravel().tolist() == c["row_of"]


@pytest.mark.parametrize("T,E,k,cap", [(32, 64, 8, 0), (1000, 8, 2, 0), (4096, 128, 8, 320),
                                       (300, 16, 4, 50), (77, 5, 1, 3), (64, 8, 2, 1)])
def test_permute_bruteforce(T, E, k, cap):
    rng = np.random.default_rng(T + E)
    # skewed expert choice so capacity bites
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    hot = rng.random((T, 1)) < 0.3
    ids = np.where(hot & (np.arange(k) == 0), 0, ids).astype(np.int32)
    for t in range(T):   # keep experts distinct per token
        if ids[t, 0] == 0:
            others = [e for e in rng.permutation(E) if e != 0][: k - 1]
            ids[t, 1:] = others
    p = oracle.permute(ids, E, cap)
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")              # (expert, assignment) order
    keep = np.zeros(flat.size, bool)
    for e in range(E):
        grp = order[flat[order] == e]
        keep[grp if cap <= 0 else grp[:cap]] = True
    expect_sorted = order[keep[order]]
    assert np.array_equal(p["sorted"], expect_sorted)
    counts = np.bincount(flat, minlength=E)
    kept = counts if cap <= 0 else np.minimum(counts, cap)
    assert np.array_equal(p["counts"], kept)
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(kept)]))
    row_of = p["row_of"].ravel()
    assert np.array_equal(row_of >= 0, keep)
    assert np.array_equal(p["sorted"][row_of[keep]], np.nonzero(keep)[0])
    if cap <= 0:   # every token placed exactly k times
        assert p["kept"] == T * k and sorted(p["sorted"].tolist()) == list(range(T * k))


def test_capacity_closed_form():
    assert oracle.capacity(1.25, 4096, 8, 128) == 320
    assert oracle.capacity(0.5, 16, 2, 8) == 2
    assert oracle.capacity(1.0, 10, 3, 4) == 8        # ceil(7.5)
    assert oracle.capacity(0.0, 100, 8, 64) == 0      # no limit
    assert oracle.capacity(-1.0, 100, 8, 64) == 0


def test_permute_out_of_range_ids_dropped():
    ids = np.array([[0, 5], [-1, 1]], np.int32)
    p = oracle.permute(ids, 2, 0)
    assert p["row_of"].ravel().tolist() == [0, -1, -1, 1]
    assert p["counts"].tolist() == [1, 1]


# ------------------------------------------------------------- SmoothQuant

def test_smoothquant_golden(golden_dir):
    g = _load(golden_dir, "smoothquant_tiny.json")
    cx = f32_to_bf16_bits(np.array(g["calib_x"], np.float32))
    cal = oracle.calibrate(cx, np.array(g["w_gate"], np.float32), np.array(g["w_up"], np.float32),
                           np.array(g["w_down"], np.float32), g["alpha"])
    assert cal["s"].tolist() == g["s"]
    assert cal["inv_s"].tolist() == g["inv_s"]
    assert cal["q_gu"].tolist() == g["q_gu"]
    assert cal["q_d"].tolist() == g["q_d"]
    np.testing.assert_array_equal(cal["sw_gu"], (np.array(g["sw_gu_times_127"], np.float32) / np.float32(127)))
    np.testing.assert_array_equal(cal["sw_d"], (np.array(g["sw_d_times_127"], np.float32) / np.float32(127)))


def _small_layer(E=4, F=64, H=128, n=96, seed=3, outliers=True):
    rng = np.random.default_rng(seed)
    wg = (rng.standard_normal((E, F, H)) * 0.02).astype(np.float32)
    wu = (rng.standard_normal((E, F, H)) * 0.02).astype(np.float32)
    wd = (rng.standard_normal((E, H, F)) * 0.02).astype(np.float32)
    x = rng.standard_normal((n, H)).astype(np.float32)
    if outliers:
        x[:, [3, 77]] *= 50
    return wg, wu, wd, f32_to_bf16_bits(x)


@pytest.mark.parametrize("alpha", [0.6, 0.3, 0.5])
def test_smoothquant_identity_and_balance(alpha):
    """X diag(s)^-1 diag(s) W^T = X W^T; the smoothed weights the oracle
    quantises reproduce X W^T from the smoothed activations; and the smoothed
    ranges satisfy max|X'_j| = (ax_j aw_j)^(1-alpha), max|W'_j| = (ax_j aw_j)^alpha
    (the balance SmoothQuant is built for)."""
    wg, wu, wd, cx = _small_layer()
    E, F, H = wg.shape
    cal = oracle.calibrate(cx, wg, wu, wd, alpha, want_smoothed=True)
    s = cal["s"].astype(np.float64)
    X = bf16_bits_to_f32(cx).astype(np.float64)
    W = np.concatenate([wg, wu], axis=1).astype(np.float64)          # [E][2F][H]
    ref = np.einsum("nh,efh->nef", X, W)
    lhs = np.einsum("nh,efh->nef", X / s, W * s)
    assert np.max(np.abs(lhs - ref)) <= 1e-12 * np.max(np.abs(ref))
    # what the oracle actually quantises: fp32 W*s, activations fp32 x*inv_s
    xs = (bf16_bits_to_f32(cx) * cal["inv_s"]).astype(np.float64)
    got = np.einsum("nh,efh->nef", xs, cal["ws_gu"].astype(np.float64))
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    ax = np.abs(X).max(0)
    aw = np.abs(W).max(axis=(0, 1))
    np.testing.assert_allclose(ax / s, (ax * aw) ** (1 - alpha), rtol=2e-6)
    np.testing.assert_allclose(aw * s, (ax * aw) ** alpha, rtol=2e-6)
    np.testing.assert_allclose(np.abs(cal["ws_gu"]).max(axis=(0, 1)), (ax * aw) ** alpha, rtol=2e-6)
    assert np.all(cal["inv_s"] == (np.float32(1) / cal["s"]))


def test_smoothquant_shared_across_experts_and_projections():
    """One s per input channel for the whole layer: the weight range of a
    channel is the max over every expert's gate AND up rows."""
    wg, wu, wd, cx = _small_layer(outliers=False)
    wu[3, 5, 17] = 2.0          # only expert 3's up projection sees this
    cal = oracle.calibrate(cx, wg, wu, wd, 0.6)
    ax17 = np.abs(bf16_bits_to_f32(cx)[:, 17]).max()
    expect = np.float32(math.pow(float(ax17), 0.6000000238418579) / math.pow(2.0, 1 - 0.6000000238418579))
    assert cal["s"][17] == expect


def test_smoothquant_zero_channel_and_unsmoothed_down():
    wg, wu, wd, cx = _small_layer(outliers=False)
    cx[:, 9] = 0
    cal = oracle.calibrate(cx, wg, wu, wd, 0.6)
    assert cal["s"][9] == 1.0 and cal["inv_s"][9] == 1.0
    # down projection is not smoothed: its codes are the plain per-row quantiser
    q, sc = oracle.quant_rows(wd.reshape(-1, wd.shape[2]))
    assert np.array_equal(cal["q_d"].reshape(q.shape), q)
    assert np.array_equal(cal["sw_d"].ravel(), sc)


def test_weight_codes_per_output_channel():
    wg, wu, wd, cx = _small_layer()
    cal = oracle.calibrate(cx, wg, wu, wd, 0.6, want_smoothed=True)
    ws = cal["ws_gu"].astype(np.float64)
    q = cal["q_gu"].astype(np.float64)
    sc = cal["sw_gu"].astype(np.float64)[..., None]
    assert np.all(np.abs(ws - q * sc) <= sc * (0.5 + 1e-4))
    assert np.all(np.abs(cal["q_gu"]).max(axis=2) == 127)          # each output row spans +-127


# ----------------------------------------------------------- act quant

def test_act_quant_roundtrip():
    wl = synth.workload("tiny", T=40)
    L = synth.make_layer(synth.workload("decode", E=2, F=64))   # outlier channels, H 4096
    wg, wu, wd, cx = L.w_gate, L.w_up, L.w_down, L.calib_x
    cal = oracle.calibrate(cx, wg, wu, wd, 0.6)
    I = synth.make_inputs(synth.workload("decode", E=2, F=64), L, T=40)
    qx, sx = oracle.act_quant(I.x, cal["inv_s"])
    xs = bf16_bits_to_f32(I.x).astype(np.float64) / cal["s"].astype(np.float64)
    err = np.abs(xs - qx * sx[:, None].astype(np.float64))
    bound = sx[:, None].astype(np.float64) * (0.5 + 1e-4) + np.abs(xs) * 2e-7
    assert np.all(err <= bound)
    assert np.all(np.abs(qx).max(1) == 127)
    del wl


# ------------------------------------------------------------ int8 GEMMs

def _identity_perm(T, k, E, rng):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    return ids, oracle.permute(ids, E, 0)


def test_int8_gemms_exact_integer_matmul():
    """acc1 and acc2 equal exact integer matmuls."""
    rng = np.random.default_rng(11)
    E, F, H, T, k = 3, 64, 128, 10, 2
    cal = dict(q_gu=rng.integers(-127, 128, (E, 2 * F, H)).astype(np.int8),
               sw_gu=rng.uniform(1e-4, 1e-3, (E, 2 * F)).astype(np.float32),
               q_d=rng.integers(-127, 128, (E, H, F)).astype(np.int8),
               sw_d=rng.uniform(1e-4, 1e-3, (E, H)).astype(np.float32))
    qx = rng.integers(-127, 128, (T, H)).astype(np.int8)
    sx = rng.uniform(0.01, 0.05, T).astype(np.float32)
    ids, p = _identity_perm(T, k, E, rng)
    rows = np.arange(p["kept"], dtype=np.int32)
    r = oracle.expert_rows(rows, ids, p["sorted"], qx, sx, cal)
    for i in range(p["kept"]):
        a = p["sorted"][i]
        t, e = a // k, ids.ravel()[a]
        acc1 = cal["q_gu"][e].astype(np.int64) @ qx[t].astype(np.int64)
        assert np.array_equal(r["acc1"][i], acc1)
        acc2 = cal["q_d"][e].astype(np.int64) @ r["qh"][i].astype(np.int64)
        # y = acc2 * sh * sw_d in fp64: recover acc2 exactly
        rec = r["y"][i] / (np.float64(r["sh"][i]) * cal["sw_d"][e].astype(np.float64))
        assert np.array_equal(np.rint(rec).astype(np.int64), acc2)
        np.testing.assert_allclose(rec, acc2, rtol=1e-12, atol=1e-9)


def test_int8_gemm_extreme_codes_max_k():
    """All +-127 codes at K = 8192: |acc| = 127^2 * K (no int32 overflow)."""
    H, F = 8192, 64
    cal = dict(q_gu=np.full((1, 2 * F, H), -127, np.int8), sw_gu=np.full((1, 2 * F), 1e-6, np.float32),
               q_d=np.full((1, H, F), 127, np.int8), sw_d=np.full((1, H), 1e-6, np.float32))
    qx = np.full((1, H), 127, np.int8)
    sx = np.ones(1, np.float32)
    ids = np.zeros((1, 1), np.int32)
    r = oracle.expert_rows(np.zeros(1, np.int32), ids, np.zeros(1, np.int32), qx, sx, cal)
    assert np.all(r["acc1"] == -127 * 127 * H)
    assert -127 * 127 * H > -2 ** 31


# ---------------------------------------------- whole layer vs fp64 layer

def _fp64_layer(x_f32, wg, wu, wd, ids, w, row_of):
    """The unquantised layer in fp64 (diagnostic reference)."""
    T, k = ids.shape
    out = np.zeros((T, wd.shape[1]))
    for t in range(T):
        for j in range(k):
            if row_of[t, j] < 0:
                continue
            e = ids[t, j]
            g = wg[e].astype(np.float64) @ x_f32[t]
            u = wu[e].astype(np.float64) @ x_f32[t]
            h = g / (1 + np.exp(-g)) * u
            out[t] += float(w[t, j]) * (wd[e].astype(np.float64) @ h)
    return out


@pytest.mark.parametrize("case", ["dense", "tiny", "tiny_outliers"])
def test_fp8_layer_close_to_unquantised(case):
    """The FP8 (e4m3) layer is within FP8 quantisation error of the fp64
    unquantised layer (3 mantissa bits: a few 1e-2 relative RMS), and
    swapping gate and up is far outside it."""
    over = dict(dense=dict(E=1, k=1, T=24), tiny=dict(),
                tiny_outliers=dict(outlier_frac=0.02, outlier_mult=50.0))[case]
    wl = synth.workload("tiny", **over)
    L = synth.make_layer(wl)
    I = synth.make_inputs(wl, L)
    cal = oracle.calibrate(L.calib_x, L.w_gate, L.w_up, L.w_down, wl.alpha, fmt=oracle.FMT_FP8)
    o = oracle.forward(I.x, cal, wl.k, logits=I.logits, fmt=oracle.FMT_FP8)
    x64 = bf16_bits_to_f32(I.x).astype(np.float64)
    ref = _fp64_layer(x64, L.w_gate, L.w_up, L.w_down, o["ids"], o["w"], o["row_of"])
    got = bf16_bits_to_f32(o["out"]).astype(np.float64)
    rel = np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
    assert rel < 8e-2, rel
    swapped = _fp64_layer(x64, L.w_up, L.w_gate, L.w_down, o["ids"], o["w"], o["row_of"])
    rel_sw = np.sqrt(np.mean((got - swapped) ** 2)) / np.sqrt(np.mean(swapped ** 2))
    assert rel_sw > 0.3, rel_sw


@pytest.mark.parametrize("case", ["dense", "tiny", "tiny_drop", "tiny_outliers"])
def test_layer_close_to_unquantised(case):
    """W8A8 output is within quantisation error of the fp64 unquantised layer:
    relative RMS error ~1e-2. A dropped term, a sign error, swapped gate/up or
    a transposed operand gives O(1) error."""
    if case == "dense":   # E = 1, k = 1: a dense W8A8 SwiGLU MLP
        wl = synth.workload("tiny", E=1, k=1, T=24)
    elif case == "tiny_outliers":
        wl = synth.workload("tiny", outlier_frac=0.02, outlier_mult=50.0)
    elif case == "tiny_drop":
        wl = synth.workload("tiny", capacity_factor=0.5, T=32)
    else:
        wl = synth.workload("tiny")
    L = synth.make_layer(wl)
    I = synth.make_inputs(wl, L)
    cal = oracle.calibrate(L.calib_x, L.w_gate, L.w_up, L.w_down, wl.alpha)
    o = oracle.forward(I.x, cal, wl.k, logits=I.logits, capacity_factor=wl.capacity_factor)
    ref = _fp64_layer(bf16_bits_to_f32(I.x).astype(np.float64), L.w_gate, L.w_up, L.w_down,
                      o["ids"], o["w"], o["row_of"])
    got = bf16_bits_to_f32(o["out"]).astype(np.float64)
    rel = np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
    assert rel < 4e-2, rel
    if case == "tiny_drop":
        assert (o["row_of"] < 0).any()
        # a token with every slot dropped outputs exactly zero
        dead = np.all(o["row_of"] < 0, axis=1)
        assert np.all(o["out"][dead] & 0x7FFF == 0)
    # a planted mistake is visible at this tolerance: swap gate and up
    swapped = _fp64_layer(bf16_bits_to_f32(I.x).astype(np.float64), L.w_up, L.w_gate, L.w_down,
                          o["ids"], o["w"], o["row_of"])
    rel_sw = np.sqrt(np.mean((got - swapped) ** 2)) / np.sqrt(np.mean(ref ** 2))
    assert rel_sw > 0.3


def test_forward_stages_consistent():
    """forward() equals its stages run one by one."""
    wl = synth.workload("tiny")
    L = synth.make_layer(wl)
    I = synth.make_inputs(wl, L)
    cal = oracle.calibrate(L.calib_x, L.w_gate, L.w_up, L.w_down, wl.alpha)
    o = oracle.forward(I.x, cal, wl.k, logits=I.logits)
    ids, w = oracle.route(I.logits, wl.k)
    p = oracle.permute(ids, wl.E, 0)
    qx, sx = oracle.act_quant(I.x, cal["inv_s"])
    r = oracle.expert_rows(np.arange(p["kept"], dtype=np.int32), ids, p["sorted"], qx, sx, cal)
    out = oracle.combine(None, w, p["row_of"], r["y"])
    assert np.array_equal(o["out"], out)
    assert np.array_equal(o["qh"], r["qh"]) and np.array_equal(o["acc1"], r["acc1"])


def test_forward_empty_and_pre_routed():
    wl = synth.workload("tiny")
    L = synth.make_layer(wl)
    cal = oracle.calibrate(L.calib_x, L.w_gate, L.w_up, L.w_down, wl.alpha)
    x0 = np.zeros((0, wl.H), np.uint16)
    o = oracle.forward(x0, cal, wl.k, logits=np.zeros((0, wl.E), np.float32))
    assert o["kept"] == 0 and o["out"].shape == (0, wl.H)
    # pre-routed with k = 1 equals w * y of that expert row
    I = synth.make_inputs(wl, L)
    ids = np.full((wl.T, 1), 3, np.int32)
    w = np.full((wl.T, 1), 0.5, np.float32)
    o = oracle.forward(I.x, cal, 1, ids=ids, w=w)
    assert o["kept"] == wl.T and np.all(o["counts"][3] == wl.T)
    expect = np.array([[oracle.f64_to_bf16(0.5 * v) for v in row] for row in o["y"]], np.uint16)
    assert np.array_equal(o["out"], expect)
