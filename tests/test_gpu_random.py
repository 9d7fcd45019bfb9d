"""Parity of the HIP path against the CPU oracle on layer configurations drawn at
random (fixed seed, so every run checks the same cases): token counts, expert
counts, top-k, hidden and FFN sizes across the supported range, with or
without a capacity limit, tied logits, outlier channels or pre-routed inputs,
on the streaming and the tiled GEMM path. Every stage is compared as in the
small-shape parity tests (routing, grouping, codes and GEMM1 accumulators
bit-exact; requantised codes within one step in at most 0.1 % of entries;
output within 2e-2 x RMS plus half a bf16 step, plus the effect of the
requantised codes that may flip). Further families: the widest routing,
medium sizes, FP8 experts, the router projection, activation clips (INT8 and
FP8). Sizes are capped so that the oracle finishes each case in seconds.
"""
import numpy as np
import pytest

import synth
from test_gpu_parity import _full_parity, _layer_and_cal, _say, torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu

N_CASES = 160


def _draw(i):
    rng = np.random.default_rng(np.random.SeedSequence([2024, i]))
    H = int(rng.choice([256, 512, 768, 1024, 1280]))
    F = int(rng.choice([128, 256, 384, 640, 896]))
    E = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 65, 100, 128]))
    k = int(rng.integers(1, min(E, 8) + 1))
    # weight bytes E*3*H*F*4 and oracle work T*k*3*H*F kept small
    if E * 3 * H * F * 4 > 300e6:
        H, F = 256, 128
    t_max = max(1, min(4000, int(2.5e9 // (k * 3 * H * F))))
    T = int(rng.integers(1, t_max + 1))
    over = dict(T=T, H=H, F=F, E=E, k=k, layer_seed=7000 + i, input_seed=8000 + i)
    if rng.random() < 0.3:
        over["capacity_factor"] = float(np.round(rng.uniform(0.5, 1.5), 2))
    if rng.random() < 0.3:
        over["logit_step"] = 0.25
    if rng.random() < 0.2:
        over.update(outlier_frac=0.02, outlier_mult=50.0, lognormal_tokens=True)
    if rng.random() < 0.15:
        over.update(pre_routed=True, zipf_s=1.1)
    path = int(rng.integers(1, 3))
    return over, path


CASES = [_draw(i) for i in range(N_CASES)]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config_parity(torch_cuda, i):  # noqa: F811
    over, path = CASES[i]
    wl = synth.workload("tiny", **over)
    _say("[random] case=%d path=%d %s" % (i, path, over))
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    _full_parity(wl, inputs, cal, path)



# Draws over the widest routing the library accepts: 129 to 1024 experts
# (two to sixteen experts per router lane) and top-k up to 32, small hidden and
# FFN sizes, with or without capacity and tied logits.
N_WIDE = 24


def _draw_wide(i):
    rng = np.random.default_rng(np.random.SeedSequence([2026, i]))
    E = int(rng.choice([129, 200, 256, 257, 512, 700, 1000, 1024]))
    k = int(rng.choice([1, 3, 8, 9, 16, 17, 31, 32]))
    H = int(rng.choice([256, 512]))
    F = int(rng.choice([128, 256]))
    T = int(rng.integers(1, max(2, int(2.5e9 // (k * 3 * H * F))) + 1))
    T = min(T, 1500)
    over = dict(T=T, H=H, F=F, E=E, k=k, layer_seed=9000 + i, input_seed=9500 + i)
    if rng.random() < 0.4:
        over["capacity_factor"] = float(np.round(rng.uniform(0.6, 1.5), 2))
    if rng.random() < 0.4:
        over["logit_step"] = 0.25
    return over, int(rng.integers(1, 3))


CASES_WIDE = [_draw_wide(i) for i in range(N_WIDE)]


@pytest.mark.parametrize("i", range(N_WIDE))
def test_random_config_wide_routing_parity(torch_cuda, i):  # noqa: F811
    over, path = CASES_WIDE[i]
    wl = synth.workload("tiny", **over)
    _say("[random wide] case=%d path=%d %s" % (i, path, over))
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    _full_parity(wl, inputs, cal, path)


# The FP8 (e4m3) expert path on further draws, to its own bars (activation
# codes and scales bit-exact; every other bar derived from the oracle's
# quantities and the accumulation assumption, test_gpu_fp8.fp8_bounds).
N_FP8 = 36
CASES_FP8 = [_draw(100 + i) for i in range(N_FP8)]


@pytest.mark.parametrize("i", range(N_FP8))
def test_random_config_fp8_parity(torch_cuda, i):  # noqa: F811
    from test_gpu_fp8 import fp8_full_parity
    over, path = CASES_FP8[i]
    wl = synth.workload("tiny", **over)
    _say("[random fp8] case=%d path=%d %s" % (i, path, over))
    fp8_full_parity(wl, path)


# Router-projection mode (logits = x . W_r^T on the GPU) on further draws.
N_ROUTER = 24
CASES_ROUTER = [_draw(200 + i) for i in range(N_ROUTER)]


@pytest.mark.parametrize("i", range(N_ROUTER))
def test_random_config_router_parity(torch_cuda, i):  # noqa: F811
    from test_gpu_router import router_full_parity
    over, path = CASES_ROUTER[i]
    over = dict(over, pre_routed=False)
    wl = synth.workload("tiny", **over)
    _say("[random router] case=%d path=%d %s" % (i, path, over))
    router_full_parity(torch_cuda, wl, path)


# Activation clips on further draws: dynamic saturation at a percentile
# that leaves 2-12 values of a token above the level, with or without the static
# clip from the calibration tokens.
N_CLIP = 24


def _draw_clip(i):
    import oracle
    over, path = _draw(300 + i)
    rng = np.random.default_rng(np.random.SeedSequence([2025, i]))
    H = over["H"]
    m = int(rng.integers(2, 13))
    p = float(np.float32(100.0 * (H - m + 0.5) / H))
    assert 2 <= H - oracle.percentile_rank(p, H) + 1 <= 16
    return over, path, bool(rng.random() < 0.5), p


CASES_CLIP = [_draw_clip(i) for i in range(N_CLIP)]


@pytest.mark.parametrize("i", range(N_CLIP))
def test_random_config_clip_parity(torch_cuda, i):  # noqa: F811
    from test_gpu_clip import clip_full_parity
    over, path, static, sat_p = CASES_CLIP[i]
    wl = synth.workload("tiny", **over)
    _say("[random clip] case=%d path=%d static=%s sat=%.6g %s" % (i, path, static, sat_p, over))
    clip_full_parity(torch_cuda, wl, path, static, sat_p)


# Medium shapes: hidden 1536-4096, FFN 512-2048, up to 64 experts, so that the
# K loops run 24-64 stages and GEMM2 has up to 11 N tiles (weights capped at
# 1.2 GB, oracle work at 1.5e10 multiply-adds per draw).
N_MEDIUM = 12


def _draw_medium(i):
    rng = np.random.default_rng(np.random.SeedSequence([2030, i]))
    H = int(rng.choice([1536, 2048, 2560, 3072, 4096]))
    F = int(rng.choice([512, 768, 1024, 1536, 2048]))
    E = int(rng.choice([4, 8, 16, 33, 64]))
    k = int(rng.integers(1, min(E, 8) + 1))
    if E * 3 * H * F > 1.2e9:
        E = max(1, int(1.2e9 // (3 * H * F)))
        k = min(k, E)
    t_max = max(1, min(1500, int(1.5e10 // (k * 3 * H * F))))
    T = int(rng.integers(1, t_max + 1))
    over = dict(T=T, H=H, F=F, E=E, k=k, layer_seed=11000 + i, input_seed=12000 + i)
    if rng.random() < 0.3:
        over["capacity_factor"] = float(np.round(rng.uniform(0.5, 1.5), 2))
    if rng.random() < 0.3:
        over.update(outlier_frac=0.02, outlier_mult=50.0, lognormal_tokens=True)
    return over, int(rng.integers(1, 3))


CASES_MEDIUM = [_draw_medium(i) for i in range(N_MEDIUM)]


@pytest.mark.parametrize("i", range(N_MEDIUM))
def test_random_config_medium_parity(torch_cuda, i):  # noqa: F811
    over, path = CASES_MEDIUM[i]
    wl = synth.workload("tiny", **over)
    _say("[random medium] case=%d path=%d %s" % (i, path, over))
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    _full_parity(wl, inputs, cal, path)


# FP8 experts on four further medium-size draws, to the FP8 bars.
N_MEDIUM_FP8 = 4
CASES_MEDIUM_FP8 = [_draw_medium(100 + i) for i in range(N_MEDIUM_FP8)]


@pytest.mark.parametrize("i", range(N_MEDIUM_FP8))
def test_random_config_medium_fp8_parity(torch_cuda, i):  # noqa: F811
    from test_gpu_fp8 import fp8_full_parity
    over, path = CASES_MEDIUM_FP8[i]
    wl = synth.workload("tiny", **over)
    _say("[random medium fp8] case=%d path=%d %s" % (i, path, over))
    fp8_full_parity(wl, path)


# FP8 experts with activation clips, on the clip family's first eight draws.
N_FP8_CLIP = 8


@pytest.mark.parametrize("i", range(N_FP8_CLIP))
def test_random_config_fp8_clip_parity(torch_cuda, i):  # noqa: F811
    from test_gpu_clip import fp8_clip_full_parity
    over, path, static, sat_p = CASES_CLIP[i]
    wl = synth.workload("tiny", **over)
    _say("[random fp8 clip] case=%d path=%d static=%s sat=%.6g %s"
         % (i, path, static, sat_p, over))
    fp8_clip_full_parity(torch_cuda, wl, path, static, sat_p)
