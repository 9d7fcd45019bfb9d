"""The benchmark's host-side arithmetic, checked on the CPU: the algorithmic
bytes it divides by the measured times, the stages it expects to time, and
its refusal of more than one GPU. The expected values are the closed forms
written out by hand for the workloads' sizes."""
import os
import subprocess
import sys

import numpy as np

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_algorithmic_bytes():
    """Decode: 32 tokens, hidden 4096, FFN 1536, 64 experts all touched, top-8.
    GEMM1 reads every touched expert's gate/up codes (2 * 1536 * 4096 bytes)
    and their fp32 scales (4 * 2 * 1536); the layer reads the gate/up and
    down codes (3 * 1536 * 4096) and all their scales (4 * (3072 + 4096)),
    inv_s (4 * 4096), the tokens in and out (2 + 2 bytes * 32 * 4096) and the
    fp32 logits (4 * 32 * 64)."""
    wl = synth.workload("decode")
    assert (wl.T, wl.H, wl.F, wl.E, wl.k, wl.pre_routed) == (32, 4096, 1536, 64, 8, False)
    assert bench.gemm1_bytes(wl, 64) == 64 * (2 * 1536 * 4096 + 4 * 2 * 1536) == 806_092_800
    counts = np.full(64, 4)
    b, touched = bench.layer_bytes(wl, counts, wl.T)
    assert touched == 64
    assert b == (64 * (3 * 1536 * 4096 + 4 * (3072 + 4096)) + 4 * 4096 + 4 * 32 * 4096
                 + 4 * 32 * 64) == 1_210_343_424


def test_untouched_experts_and_pre_routed_bytes():
    """Only touched experts' weights count; pre-routed input is int32 ids and
    fp32 weights (8 bytes per assignment) instead of fp32 logits."""
    wl = synth.workload("ep_share")
    assert wl.pre_routed
    counts = np.zeros(wl.E, np.int64)
    counts[:5] = 7
    b, touched = bench.layer_bytes(wl, counts, wl.T)
    assert touched == 5
    H, F, T, k = wl.H, wl.F, wl.T, wl.k
    assert b == 5 * (3 * H * F + 4 * (2 * F + H)) + 4 * H + 4 * T * H + 8 * T * k


def test_launched_stages():
    """Up to 2048 assignments routing, grouping and activation quantisation
    are one launch; beyond, each has its own."""
    assert bench.launched_stages(synth.workload("decode")) == \
        ["route", "gemm1", "requant", "gemm2", "combine"]
    assert bench.launched_stages(synth.workload("prefill")) == \
        ["route", "scan", "scatter", "act_quant", "gemm1", "requant", "gemm2", "combine"]


def test_more_than_one_gpu_refused():
    """--gpus above 1 exits with status 2 and says why, before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "measures one GPU only" in r.stderr, r.stderr
    assert r.stdout == ""
