"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Every case prints what names it before touching the GPU. Small shapes are
compared element by element over every stage. The full-size workloads
(prefill, stress, the expert-parallel share) are compared on every kept row
and every token too: the integer stages in one piece, the GEMM stages and the
output in chunks of tokens that the oracle computes one after the other.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
import synth
from moe_testlib import (OutCheck, QH_MISMATCH_FRAC, SH_RTOL, check_act_quant, check_out,
                         check_requant, check_routing_and_grouping, flip_allowance, layer_of,
                         rows_of, run_gpu, unpack_tiled, upload_weights)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_int8_expert_amd as m
    m.load_library()
    return torch


@functools.lru_cache(maxsize=2)
def _layer_and_cal(wl: synth.Workload):
    """The seeded layer and its oracle calibration, kept for the next test on
    the same workload (both only read)."""
    layer = layer_of(wl)
    cal = oracle.calibrate(layer.calib_x, layer.w_gate, layer.w_up, layer.w_down, wl.alpha)
    return layer, cal


def _gpu_layer(wl, cal):
    import w8a8_int8_expert_amd as m
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    upload_weights(g, cal)
    return g


def _full_parity(wl, inputs, cal, gemm_path):
    g = run_gpu(_gpu_layer(wl, cal), inputs, wl.k, wl.capacity_factor, gemm_path)
    o = oracle.forward(inputs.x, cal, wl.k, logits=inputs.logits, ids=inputs.ids, w=inputs.w,
                       capacity_factor=wl.capacity_factor)
    check_routing_and_grouping(g, o)
    check_act_quant(g, o["qx"], o["sx"])
    kept = o["kept"]
    if kept:
        acc1 = g["gpu_tensors"]["acc1"].view(-1, 2 * wl.F)[:kept].cpu().numpy()
        assert np.array_equal(acc1, o["acc1"]), "GEMM1 accumulators differ"
        qh = g["gpu_tensors"]["qh"].view(-1, wl.F)[:kept].cpu().numpy()
        sh = g["gpu_tensors"]["sh"][:kept].cpu().numpy()
        check_requant(qh, sh, o["qh"], o["sh"])
    return check_out(g["out"], o["out_exact"], allow=flip_allowance(o, cal, wl.k))


SMALL = {
    "tiny": dict(),
    "tiny_T1": dict(T=1),
    "tiny_T3": dict(T=3),
    "tiny_T65": dict(T=65),
    "tiny_T200": dict(T=200),
    "tiny_drop": dict(capacity_factor=0.5, T=40),
    "tiny_dense": dict(E=1, k=1, T=24),
    "tiny_E5k3": dict(E=5, k=3, T=50),
    "tiny_ties": dict(logit_step=0.5, T=70),
    "tiny_outliers": dict(outlier_frac=0.02, outlier_mult=50.0, lognormal_tokens=True, T=33),
    "wide_E256": dict(E=256, k=8, H=256, F=128, T=130),
    "pre_routed": dict(pre_routed=True, zipf_s=1.1, k=1, E=8, T=100),
    "pre_routed_k2": dict(pre_routed=True, zipf_s=0.0, k=2, E=8, T=17),
    "H512_F384": dict(H=512, F=384, T=48),
    # several 256-row M tiles per expert with ragged tails; 2 N tiles in each GEMM of the
    # tiled path, GEMM2's second one partial (128 of 384 columns)
    "mid_tiled": dict(T=1000, E=4, k=2, H=512, F=384),
    # 5 N tiles in both GEMMs (no tile group larger than 1), both last tiles partial
    # (128 of 192 h columns, 256 of 384 outputs), capacity drops
    "mid_odd_nt": dict(T=600, E=3, k=1, H=1792, F=896, capacity_factor=0.9),
    # the largest hidden and FFN sizes the library accepts (65536): 1024-stage K loops,
    # 342 GEMM1 N tiles with a partial last one, uncached activation rows
    "max_hidden": dict(H=65536, F=128, E=2, k=1, T=40),
    "max_ffn": dict(H=256, F=65536, E=2, k=1, T=40),
    # the batched routing path (T*k > 2048) at its block-size boundaries: 16 tokens per
    # block up to 4096 tokens, 32 up to 8192, then 64 (last blocks partial), with expert
    # counts that are not multiples of 16 (the scan's expert batches), two experts per
    # router lane (E > 64) and capacity drops
    "route_T4096_E40": dict(T=4096, E=40, k=2, H=256, F=128),
    "route_T4097_E20": dict(T=4097, E=20, k=3, H=256, F=128),
    "route_T8193_E72": dict(T=8193, E=72, k=2, H=256, F=128),
    "route_T5000_cap": dict(T=5000, E=16, k=2, H=256, F=128, capacity_factor=0.8),
    # the widest routing the library accepts: experts held 8 and 16 per router lane
    # (512 and 1024 experts) and top-k up to 32, through the fused prologue (T*k <= 2048)
    # and the batched path, with and without capacity
    "wide_E512_k16": dict(E=512, k=16, H=256, F=128, T=120),
    "wide_E1024_k32": dict(E=1024, k=32, H=256, F=128, T=64),
    "route_E512_k16": dict(E=512, k=16, H=256, F=128, T=700),
    "route_E1024_k32_cap": dict(E=1024, k=32, H=256, F=128, T=1000, capacity_factor=1.5),
    # top-32 of 40 experts held one per lane (rank-based top-k), and top-16 batched
    "k32_E40": dict(E=40, k=32, H=256, F=128, T=50),
    "route_k16_E64": dict(E=64, k=16, H=256, F=128, T=300),
    # capacity 1 (ceil(cf * T * k / E) for the smallest cf): each expert keeps its first
    # assignment, most tokens lose every slot and come out zero; fused and batched routing
    "tiny_cap1": dict(capacity_factor=1e-4, T=50),
    "route_cap1": dict(capacity_factor=1e-4, T=3000, E=16, k=2, H=256, F=128),
}


@pytest.mark.parametrize("gemm_path", [1, 2])
@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_full_parity(torch_cuda, case, gemm_path):
    wl = synth.workload("tiny", **SMALL[case])
    _say("[parity] case=%s path=%d T=%d H=%d F=%d E=%d k=%d" % (case, gemm_path, wl.T, wl.H, wl.F,
                                                                wl.E, wl.k))
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    _full_parity(wl, inputs, cal, gemm_path)


def test_all_tokens_one_expert_with_capacity(torch_cuda):
    """Every token ties on every expert: ids 0..k-1, capacity drops the tail."""
    wl = synth.workload("tiny", T=64, capacity_factor=1.0)
    _say("[parity] case=all-ties capacity=1.0")
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    inputs.logits = np.zeros_like(inputs.logits)
    inputs.logits[:, ::2] = -0.0
    for path in (1, 2):
        _full_parity(wl, inputs, cal, path)


def test_decode_full_parity(torch_cuda):
    wl = synth.workload("decode")
    _say("[parity] case=decode full T=%d" % wl.T)
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    for path in (1, 2):
        _say("[parity] decode path=%d" % path)
        _full_parity(wl, inputs, cal, path)


# Tokens whose kept rows the oracle computes at a time (bounds its host memory:
# about 0.5 GB of fp64 y rows at the prefill shape).
CHUNK_TOKENS = 2048


def _full_size_parity(wl, layer, cal):
    """Every kept row and every token of a full-size workload against the oracle."""
    inputs = synth.make_inputs(wl, layer)
    g = run_gpu(_gpu_layer(wl, cal), inputs, wl.k, wl.capacity_factor, 0)
    # integer stages in full
    if inputs.logits is not None:
        ids, w = oracle.route(inputs.logits, wl.k)
    else:
        ids, w = inputs.ids, inputs.w
    cap = oracle.capacity(wl.capacity_factor, wl.T, wl.k, wl.E)
    p = oracle.permute(ids, wl.E, cap)
    qx, sx = oracle.act_quant(inputs.x, cal["inv_s"])
    check_routing_and_grouping(g, dict(ids=ids, w=w, **p))
    check_act_quant(g, qx, sx)
    _say("[parity] %s: routing, grouping and activation codes exact (%d kept rows)"
         % (wl.name, p["kept"]))
    oc = OutCheck()
    n_diff = n_all = 0
    yri = np.full(max(p["kept"], 1), -1, np.int64)
    for t0 in range(0, wl.T, CHUNK_TOKENS):
        toks = np.arange(t0, min(wl.T, t0 + CHUNK_TOKENS))
        rows = p["row_of"][toks].ravel()
        rows = np.sort(rows[rows >= 0]).astype(np.int32)
        r = oracle.expert_rows(rows, ids, p["sorted"], qx, sx, cal, want_h=False)
        acc1 = rows_of(g, rows, "acc1", 2 * wl.F)
        bad = np.nonzero(np.any(acc1 != r["acc1"], axis=1))[0]
        assert bad.size == 0, "GEMM1 accumulators differ on %d rows (first: row %d)" % (
            bad.size, rows[bad[0]])
        qh = rows_of(g, rows, "qh", wl.F)
        d = qh.astype(np.int32) - r["qh"].astype(np.int32)
        assert np.abs(d).max(initial=0) <= 1, "requant codes differ by more than 1"
        n_diff += int(np.count_nonzero(d))
        n_all += d.size
        sh = g["gpu_tensors"]["sh"].cpu().numpy()[rows]
        np.testing.assert_allclose(sh, r["sh"], rtol=SH_RTOL, atol=0)
        yri[:] = -1
        yri[rows] = np.arange(rows.size)
        _, exact = oracle.combine(toks, w, p["row_of"], r["y"], y_row_index=yri, want_exact=True)
        oc.add(g["out"][toks], exact)
        _say("[parity] %s: tokens %d..%d (%d rows) match" % (wl.name, toks[0], toks[-1], rows.size))
    frac = n_diff / max(n_all, 1)
    _say("[parity] %s: requant codes off by one: %d of %d (%.4f %%)"
         % (wl.name, n_diff, n_all, 100 * frac))
    assert frac <= QH_MISMATCH_FRAC
    return oc.finish(wl.name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill", "stress", "ep_share"])
def test_full_size_parity(torch_cuda, name):
    wl = synth.workload(name)
    _say("[parity] case=%s full T=%d H=%d E=%d k=%d F=%d" % (name, wl.T, wl.H, wl.E, wl.k,
                                                             wl.F))
    layer, cal = _layer_and_cal(wl if name != "prefill" else synth.workload("decode"))
    _full_size_parity(wl, layer, cal)


@pytest.mark.parametrize("name", ["tiny", "decode", "stress", "ep_share"])
def test_calibrate_parity(torch_cuda, name):
    """GPU calibration reproduces the oracle's scales and codes bit for bit."""
    import torch
    import w8a8_int8_expert_amd as m
    from moe_testlib import bf16_tensor
    wl = synth.workload(name)
    _say("[calibrate] case=%s H=%d F=%d E=%d" % (name, wl.H, wl.F, wl.E))
    layer, cal = _layer_and_cal(wl)
    dev = torch.device("cuda")
    g = m.MoEW8A8(wl.H, wl.F, wl.E, wl.k)
    wg = torch.from_numpy(layer.w_gate).to(dev)
    wu = torch.from_numpy(layer.w_up).to(dev)
    wd = torch.from_numpy(layer.w_down).to(dev)
    g.calibrate(bf16_tensor(layer.calib_x, dev), wg, wu, wd, wl.alpha)
    torch.cuda.synchronize()
    del wg, wu, wd
    assert np.array_equal(g.smooth.cpu().numpy().view(np.uint32), cal["s"].view(np.uint32))
    assert np.array_equal(g.inv_smooth.cpu().numpy().view(np.uint32), cal["inv_s"].view(np.uint32))
    assert np.array_equal(g.s_gate_up.cpu().numpy().view(np.uint32), cal["sw_gu"].view(np.uint32))
    assert np.array_equal(g.s_down.cpu().numpy().view(np.uint32), cal["sw_d"].view(np.uint32))
    q_gu = unpack_tiled(g.w_gate_up.cpu().numpy(), wl.E, 2 * wl.F, wl.H)
    assert np.array_equal(q_gu, cal["q_gu"])
    q_d = unpack_tiled(g.w_down.cpu().numpy(), wl.E, wl.H, wl.F)
    assert np.array_equal(q_d, cal["q_d"])


@pytest.mark.parametrize("gemm_path", [1, 2])
def test_zero_token_rows(torch_cuda, gemm_path):
    """Tokens whose activations are all +0 or all -0: scale 0 and codes 0, so
    their expert rows have GEMM1 sums 0, h 0 and a row maximum of 0 (scale 0,
    codes 0 in the requantisation), and their output is 0; the other tokens
    are unaffected."""
    wl = synth.workload("tiny", T=30)
    _say("[parity] zero rows path=%d" % gemm_path)
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    x = inputs.x.copy()
    x[[0, 7, 8]] = 0
    x[[12, 29]] = 0x8000
    inputs = synth.Inputs(x=x, logits=inputs.logits)
    _full_parity(wl, inputs, cal, gemm_path)
    g = run_gpu(_gpu_layer(wl, cal), inputs, wl.k, wl.capacity_factor, gemm_path)
    out = synth.bf16_bits_to_f32(g["out"]).reshape(wl.T, wl.H)
    assert not np.any(out[[0, 7, 8, 12, 29]]), "a zero token's output is not zero"
    assert not np.any(g["sx"][[0, 7, 8, 12, 29]])


@pytest.mark.parametrize("gemm_path", [1, 2])
@pytest.mark.parametrize("T", [40, 3000])
def test_invalid_expert_ids(torch_cuda, T, gemm_path):
    """Pre-routed ids outside [0, E) (-1, E, E + 5, the int32 extremes) are
    dropped like capacity overflow: no row, no share of the output. Checked
    against the oracle, which drops them too, through the fused prologue
    (T = 40) and the batched routing (T * k = 6000)."""
    wl = synth.workload("tiny", T=T, pre_routed=True, zipf_s=1.1)
    _say("[parity] invalid ids T=%d path=%d" % (T, gemm_path))
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    ids = inputs.ids.copy()
    E = wl.E
    bad = [-1, E, E + 5, np.iinfo(np.int32).min, np.iinfo(np.int32).max]
    rng = np.random.default_rng(5)
    where = rng.choice(ids.size, size=max(5, ids.size // 7), replace=False)
    ids.reshape(-1)[where] = np.resize(np.array(bad, np.int32), where.size)
    ids[0, :] = -1  # a token with every slot dropped
    inputs = synth.Inputs(x=inputs.x, ids=ids, w=inputs.w)
    _full_parity(wl, inputs, cal, gemm_path)


@pytest.mark.parametrize("gemm_path", [1, 2])
@pytest.mark.parametrize("T,cf", [(40, 0.0), (3000, 0.0), (3000, 1.0)],
                         ids=["T40", "T3000", "T3000_cap"])
def test_repeated_expert_ids(torch_cuda, T, cf, gemm_path):
    """Pre-routed tokens that name one expert in several slots: each slot is
    an assignment of its own (a row per slot, weighted by that slot's weight,
    counted against the capacity in (token, slot) order), as in the oracle.
    Through the fused prologue (T = 40) and the batched routing (T * k = 6000,
    also with capacity drops)."""
    wl = synth.workload("tiny", T=T, pre_routed=True, zipf_s=1.1, capacity_factor=cf)
    _say("[parity] repeated ids T=%d cf=%g path=%d" % (T, cf, gemm_path))
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    ids = inputs.ids.copy()
    rng = np.random.default_rng(7)
    rows = rng.choice(wl.T, size=max(4, wl.T // 3), replace=False)
    ids[rows, 1:] = ids[rows, :1]          # every slot of these tokens: one expert
    ids[0, :] = 2                          # token 0 too, whatever it had
    assert (ids[:, 0] == ids[:, 1]).sum() >= rows.size
    inputs = synth.Inputs(x=inputs.x, ids=ids, w=inputs.w)
    _full_parity(wl, inputs, cal, gemm_path)


def test_weights_past_2gib(torch_cuda):
    """A layer whose gate/up codes pass 2^31 bytes (33 experts, H 8192,
    F 4096: 2.2 GB, the down codes 1.1 GB), so that every weight and row
    offset must be 64-bit: every stage against the oracle on both GEMM paths.
    (A 64-expert layer, 4.3 GB, passed as well.)"""
    wl = synth.workload("tiny", T=24, E=33, k=8, H=8192, F=4096, layer_seed=31337,
                        input_seed=31338)
    _say("[parity] weights past 2 GiB: E=33 H=8192 F=4096 T=24 k=8")
    layer, cal = _layer_and_cal(wl)
    assert cal["q_gu"].nbytes > (1 << 31)
    inputs = synth.make_inputs(wl, layer)
    del layer
    for path in (1, 2):
        _say("[parity] weights past 2 GiB path=%d" % path)
        _full_parity(wl, inputs, cal, path)


def test_two_streams_concurrent(torch_cuda):
    """Two layers (their own weights and workspaces) run on two side streams at
    once, forwards interleaved: every output equals the one each layer gives
    alone on the default stream, bit for bit (the kernels are deterministic
    and the library keeps no state between calls outside the workspace)."""
    torch = torch_cuda
    dev = torch.device("cuda")
    _say("[streams] tiny E=8 k=2 and mid E=16 k=4 on two side streams")
    layers = []
    for over in (dict(T=40), dict(T=300, E=16, k=4, H=512, F=384)):
        wl = synth.workload("tiny", **over)
        layer, cal = _layer_and_cal(wl)
        inputs = synth.make_inputs(wl, layer)
        g = _gpu_layer(wl, cal)
        x = torch.from_numpy(inputs.x.view("int16")).to(dev).view(torch.bfloat16)
        lg = torch.from_numpy(inputs.logits).to(dev)
        ref = g.forward(x, lg).clone()
        g.workspace(wl.T)
        layers.append((g, x, lg, ref))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [[], []]
    for it in range(12):
        for j, (g, x, lg, _) in enumerate(layers):
            with torch.cuda.stream(streams[j]):
                outs[j].append(g.forward(x, lg))
    torch.cuda.synchronize()
    for j, (_, _, _, ref) in enumerate(layers):
        for o in outs[j]:
            assert torch.equal(o, ref), "layer %d differs when run concurrently" % j


NONFINITE = {
    # the fused small-batch prologue (8 experts: one rank per lane)
    "tiny": dict(T=40),
    # the routing launches of a larger batch, 128 experts (two per lane)
    "E128_k8": dict(T=400, E=128, k=8, H=256, F=128),
}


@pytest.mark.parametrize("name", sorted(NONFINITE))
def test_nonfinite_logits(torch_cuda, name):
    """Router logits with NaN and infinite entries. Reading: a NaN ranks below
    every number, -inf below every finite one, so a row with at least k
    finite logits routes as if its NaNs were -inf: that oracle's ids and
    weights, and its output. A row with no finite logit takes experts
    0..k-1 (equal keys: the lower index wins), its weights and output are
    NaN and are not compared."""
    wl = synth.workload("tiny", **NONFINITE[name])
    _say("[nonfinite] %s %s" % (name, NONFINITE[name]))
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    lg = inputs.logits.copy()
    T, E, k = wl.T, wl.E, wl.k
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    lg[0, 3] = nan                      # one NaN
    lg[1, : E - k] = nan                # exactly k finite logits left
    lg[2, ::2] = -inf                   # masked experts
    lg[3, :] = nan                      # no finite logit
    lg[4, 1], lg[4, E - 1] = nan, -inf
    lg[5, E // 2] = inf                 # one +inf: chosen first, with weight NaN
    g = run_gpu(_gpu_layer(wl, cal), synth.Inputs(x=inputs.x, logits=lg), k)
    ids = g["ids"]
    assert ids.min() >= 0 and ids.max() < E
    assert all(len(set(r)) == k for r in ids.tolist()), "repeated expert in a row"
    assert ids[3].tolist() == list(range(k))
    assert ids[5, 0] == E // 2
    o = oracle.forward(inputs.x, cal, k, logits=np.where(np.isnan(lg), -inf, lg))
    assert np.array_equal(ids, o["ids"]), "routing ids differ"
    cmp_rows = np.ones(T, bool)
    cmp_rows[[3, 5]] = False
    assert np.max(np.abs(g["w"][cmp_rows].astype(np.float64) - o["w"][cmp_rows]),
                  initial=0.0) <= 1e-6
    H = wl.H
    c = OutCheck()
    c.add(g["out"].reshape(T, H)[cmp_rows], o["out_exact"].reshape(T, H)[cmp_rows])
    c.finish(name)


@pytest.mark.parametrize("gemm_path", [1, 2])
def test_deterministic_large(torch_cuda, gemm_path):
    """Three runs of a batch of 3000 tokens (64 experts, top-8, capacity 1.25:
    batched routing, many tiles whose order is taken from an atomic queue on
    the tiled path, row maxima by atomics) give identical bits in the output
    and in every debug stage."""
    torch = torch_cuda
    wl = synth.workload("tiny", T=3000, E=64, k=8, H=512, F=256, capacity_factor=1.25)
    _say("[parity] case=determinism T=3000 E=64 k=8 path=%d" % gemm_path)
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    gl = _gpu_layer(wl, cal)
    runs = [run_gpu(gl, inputs, wl.k, wl.capacity_factor, gemm_path) for _ in range(3)]
    first = runs[0]
    for r in runs[1:]:
        assert np.array_equal(r["out"], first["out"])
        for name in ("ids", "row_of", "sorted", "qx", "sx"):
            assert np.array_equal(r[name], first[name]), name
        for name in ("acc1", "qh", "sh", "y"):
            a = first["gpu_tensors"][name]
            b = r["gpu_tensors"][name]
            n = a.numel() * first["kept"] // max(wl.T * wl.k, 1)
            assert bool((a[:n].view(torch.uint8) == b[:n].view(torch.uint8)).all()), name


def test_deterministic_and_t0(torch_cuda):
    """Two runs give identical bits; T = 0 is a no-op."""
    import torch
    import w8a8_int8_expert_amd as m
    wl = synth.workload("tiny", T=100)
    _say("[parity] case=determinism")
    layer, cal = _layer_and_cal(wl)
    inputs = synth.make_inputs(wl, layer)
    gl = _gpu_layer(wl, cal)
    for path in (1, 2):
        a = run_gpu(gl, inputs, wl.k, 0.0, path)["out"]
        b = run_gpu(gl, inputs, wl.k, 0.0, path)["out"]
        assert np.array_equal(a, b)
    x0 = torch.empty(0, wl.H, dtype=torch.bfloat16, device="cuda")
    lg0 = torch.empty(0, wl.E, dtype=torch.float32, device="cuda")
    out0 = gl.forward(x0, router_logits=lg0)
    assert out0.shape == (0, wl.H)
    rc = m.moe_w8a8_forward(gl.d, gl.weights, x0, 0, lg0, None, None, 0.0, out0, None, 0)
    assert rc == m.MOE_W8A8_OK
