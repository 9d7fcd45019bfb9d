"""The C-ABI library loads, exports every declared entry point, and validates
its arguments on the host (no GPU is touched by these cases)."""
import ctypes
import os
import re

import pytest

import w8a8_int8_expert_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a non-NULL pointer that validation never dereferences


@pytest.fixture(scope="module")
def lib():
    # The sanitizer test runs these cases against an instrumented build of the
    # library, named by this variable.
    path = os.environ.get("MOE_W8A8_TEST_LIB", m.LIB_PATH)
    if not os.path.exists(path):
        from w8a8_int8_expert_amd import build
        build.build()
    return m.load_library(path)


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_w8a8_\w+)\s*\(", src,
                                re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(m.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, 7):
        assert m.moe_w8a8_strerror(code)
    assert m.moe_w8a8_strerror(-3) == "workspace missing or too small"


def test_workspace_size_nondecreasing(lib):
    """A workspace sized for the largest batch serves every smaller one, also across
    the routing kernels' block-size steps (16/32/64 tokens at 4096 and 8192) and the
    small-batch path's limit (T*k = 2048)."""
    import w8a8_int8_expert_amd as m
    Ts = sorted(set(list(range(0, 300)) + list(range(1000, 1030)) + list(range(2040, 2060)) +
                    list(range(4085, 4110)) + list(range(8185, 8210)) + [16383, 16384, 16385]))
    for d in (m.dims(256, 128, 1024, 1), m.dims(256, 128, 8, 2), m.dims(4096, 1536, 64, 8),
              m.dims(8192, 2048, 32, 1)):
        sizes = [m.moe_w8a8_workspace_size(d, T) for T in Ts]
        assert all(s > 0 for s in sizes)
        bad = [(Ts[i], Ts[i + 1]) for i in range(len(Ts) - 1) if sizes[i + 1] < sizes[i]]
        assert not bad, "workspace shrinks between T=%s" % (bad[:3],)


def test_workspace_size_pure(lib):
    d = m.dims(4096, 1536, 64, 8)
    a = m.moe_w8a8_workspace_size(d, 32)
    assert a == m.moe_w8a8_workspace_size(d, 32) > 0
    assert m.moe_w8a8_workspace_size(d, 16384) > a
    assert m.moe_w8a8_workspace_size(d, 0) >= 2 * 4 * 4096
    assert m.moe_w8a8_workspace_size(d, -1) == 0
    assert m.moe_w8a8_workspace_size(m.dims(4096, 1536, 64, 65), 1) == 0     # k > E
    assert m.moe_w8a8_workspace_size(m.dims(4000, 1536, 64, 8), 1) == 0     # H % 256
    assert m.moe_w8a8_workspace_size(m.dims(4096, 1536, 2048, 8), 1) == 0   # E > 1024


def test_row_limit_without_overflow(lib):
    """A batch is refused once T*k or the padded row count T*k + 15*min(T*k, E)
    reaches 2^31, exactly at that boundary, and a T whose T*k overflows int64
    is refused too (workspace size 0, forward and router INVALID, nothing
    launched)."""
    lim = (1 << 31) - 1
    d = m.dims(256, 128, 1, 1)          # E = 1: padding adds at most 15 rows
    assert m.moe_w8a8_workspace_size(d, lim - 15) > 0
    assert m.moe_w8a8_workspace_size(d, lim - 14) == 0
    d = m.dims(256, 128, 1024, 1)       # E = 1024: up to 15360 padding rows
    assert m.moe_w8a8_workspace_size(d, lim - 15 * 1024) > 0
    assert m.moe_w8a8_workspace_size(d, lim - 15 * 1024 + 1) == 0
    d = m.dims(256, 128, 64, 32)
    t = (lim - 15 * 64) // 32
    assert m.moe_w8a8_workspace_size(d, t) > 0
    assert m.moe_w8a8_workspace_size(d, t + 1) == 0
    for T in ((1 << 62), (1 << 63) - 1, (1 << 63) // 32 + 1):
        assert m.moe_w8a8_workspace_size(d, T) == 0
        assert _fwd(d, T=T, ws_bytes=(1 << 63) - 1) == m.MOE_W8A8_ERR_INVALID
        assert m.moe_w8a8_router_logits(d, FAKE, T, FAKE, FAKE, FAKE, 1 << 62,
                                        stream=0) == m.MOE_W8A8_ERR_INVALID
        assert m.moe_w8a8_forward_noalloc(d, _weights(), FAKE, T, FAKE, None, None, 0.0, FAKE,
                                          None, stream=0) == m.MOE_W8A8_ERR_INVALID


def _weights():
    return m.moe_w8a8_weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def _fwd(d, T=4, logits=FAKE, ids=None, w=None, ws=FAKE, ws_bytes=1 << 40, dbg=None, cf=0.0,
         weights=None, x=FAKE, out=FAKE):
    return m.moe_w8a8_forward(d, weights or _weights(), x, T, logits, ids, w, cf, out, ws,
                              ws_bytes, dbg, stream=0)


def test_forward_validation(lib):
    d = m.dims(256, 512, 8, 2)
    L = lib
    # NULL dims
    assert L.moe_w8a8_forward(None, ctypes.byref(_weights()), FAKE, 4, FAKE, None, None, 0.0,
                              FAKE, FAKE, 1 << 40, None, None) == m.MOE_W8A8_ERR_INVALID
    assert _fwd(m.dims(256, 512, 8, 9)) == m.MOE_W8A8_ERR_INVALID          # k > E
    assert _fwd(m.dims(0, 512, 8, 2)) == m.MOE_W8A8_ERR_INVALID
    assert _fwd(d, T=-1) == m.MOE_W8A8_ERR_INVALID
    assert _fwd(d, logits=FAKE, ids=FAKE, w=FAKE) == m.MOE_W8A8_ERR_INVALID  # both
    assert _fwd(d, logits=None) == m.MOE_W8A8_ERR_INVALID       # neither, no router matrix
    assert _fwd(d, logits=None, ids=FAKE, w=None) == m.MOE_W8A8_ERR_INVALID  # half pre-routed
    assert _fwd(d, x=None) == m.MOE_W8A8_ERR_INVALID
    assert _fwd(d, out=None) == m.MOE_W8A8_ERR_INVALID
    assert _fwd(d, cf=float("nan")) == m.MOE_W8A8_ERR_INVALID
    bad = _weights()
    bad.w_down = None
    assert _fwd(d, weights=bad) == m.MOE_W8A8_ERR_INVALID
    dbg = m.moe_w8a8_debug()
    dbg.gemm_path = 3
    assert _fwd(d, dbg=dbg) == m.MOE_W8A8_ERR_INVALID
    badf = _weights()
    badf.format = 2
    assert _fwd(d, weights=badf) == m.MOE_W8A8_ERR_INVALID               # unknown format
    bads = _weights()
    for p in (-1.0, 100.5, float("nan")):
        bads.act_sat_percentile = p
        assert _fwd(d, weights=bads) == m.MOE_W8A8_ERR_INVALID
    bads.act_sat_percentile = 90.0                                       # H 256: m = 26 > 16
    assert _fwd(d, weights=bads) == m.MOE_W8A8_ERR_UNSUPPORTED
    assert _fwd(m.dims(320, 512, 8, 2)) == m.MOE_W8A8_ERR_UNSUPPORTED      # H % 256
    assert _fwd(m.dims(256, 500, 8, 2)) == m.MOE_W8A8_ERR_UNSUPPORTED      # F % 128
    assert _fwd(m.dims(256, 512, 64, 33)) == m.MOE_W8A8_ERR_UNSUPPORTED    # k > 32
    need = m.moe_w8a8_workspace_size(d, 4)
    assert _fwd(d, ws_bytes=need - 1) == m.MOE_W8A8_ERR_WORKSPACE
    assert _fwd(d, ws=None) == m.MOE_W8A8_ERR_WORKSPACE
    assert _fwd(d, T=1 << 30, ws_bytes=1) == m.MOE_W8A8_ERR_INVALID         # T*k >= 2^31
    # T == 0 is a successful no-op (nothing is enqueued)
    assert _fwd(d, T=0, ws=None, ws_bytes=0, x=None, out=None) == m.MOE_W8A8_OK


def test_router_logits_validation(lib):
    d = m.dims(1024, 512, 8, 2)   # H > 512: the per-part sums need the workspace
    def rl(d=d, x=FAKE, T=4, w=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return m.moe_w8a8_router_logits(d, x, T, w, out, ws, ws_bytes, stream=0)
    assert rl(x=None) == m.MOE_W8A8_ERR_INVALID
    assert rl(w=None) == m.MOE_W8A8_ERR_INVALID
    assert rl(out=None) == m.MOE_W8A8_ERR_INVALID
    assert rl(T=-1) == m.MOE_W8A8_ERR_INVALID
    assert rl(d=m.dims(1024, 512, 8, 9)) == m.MOE_W8A8_ERR_INVALID         # k > E
    assert rl(d=m.dims(1000, 512, 8, 2)) == m.MOE_W8A8_ERR_UNSUPPORTED     # H % 256
    assert rl(ws=None) == m.MOE_W8A8_ERR_WORKSPACE
    assert rl(ws_bytes=m.moe_w8a8_workspace_size(d, 4) - 1) == m.MOE_W8A8_ERR_WORKSPACE
    assert rl(T=0, x=None, w=None, out=None, ws=None, ws_bytes=0) == m.MOE_W8A8_OK


def test_calibrate_validation(lib):
    d = m.dims(256, 512, 8, 2)
    w = _weights()
    def cal(d=d, alpha=0.6, n=64, cx=FAKE, ws=FAKE, ws_bytes=1 << 30, out=w):
        return m.moe_w8a8_calibrate(d, alpha, cx, n, FAKE, FAKE, FAKE, out, ws, ws_bytes, 0)
    assert cal(alpha=1.5) == m.MOE_W8A8_ERR_INVALID
    assert cal(alpha=float("nan")) == m.MOE_W8A8_ERR_INVALID
    assert cal(n=-1) == m.MOE_W8A8_ERR_INVALID
    for n in ((1 << 61) // 256, (1 << 62), (1 << 63) - 1):       # n_calib * H >= 2^61
        assert cal(n=n) == m.MOE_W8A8_ERR_INVALID
    assert cal(cx=None) == m.MOE_W8A8_ERR_INVALID
    bad = _weights()
    bad.smooth = None
    assert cal(out=bad) == m.MOE_W8A8_ERR_INVALID
    assert cal(d=m.dims(256, 500, 8, 2)) == m.MOE_W8A8_ERR_UNSUPPORTED
    assert cal(ws_bytes=16) == m.MOE_W8A8_ERR_WORKSPACE
    assert cal(ws=None) == m.MOE_W8A8_ERR_WORKSPACE
    badf = _weights()
    badf.format = 7
    assert cal(out=badf) == m.MOE_W8A8_ERR_INVALID


def test_calibrate_clip_validation(lib):
    d = m.dims(256, 512, 8, 2)
    def cc(p=99.9, cx=FAKE, n=64, inv=FAKE, out=FAKE, d=d):
        return m.moe_w8a8_calibrate_clip(d, p, cx, n, inv, out, stream=0)
    for p in (0.0, -1.0, 100.1, float("nan")):
        assert cc(p=p) == m.MOE_W8A8_ERR_INVALID
    assert cc(cx=None) == m.MOE_W8A8_ERR_INVALID
    assert cc(n=-1) == m.MOE_W8A8_ERR_INVALID
    assert cc(inv=None) == m.MOE_W8A8_ERR_INVALID
    assert cc(out=None) == m.MOE_W8A8_ERR_INVALID
    assert cc(d=m.dims(320, 512, 8, 2)) == m.MOE_W8A8_ERR_UNSUPPORTED
    # n_calib * H >= 2^61, including counts whose product overflows int64
    for n in ((1 << 61) // 256, (1 << 62), (1 << 63) - 1):
        assert cc(n=n) == m.MOE_W8A8_ERR_INVALID


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("w8a8_int8_expert_amd")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError):
            mod.load_library(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


def test_binding_rejects_mismatched_tensors(lib):
    """The Python binding checks dtype, shape, contiguity and device of every
    tensor before it hands raw pointers to the library (CPU tensors on a
    CPU-placed layer: every case is refused before any call into the library)."""
    import torch
    H, F, E, k, T = 256, 128, 8, 2, 5
    g = m.MoEW8A8(H, F, E, k, device="cpu")
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    lg = torch.zeros(T, E, dtype=torch.float32)
    ids = torch.zeros(T, k, dtype=torch.int32)
    w = torch.zeros(T, k, dtype=torch.float32)
    bad = [
        dict(x=x.float(), router_logits=lg),                        # x not bf16
        dict(x=torch.zeros(T, H + 8, dtype=torch.bfloat16), router_logits=lg),  # width != H
        dict(x=torch.zeros(H, T, dtype=torch.bfloat16).t(), router_logits=lg),  # not contiguous
        dict(x=x, router_logits=lg.to(torch.bfloat16)),             # logits not fp32
        dict(x=x, router_logits=torch.zeros(T, E + 1)),             # logits [T][E+1]
        dict(x=x, topk_ids=ids.long(), topk_w=w),                   # int64 ids (torch.topk's)
        dict(x=x, topk_ids=torch.zeros(T, k + 1, dtype=torch.int32), topk_w=w),
        dict(x=x, topk_ids=ids, topk_w=w.double()),
        dict(x=x, router_logits=lg, out=torch.zeros(T, H)),         # out not bf16
        dict(x=x, router_logits=lg, out=torch.zeros(T - 1, H, dtype=torch.bfloat16)),
    ]
    for kw in bad:
        with pytest.raises(m.MoEW8A8Error):
            g.forward(**kw)
    with pytest.raises(m.MoEW8A8Error):
        g.calibrate(x, torch.zeros(E, F, H), torch.zeros(E, F, H), torch.zeros(E, F, H), 0.6)
    with pytest.raises(m.MoEW8A8Error):
        g.calibrate(x.float(), torch.zeros(E, F, H), torch.zeros(E, F, H),
                    torch.zeros(E, H, F), 0.6)
    if torch.cuda.is_available():  # a tensor on another device than the layer's
        with pytest.raises(m.MoEW8A8Error):
            g.forward(x.cuda(), router_logits=lg)


def test_binding_calls_on_the_layers_device(lib, monkeypatch):
    """Every method of the binding calls into the library inside the layer's
    device context (the library launches on the current device and torch's
    current stream of it). The library entry points and the context are
    replaced by recorders: nothing runs on a device."""
    import contextlib
    import torch
    H, F, E, k, T = 256, 128, 8, 2, 5
    g = m.MoEW8A8(H, F, E, k, device="cpu")
    depth = [0]
    seen = []

    @contextlib.contextmanager
    def on_device():
        depth[0] += 1
        try:
            yield
        finally:
            depth[0] -= 1
    monkeypatch.setattr(g, "_on_device", on_device)
    for name in ("moe_w8a8_forward", "moe_w8a8_forward_noalloc", "moe_w8a8_calibrate",
                 "moe_w8a8_calibrate_clip", "moe_w8a8_router_logits", "moe_w8a8_pack"):
        def rec(*a, _name=name, **kw):
            seen.append((_name, depth[0]))
            return m.MOE_W8A8_OK
        monkeypatch.setattr(m, name, rec)
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    lg = torch.zeros(T, E, dtype=torch.float32)
    g.forward(x, router_logits=lg)
    g.forward_noalloc(x, torch.empty(T, H, dtype=torch.bfloat16), router_logits=lg)
    g.calibrate(x, torch.zeros(E, F, H), torch.zeros(E, F, H), torch.zeros(E, H, F), 0.6)
    g.calibrate_clip(x, 99.9)
    g.set_router(torch.zeros(E, H, dtype=torch.bfloat16))
    g.router_logits(x)
    g.load_quantized(torch.zeros(E, 2 * F, H, dtype=torch.int8), torch.ones(E, 2 * F),
                     torch.zeros(E, H, F, dtype=torch.int8), torch.ones(E, H), torch.ones(H),
                     torch.ones(H))
    assert [n for n, _ in seen] == ["moe_w8a8_forward", "moe_w8a8_forward_noalloc",
                                    "moe_w8a8_calibrate", "moe_w8a8_calibrate_clip",
                                    "moe_w8a8_router_logits", "moe_w8a8_pack", "moe_w8a8_pack"]
    assert all(d == 1 for _, d in seen), seen


def test_pack_validation(lib):
    """moe_w8a8_pack refuses bad sizes, NULL, misaligned or overlapping buffers
    before anything is enqueued."""
    A, B = 0x100000, 0x900000   # 16-byte aligned, 8 MiB apart
    INV, UNS = m.MOE_W8A8_ERR_INVALID, m.MOE_W8A8_ERR_UNSUPPORTED
    assert lib.moe_w8a8_pack(0, 16, 64, A, B, None) == INV
    assert lib.moe_w8a8_pack(1, 0, 64, A, B, None) == INV
    assert lib.moe_w8a8_pack(1, 16, -64, A, B, None) == INV
    assert lib.moe_w8a8_pack(1, 16, 64, None, B, None) == INV
    assert lib.moe_w8a8_pack(1, 16, 64, A, None, None) == INV
    assert lib.moe_w8a8_pack(1, 16, 64, A + 8, B, None) == INV        # misaligned
    assert lib.moe_w8a8_pack(1, 16, 64, A, A + 512, None) == INV      # overlapping
    assert lib.moe_w8a8_pack(4, 16, 64, A, A + 2048, None) == INV     # 4 KB overlaps
    assert lib.moe_w8a8_pack(1, 24, 64, A, B, None) == UNS            # N % 16
    assert lib.moe_w8a8_pack(1, 16, 96, A, B, None) == UNS            # K % 64
    assert lib.moe_w8a8_pack(1 << 20, 1 << 14, 1 << 14, A, B, None) == INV   # > 2^40 bytes


def test_library_shares_torch_hip_runtime():
    """Loading the library before torch is imported still leaves one HIP runtime
    in the process, torch's: the binding's device memory and streams belong to
    it. (A second runtime, initialised after torch's, finds no device.)"""
    import subprocess
    import sys
    code = ("import w8a8_int8_expert_amd as m\n"
            "m.load_library()\n"
            "import torch\n"
            "print(sorted(set(l.split()[-1] for l in open('/proc/self/maps') if 'amdhip64' in l)))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    maps = eval(r.stdout.strip().splitlines()[-1])
    assert len(maps) == 1 and "/torch/lib/" in maps[0], maps


def test_header_is_c99_and_links_from_c(tmp_path):
    """include/moe_w8a8.h compiles as strict C99, and a C program links the
    library and calls its host-side entry points (workspace size, error
    strings), with the answers the Python binding gets."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(m.LIB_PATH)
    src = tmp_path / "client.c"
    src.write_text(
        "#include <stdio.h>\n#include \"moe_w8a8.h\"\n"
        "int main(void) {\n"
        "  moe_w8a8_dims d = {4096, 1536, 64, 8};\n"
        "  printf(\"%zu\\n%s\\n\", moe_w8a8_workspace_size(&d, 32),\n"
        "         moe_w8a8_strerror(MOE_W8A8_ERR_WORKSPACE));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "client"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(root, "include"), str(src), "-L", libdir, "-lmoe_w8a8",
                    "-Wl,-rpath," + libdir, "-o", str(exe)], check=True, timeout=120)
    r = subprocess.run([str(exe)], capture_output=True, text=True, check=True, timeout=60)
    ws, msg = r.stdout.splitlines()
    assert int(ws) == m.moe_w8a8_workspace_size(m.dims(4096, 1536, 64, 8), 32) > 0
    assert msg == m.moe_w8a8_strerror(m.MOE_W8A8_ERR_WORKSPACE)


def test_misaligned_pointers_refused(lib):
    """Each entry point refuses a device pointer below the alignment its kernels
    rely on (the header's rule) with MOE_W8A8_ERR_INVALID, before any launch."""
    d = m.dims(256, 512, 8, 2)
    for kw in (dict(x=FAKE + 8), dict(out=FAKE + 4), dict(logits=FAKE + 2),
               dict(ws=FAKE + 128)):
        assert _fwd(d, **kw) == m.MOE_W8A8_ERR_INVALID, kw
    assert _fwd(d, logits=None, ids=FAKE + 2, w=FAKE) == m.MOE_W8A8_ERR_INVALID
    assert _fwd(d, logits=None, ids=FAKE, w=FAKE + 1) == m.MOE_W8A8_ERR_INVALID
    for field, off in (("w_gate_up", 8), ("w_down", 4), ("inv_smooth", 8), ("s_gate_up", 2),
                       ("s_down", 1), ("act_clip", 2), ("w_router", 8)):
        wt = _weights()
        setattr(wt, field, FAKE + off)
        assert _fwd(d, weights=wt) == m.MOE_W8A8_ERR_INVALID, field
    dbg = m.moe_w8a8_debug()
    dbg.acc1 = FAKE + 4
    assert _fwd(d, dbg=dbg) == m.MOE_W8A8_ERR_INVALID
    dbg = m.moe_w8a8_debug()
    dbg.row_of = FAKE + 2
    assert _fwd(d, dbg=dbg) == m.MOE_W8A8_ERR_INVALID
    # the same checks come before the no-allocation forward touches the GPU
    assert lib.moe_w8a8_forward_noalloc(ctypes.byref(d), ctypes.byref(_weights()), FAKE + 8, 4,
                                        FAKE, None, None, 0.0, FAKE, None,
                                        None) == m.MOE_W8A8_ERR_INVALID
    # calibrate, its clip and the router projection
    w = _weights()
    assert lib.moe_w8a8_calibrate(ctypes.byref(d), 0.6, FAKE + 1, 4, FAKE, FAKE, FAKE,
                                  ctypes.byref(w), FAKE, 1 << 40, None) == m.MOE_W8A8_ERR_INVALID
    assert lib.moe_w8a8_calibrate(ctypes.byref(d), 0.6, FAKE, 4, FAKE + 2, FAKE, FAKE,
                                  ctypes.byref(w), FAKE, 1 << 40, None) == m.MOE_W8A8_ERR_INVALID
    assert lib.moe_w8a8_calibrate(ctypes.byref(d), 0.6, FAKE, 4, FAKE, FAKE, FAKE,
                                  ctypes.byref(w), FAKE + 64, 1 << 40,
                                  None) == m.MOE_W8A8_ERR_INVALID
    wq = _weights()
    wq.w_gate_up = FAKE + 4
    assert lib.moe_w8a8_calibrate(ctypes.byref(d), 0.6, FAKE, 4, FAKE, FAKE, FAKE,
                                  ctypes.byref(wq), FAKE, 1 << 40, None) == m.MOE_W8A8_ERR_INVALID
    assert lib.moe_w8a8_calibrate_clip(ctypes.byref(d), 99.0, FAKE + 1, 4, FAKE, FAKE,
                                       None) == m.MOE_W8A8_ERR_INVALID
    assert lib.moe_w8a8_calibrate_clip(ctypes.byref(d), 99.0, FAKE, 4, FAKE, FAKE + 2,
                                       None) == m.MOE_W8A8_ERR_INVALID
    dr = m.dims(1024, 512, 8, 2)
    assert lib.moe_w8a8_router_logits(ctypes.byref(dr), FAKE + 8, 4, FAKE, FAKE, FAKE, 1 << 40,
                                      None) == m.MOE_W8A8_ERR_INVALID
    assert lib.moe_w8a8_router_logits(ctypes.byref(dr), FAKE, 4, FAKE + 8, FAKE, FAKE, 1 << 40,
                                      None) == m.MOE_W8A8_ERR_INVALID
