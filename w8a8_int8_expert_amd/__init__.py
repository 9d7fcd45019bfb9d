"""Python binding of libmoe_w8a8 (the W8A8 MoE expert layer for MI355X).

The functions named like the C entry points (moe_w8a8_forward, ...) only
marshal arguments to the shared library; every step of the layer runs in its
HIP kernels. PyTorch supplies device memory and the current stream. The
binding refuses to run without the built library: there is no fallback.

`MoEW8A8` is convenience plumbing on top: it allocates the quantised weights
and a workspace with torch and calls the entry points on the current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w8a8.so")

MOE_W8A8_OK = 0
MOE_W8A8_ERR_INVALID = -1
MOE_W8A8_ERR_UNSUPPORTED = -2
MOE_W8A8_ERR_WORKSPACE = -3
MOE_W8A8_ERR_HIP = -4
MOE_W8A8_ERR_SCRATCH = -5
MOE_W8A8_SCRATCH_BYTES = 64 << 20
MOE_W8A8_FORMAT_INT8 = 0
MOE_W8A8_FORMAT_FP8 = 1

_P = ctypes.c_void_p


class moe_w8a8_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class moe_w8a8_weights(ctypes.Structure):
    _fields_ = [("w_gate_up", _P), ("w_down", _P), ("s_gate_up", _P), ("s_down", _P),
                ("smooth", _P), ("inv_smooth", _P), ("w_router", _P), ("act_clip", _P),
                ("act_sat_percentile", ctypes.c_float), ("format", ctypes.c_int32)]


class moe_w8a8_debug(ctypes.Structure):
    _fields_ = [("topk_ids", _P), ("topk_w", _P), ("expert_counts", _P), ("expert_offsets", _P),
                ("sorted_assign", _P), ("row_of", _P), ("qx", _P), ("sx", _P), ("acc1", _P),
                ("h", _P), ("qh", _P), ("sh", _P), ("y", _P), ("gemm_path", ctypes.c_int32),
                ("stage_events", ctypes.POINTER(_P)), ("router_logits", _P)]

STAGES = ("route", "scan", "scatter", "act_quant", "gemm1", "requant", "gemm2", "combine",
          "router")


EXPORTS = ("moe_w8a8_workspace_size", "moe_w8a8_calibrate", "moe_w8a8_calibrate_clip",
           "moe_w8a8_forward", "moe_w8a8_forward_noalloc", "moe_w8a8_router_logits",
           "moe_w8a8_pack", "moe_w8a8_strerror")

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmoe_w8a8.so; raises if it has not been built.

    torch is imported first: the binding hands the library torch's device
    memory and streams, so the library must run on torch's HIP runtime. Its
    dependency on libamdhip64.so.7 then resolves to the runtime torch already
    loaded (same soname); loaded the other way round, the process would hold
    two HIP runtimes, and the one initialised second finds no device."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmoe_w8a8.so is not built (%s); run "
                           "`python -m w8a8_int8_expert_amd.build`" % path)
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    D, W, G = ctypes.POINTER(moe_w8a8_dims), ctypes.POINTER(moe_w8a8_weights), \
        ctypes.POINTER(moe_w8a8_debug)
    lib.moe_w8a8_workspace_size.restype = ctypes.c_size_t
    lib.moe_w8a8_workspace_size.argtypes = [D, ctypes.c_int64]
    lib.moe_w8a8_calibrate.restype = ctypes.c_int
    lib.moe_w8a8_calibrate.argtypes = [D, ctypes.c_float, _P, ctypes.c_int64, _P, _P, _P, W,
                                       _P, ctypes.c_size_t, _P]
    lib.moe_w8a8_forward.restype = ctypes.c_int
    lib.moe_w8a8_forward.argtypes = [D, W, _P, ctypes.c_int64, _P, _P, _P, ctypes.c_float, _P,
                                     _P, ctypes.c_size_t, G, _P]
    lib.moe_w8a8_forward_noalloc.restype = ctypes.c_int
    lib.moe_w8a8_forward_noalloc.argtypes = [D, W, _P, ctypes.c_int64, _P, _P, _P,
                                             ctypes.c_float, _P, G, _P]
    lib.moe_w8a8_calibrate_clip.restype = ctypes.c_int
    lib.moe_w8a8_calibrate_clip.argtypes = [D, ctypes.c_float, _P, ctypes.c_int64, _P, _P, _P]
    lib.moe_w8a8_router_logits.restype = ctypes.c_int
    lib.moe_w8a8_router_logits.argtypes = [D, _P, ctypes.c_int64, _P, _P, _P, ctypes.c_size_t,
                                           _P]
    lib.moe_w8a8_pack.restype = ctypes.c_int
    lib.moe_w8a8_pack.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
    lib.moe_w8a8_strerror.restype = ctypes.c_char_p
    lib.moe_w8a8_strerror.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    """Device address of a tensor (or pass an int / None through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dims(hidden: int, ffn: int, num_experts: int, top_k: int) -> moe_w8a8_dims:
    return moe_w8a8_dims(hidden, ffn, num_experts, top_k)


def moe_w8a8_strerror(code: int) -> str:
    return load_library().moe_w8a8_strerror(code).decode()


def moe_w8a8_workspace_size(d: moe_w8a8_dims, T: int) -> int:
    return int(load_library().moe_w8a8_workspace_size(ctypes.byref(d), T))


def moe_w8a8_calibrate(d, alpha, calib_x, n_calib, w_gate, w_up, w_down, out: moe_w8a8_weights,
                       workspace, workspace_bytes, stream=None) -> int:
    return int(load_library().moe_w8a8_calibrate(
        ctypes.byref(d), float(alpha), _ptr(calib_x), int(n_calib), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), ctypes.byref(out), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def moe_w8a8_forward(d, weights: moe_w8a8_weights, x, T, router_logits, topk_ids, topk_w,
                     capacity_factor, out, workspace, workspace_bytes,
                     debug: Optional[moe_w8a8_debug] = None, stream=None) -> int:
    return int(load_library().moe_w8a8_forward(
        ctypes.byref(d), ctypes.byref(weights), _ptr(x), int(T), _ptr(router_logits),
        _ptr(topk_ids), _ptr(topk_w), float(capacity_factor), _ptr(out), _ptr(workspace),
        int(workspace_bytes), ctypes.byref(debug) if debug is not None else None,
        _stream(stream)))


def moe_w8a8_forward_noalloc(d, weights: moe_w8a8_weights, x, T, router_logits, topk_ids, topk_w,
                             capacity_factor, out, debug: Optional[moe_w8a8_debug] = None,
                             stream=None) -> int:
    return int(load_library().moe_w8a8_forward_noalloc(
        ctypes.byref(d), ctypes.byref(weights), _ptr(x), int(T), _ptr(router_logits),
        _ptr(topk_ids), _ptr(topk_w), float(capacity_factor), _ptr(out),
        ctypes.byref(debug) if debug is not None else None, _stream(stream)))


def moe_w8a8_calibrate_clip(d, percentile, calib_x, n_calib, inv_smooth, act_clip,
                            stream=None) -> int:
    return int(load_library().moe_w8a8_calibrate_clip(
        ctypes.byref(d), float(percentile), _ptr(calib_x), int(n_calib), _ptr(inv_smooth),
        _ptr(act_clip), _stream(stream)))


def moe_w8a8_router_logits(d, x, T, w_router, logits, workspace, workspace_bytes,
                           stream=None) -> int:
    return int(load_library().moe_w8a8_router_logits(
        ctypes.byref(d), _ptr(x), int(T), _ptr(w_router), _ptr(logits), _ptr(workspace),
        int(workspace_bytes), _stream(stream)))


def moe_w8a8_pack(count, N, K, src, dst, stream=None) -> int:
    return int(load_library().moe_w8a8_pack(int(count), int(N), int(K), _ptr(src), _ptr(dst),
                                             _stream(stream)))


class MoEW8A8Error(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != MOE_W8A8_OK:
        raise MoEW8A8Error("%s failed: %s (%d)" % (what, moe_w8a8_strerror(rc), rc))


class MoEW8A8:
    """Quantised layer on one device (torch tensors for memory and streams).
    Every library call is made with the layer's device current, on torch's
    current stream of that device, whichever device was current before.
    The layer owns one workspace, allocated on the stream current at its first
    use and replaced when a larger batch needs more: calls on one layer must
    not overlap on different streams (give each stream a layer of its own, or
    synchronise between the streams)."""

    def __init__(self, hidden: int, ffn: int, num_experts: int, top_k: int, device="cuda",
                 fp8: bool = False):
        import torch
        load_library()
        self.d = dims(hidden, ffn, num_experts, top_k)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        H, F, E = hidden, ffn, num_experts
        kw = dict(device=self.device)
        self.w_gate_up = torch.empty(E * 2 * F * H, dtype=torch.int8, **kw)
        self.w_down = torch.empty(E * H * F, dtype=torch.int8, **kw)
        self.s_gate_up = torch.empty(E, 2 * F, dtype=torch.float32, **kw)
        self.s_down = torch.empty(E, H, dtype=torch.float32, **kw)
        self.smooth = torch.empty(H, dtype=torch.float32, **kw)
        self.inv_smooth = torch.empty(H, dtype=torch.float32, **kw)
        self.weights = moe_w8a8_weights(*(t.data_ptr() for t in (
            self.w_gate_up, self.w_down, self.s_gate_up, self.s_down, self.smooth,
            self.inv_smooth)), None, None, 0.0,
            MOE_W8A8_FORMAT_FP8 if fp8 else MOE_W8A8_FORMAT_INT8)
        self.w_router = None
        self.act_clip = torch.zeros(1, dtype=torch.float32, **kw)
        self._ws = None

    def _on_device(self):
        """Context in which the layer's device is current: the library launches
        on the current device, on torch's current stream of that device."""
        import torch
        return torch.cuda.device(self.device)

    def _expect(self, t, name, dtype, shape):
        """Raise MoEW8A8Error unless t is a contiguous tensor of this dtype and
        shape on the layer's device (the C ABI reads raw pointers)."""
        import torch
        if not isinstance(t, torch.Tensor):
            raise MoEW8A8Error("%s must be a torch tensor" % name)
        if t.dtype != dtype:
            raise MoEW8A8Error("%s must be %s, got %s" % (name, dtype, t.dtype))
        if tuple(t.shape) != tuple(shape):
            raise MoEW8A8Error("%s must have shape %s, got %s" % (name, tuple(shape),
                                                                   tuple(t.shape)))
        if not t.is_contiguous():
            raise MoEW8A8Error("%s must be contiguous" % name)
        if t.device != self.device:
            raise MoEW8A8Error("%s must be on %s, got %s" % (name, self.device, t.device))

    def calibrate_clip(self, calib_x, percentile: float):
        """Static activation clip at the percentile of the calibration tokens'
        smoothed values (after calibrate); forward then uses it."""
        import torch
        self._expect(calib_x, "calib_x", torch.bfloat16, (calib_x.shape[0], self.d.hidden))
        with self._on_device():
            _check(moe_w8a8_calibrate_clip(self.d, percentile, calib_x, calib_x.shape[0],
                                           self.inv_smooth, self.act_clip),
                   "moe_w8a8_calibrate_clip")
        self.weights.act_clip = self.act_clip.data_ptr()

    def set_clip(self, static: bool = False, sat_percentile: float = 0.0):
        """Use (or not) the static clip, and the dynamic saturation percentile
        (0 = off)."""
        self.weights.act_clip = self.act_clip.data_ptr() if static else None
        self.weights.act_sat_percentile = float(sat_percentile)

    def set_router(self, w_router):
        """bf16 [E][H] router matrix (kept on the device; copied), or None."""
        import torch
        if w_router is None:
            self.w_router = None
            self.weights.w_router = None
            return
        H, E = self.d.hidden, self.d.num_experts
        if tuple(w_router.shape) != (E, H) or w_router.dtype != torch.bfloat16:
            raise MoEW8A8Error("router matrix must be bf16 [E][H]")
        self.w_router = w_router.to(self.device).contiguous().clone()
        self.weights.w_router = self.w_router.data_ptr()

    def router_logits(self, x, out=None):
        """fp32 [T][E] logits x . w_router^T (needs set_router)."""
        import torch
        if self.w_router is None:
            raise MoEW8A8Error("no router matrix (set_router)")
        T = x.shape[0]
        self._expect(x, "x", torch.bfloat16, (T, self.d.hidden))
        if out is None:
            out = torch.empty(T, self.d.num_experts, dtype=torch.float32, device=self.device)
        self._expect(out, "out", torch.float32, (T, self.d.num_experts))
        ws = self.workspace(T)
        with self._on_device():
            _check(moe_w8a8_router_logits(self.d, x, T, self.w_router, out, ws, ws.numel()),
                   "moe_w8a8_router_logits")
        return out

    def load_quantized(self, q_gate_up, s_gate_up, q_down, s_down, smooth, inv_smooth):
        """Load weights quantised elsewhere: row-major codes q_gate_up int8
        [E][2F][H] (gate rows, then up rows) and q_down int8 [E][H][F] (INT8 or
        e4m3 bytes, in the layer's format), packed on the device by
        moe_w8a8_pack; scales s_gate_up fp32 [E][2F], s_down fp32 [E][H];
        smooth and inv_smooth fp32 [H]. Every tensor on the layer's device."""
        import torch
        H, F, E = self.d.hidden, self.d.ffn, self.d.num_experts
        self._expect(q_gate_up, "q_gate_up", torch.int8, (E, 2 * F, H))
        self._expect(q_down, "q_down", torch.int8, (E, H, F))
        self._expect(s_gate_up, "s_gate_up", torch.float32, (E, 2 * F))
        self._expect(s_down, "s_down", torch.float32, (E, H))
        self._expect(smooth, "smooth", torch.float32, (H,))
        self._expect(inv_smooth, "inv_smooth", torch.float32, (H,))
        with self._on_device():
            _check(moe_w8a8_pack(E, 2 * F, H, q_gate_up, self.w_gate_up), "moe_w8a8_pack")
            _check(moe_w8a8_pack(E, H, F, q_down, self.w_down), "moe_w8a8_pack")
        self.s_gate_up.copy_(s_gate_up)
        self.s_down.copy_(s_down)
        self.smooth.copy_(smooth)
        self.inv_smooth.copy_(inv_smooth)

    def workspace(self, T: int):
        import torch
        need = moe_w8a8_workspace_size(self.d, T)
        if need == 0:
            raise MoEW8A8Error("unsupported dims or T")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def calibrate(self, calib_x, w_gate, w_up, w_down, alpha: float):
        """calib_x: bf16 [Nc][H]; w_gate, w_up: f32 [E][F][H]; w_down: f32 [E][H][F]."""
        import torch
        H, F, E = self.d.hidden, self.d.ffn, self.d.num_experts
        self._expect(calib_x, "calib_x", torch.bfloat16, (calib_x.shape[0], H))
        self._expect(w_gate, "w_gate", torch.float32, (E, F, H))
        self._expect(w_up, "w_up", torch.float32, (E, F, H))
        self._expect(w_down, "w_down", torch.float32, (E, H, F))
        ws = self.workspace(0)
        with self._on_device():
            _check(moe_w8a8_calibrate(self.d, alpha, calib_x, calib_x.shape[0], w_gate, w_up,
                                      w_down, self.weights, ws, ws.numel()), "moe_w8a8_calibrate")

    def forward(self, x, router_logits=None, topk_ids=None, topk_w=None,
                capacity_factor: float = 0.0, out=None, debug: Optional[moe_w8a8_debug] = None):
        """x: bf16 [T][H] -> bf16 [T][H]. Routing: router_logits, or (topk_ids,
        topk_w), or neither with a router matrix set (set_router)."""
        import torch
        T = x.shape[0]
        out = self._check_forward_args(x, router_logits, topk_ids, topk_w, out)
        ws = self.workspace(T)
        with self._on_device():
            _check(moe_w8a8_forward(self.d, self.weights, x, T, router_logits, topk_ids, topk_w,
                                    capacity_factor, out, ws, ws.numel(), debug),
                   "moe_w8a8_forward")
        return out

    def forward_noalloc(self, x, out, router_logits=None, topk_ids=None, topk_w=None,
                        capacity_factor: float = 0.0, debug: Optional[moe_w8a8_debug] = None):
        """forward into a caller-given out, with the library's static scratch
        as workspace (moe_w8a8_forward_noalloc): nothing is allocated."""
        T = x.shape[0]
        if out is None:
            raise MoEW8A8Error("forward_noalloc needs a caller-given out tensor")
        out = self._check_forward_args(x, router_logits, topk_ids, topk_w, out)
        with self._on_device():
            _check(moe_w8a8_forward_noalloc(self.d, self.weights, x, T, router_logits, topk_ids,
                                            topk_w, capacity_factor, out, debug),
                   "moe_w8a8_forward_noalloc")
        return out

    def _check_forward_args(self, x, router_logits, topk_ids, topk_w, out):
        import torch
        H, E, k = self.d.hidden, self.d.num_experts, self.d.top_k
        T = x.shape[0]
        self._expect(x, "x", torch.bfloat16, (T, H))
        if router_logits is not None:
            self._expect(router_logits, "router_logits", torch.float32, (T, E))
        if topk_ids is not None:
            self._expect(topk_ids, "topk_ids", torch.int32, (T, k))
        if topk_w is not None:
            self._expect(topk_w, "topk_w", torch.float32, (T, k))
        if out is None:
            out = torch.empty(T, H, dtype=torch.bfloat16, device=self.device)
        self._expect(out, "out", torch.bfloat16, (T, H))
        return out
