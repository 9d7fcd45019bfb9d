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
           "moe_w8a8_forward", "moe_w8a8_router_logits", "moe_w8a8_strerror")

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmoe_w8a8.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmoe_w8a8.so is not built (%s); run "
                           "`python -m w8a8_int8_expert_amd.build`" % path)
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
    lib.moe_w8a8_calibrate_clip.restype = ctypes.c_int
    lib.moe_w8a8_calibrate_clip.argtypes = [D, ctypes.c_float, _P, ctypes.c_int64, _P, _P, _P]
    lib.moe_w8a8_router_logits.restype = ctypes.c_int
    lib.moe_w8a8_router_logits.argtypes = [D, _P, ctypes.c_int64, _P, _P, _P, ctypes.c_size_t,
                                           _P]
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


class MoEW8A8Error(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != MOE_W8A8_OK:
        raise MoEW8A8Error("%s failed: %s (%d)" % (what, moe_w8a8_strerror(rc), rc))


class MoEW8A8:
    """Quantised layer on one device (torch tensors for memory and streams)."""

    def __init__(self, hidden: int, ffn: int, num_experts: int, top_k: int, device="cuda",
                 fp8: bool = False):
        import torch
        load_library()
        self.d = dims(hidden, ffn, num_experts, top_k)
        self.device = torch.device(device)
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

    def calibrate_clip(self, calib_x, percentile: float):
        """Static activation clip at the percentile of the calibration tokens'
        smoothed values (after calibrate); forward then uses it."""
        _check(moe_w8a8_calibrate_clip(self.d, percentile, calib_x, calib_x.shape[0],
                                       self.inv_smooth, self.act_clip), "moe_w8a8_calibrate_clip")
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
        if out is None:
            out = torch.empty(T, self.d.num_experts, dtype=torch.float32, device=self.device)
        ws = self.workspace(T)
        _check(moe_w8a8_router_logits(self.d, x, T, self.w_router, out, ws, ws.numel()),
               "moe_w8a8_router_logits")
        return out

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
        ws = self.workspace(0)
        _check(moe_w8a8_calibrate(self.d, alpha, calib_x, calib_x.shape[0], w_gate, w_up, w_down,
                                  self.weights, ws, ws.numel()), "moe_w8a8_calibrate")

    def forward(self, x, router_logits=None, topk_ids=None, topk_w=None,
                capacity_factor: float = 0.0, out=None, debug: Optional[moe_w8a8_debug] = None):
        """x: bf16 [T][H] -> bf16 [T][H]. Routing: router_logits, or (topk_ids,
        topk_w), or neither with a router matrix set (set_router)."""
        import torch
        T = x.shape[0]
        if out is None:
            out = torch.empty(T, self.d.hidden, dtype=torch.bfloat16, device=self.device)
        ws = self.workspace(T)
        _check(moe_w8a8_forward(self.d, self.weights, x, T, router_logits, topk_ids, topk_w,
                                capacity_factor, out, ws, ws.numel(), debug), "moe_w8a8_forward")
        return out
