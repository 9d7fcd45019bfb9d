"""CPU oracle of the W8A8 MoE expert layer (test infrastructure only).

This package wraps ``moe_oracle.c`` -- the plain, slow, obviously correct CPU
definition of the layer -- for the tests, the smoke check and the benchmark's
CPU-baseline leg. Nothing on the product path imports it, and it imports
nothing from the product package. All arrays are host numpy arrays; weights
are in the plain row-major layouts described in ``moe_oracle.c``.

The functions here only marshal arguments; every step is computed in C.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libmoe_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-Wno-unknown-pragmas", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # The sanitizer test runs the pins against an instrumented build of the
    # same source, named by this variable.
    path = os.environ.get("MOE_ORACLE_LIB")
    if not path:
        path = _LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(force=True)
    lib = ctypes.CDLL(path)
    sig = {
        "oracle_f64_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
        "oracle_quant_rows": (None, [_I64, _I64, _P, _P, _P]),
        "oracle_quant_rows_fmt": (None, [_I64, _I64, _P, _I32, _P, _P]),
        "oracle_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
        "oracle_e4m3_code": (ctypes.c_uint8, [_F32]),
        "oracle_calibrate": (ctypes.c_int, [_I32, _I32, _I32, _F32, _P, _I64, _P, _P, _P,
                                            _P, _P, _P, _P, _P, _P, _P, _I32]),
        "oracle_route": (None, [_I64, _I32, _I32, _P, _P, _P]),
        "oracle_router_logits": (None, [_I64, _I32, _I32, _P, _P, _P]),
        "oracle_capacity": (_I64, [_F32, _I64, _I32, _I32]),
        "oracle_permute": (_I64, [_I64, _I32, _I32, _P, _I64, _P, _P, _P, _P]),
        "oracle_act_quant": (None, [_I64, _I32, _P, _P, _P, _P]),
        "oracle_act_quant_clip": (None, [_I64, _I32, _P, _P, _F32, _F32, _I32, _P, _P]),
        "oracle_clip_threshold": (_F32, [_I64, _I32, _P, _P, _F32]),
        "oracle_percentile_rank": (_I64, [ctypes.c_double, _I64]),
        "oracle_expert_rows": (None, [_I64, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                      _P, _P, _I32, _P, _P, _P, _P, _P, _P]),
        "oracle_combine": (None, [_I64, _P, _I32, _I32, _P, _P, _P, _P, _P, _P]),
        "oracle_forward": (_I64, [_I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _F32,
                                  _P, _P, _P, _P, _P, _F32, _F32, _I32,
                                  _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P]),
        "oracle_num_threads": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def f64_to_bf16(v: float) -> int:
    """Round a float to bfloat16 bits (ties to even, one rounding)."""
    return int(_load().oracle_f64_to_bf16(float(v)))


def quant_rows(v: np.ndarray):
    """Symmetric per-row INT8 quantiser (fp32 rule). v: float32 [rows][n]."""
    v = _c(v, np.float32)
    rows, n = v.shape
    q = np.empty((rows, n), np.int8)
    s = np.empty(rows, np.float32)
    _load().oracle_quant_rows(rows, n, _ptr(v), _ptr(q), _ptr(s))
    return q, s


FMT_INT8, FMT_FP8 = 0, 1


def quant_rows_fmt(v: np.ndarray, fmt: int):
    """Row quantiser of either format; v float32 [rows][n]."""
    v = _c(v, np.float32)
    rows, n = v.shape
    q = np.empty((rows, n), np.int8)
    s = np.empty(rows, np.float32)
    _load().oracle_quant_rows_fmt(rows, n, _ptr(v), int(fmt), _ptr(q), _ptr(s))
    return q, s


def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(int(code) & 0xFF))


def e4m3_code(t: float) -> int:
    """Code of a value already inside [-448, 448]."""
    return int(_load().oracle_e4m3_code(float(np.float32(t))))


def calibrate(calib_x_bf16, w_gate, w_up, w_down, alpha: float, want_smoothed: bool = False,
              fmt: int = FMT_INT8):
    """SmoothQuant calibration + per-output-channel weight quantisation
    (INT8 codes, or FP8 e4m3 codes with fmt = FMT_FP8).

    calib_x_bf16: uint16 [Nc][H]; w_gate, w_up: float32 [E][F][H];
    w_down: float32 [E][H][F]. Returns a dict with s, inv_s [H], q_gu int8
    [E][2F][H], sw_gu [E][2F], q_d int8 [E][H][F], sw_d [E][H] (and ws_gu,
    the smoothed fp32 gate/up weights, when asked)."""
    cx = _c(calib_x_bf16, np.uint16)
    wg, wu, wd = _c(w_gate, np.float32), _c(w_up, np.float32), _c(w_down, np.float32)
    E, F, H = wg.shape
    assert wu.shape == (E, F, H) and wd.shape == (E, H, F) and cx.shape[1] == H
    out = dict(s=np.empty(H, np.float32), inv_s=np.empty(H, np.float32),
               q_gu=np.empty((E, 2 * F, H), np.int8), sw_gu=np.empty((E, 2 * F), np.float32),
               q_d=np.empty((E, H, F), np.int8), sw_d=np.empty((E, H), np.float32))
    if want_smoothed:
        out["ws_gu"] = np.empty((E, 2 * F, H), np.float32)
    rc = _load().oracle_calibrate(H, F, E, float(alpha), _ptr(cx), cx.shape[0],
                                  _ptr(wg), _ptr(wu), _ptr(wd), _ptr(out["s"]), _ptr(out["inv_s"]),
                                  _ptr(out["q_gu"]), _ptr(out["sw_gu"]), _ptr(out["q_d"]),
                                  _ptr(out["sw_d"]), _ptr(out.get("ws_gu")), int(fmt))
    if rc != 0:
        raise ValueError("oracle_calibrate failed: %d" % rc)
    return out


def route(logits, k: int):
    """Top-k routing; logits float32 [T][E] -> ids int32 [T][k], w float32 [T][k]."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().oracle_route(T, E, k, _ptr(lg), _ptr(ids), _ptr(w))
    return ids, w


def router_logits(x_bf16, w_router_bf16):
    """Router projection in fp64; x uint16 (bf16) [T][H], w uint16 (bf16)
    [E][H] -> float64 [T][E]."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_router_bf16, np.uint16)
    T, H = x.shape
    E = w.shape[0]
    assert w.shape[1] == H
    out = np.empty((T, E), np.float64)
    _load().oracle_router_logits(T, H, E, _ptr(x), _ptr(w), _ptr(out))
    return out


def capacity(cf: float, T: int, k: int, E: int) -> int:
    return int(_load().oracle_capacity(float(cf), T, k, E))


def permute(ids, E: int, cap: int):
    """Stable grouping by expert with capacity; ids int32 [T][k]."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    A = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_ = np.full(max(A, 1), -1, np.int32)
    row_of = np.empty(max(A, 1), np.int32)
    kept = _load().oracle_permute(T, E, k, _ptr(ids), cap, _ptr(counts), _ptr(offsets),
                                  _ptr(sorted_), _ptr(row_of))
    return dict(counts=counts, offsets=offsets, sorted=sorted_[:kept].copy(),
                row_of=row_of[:A].reshape(T, k), kept=int(kept))


def act_quant(x_bf16, inv_s, clip: float = 0.0, sat_percentile: float = 0.0,
              fmt: int = FMT_INT8):
    """Per-token smoothed INT8 quantisation; x uint16 [T][H] -> qx int8, sx f32 [T].
    clip > 0: static clipping threshold; sat_percentile in (0, 100]: dynamic
    per-token saturation at that percentile of |x * inv_s|."""
    x = _c(x_bf16, np.uint16)
    inv_s = _c(inv_s, np.float32)
    T, H = x.shape
    qx = np.empty((T, H), np.int8)
    sx = np.empty(T, np.float32)
    _load().oracle_act_quant_clip(T, H, _ptr(x), _ptr(inv_s), float(clip),
                                  float(np.float32(sat_percentile)), int(fmt), _ptr(qx), _ptr(sx))
    return qx, sx


def clip_threshold(calib_x_bf16, inv_s, percentile: float) -> np.float32:
    """Static clipping threshold: nearest-rank percentile of |x * inv_s| over
    every calibration entry."""
    x = _c(calib_x_bf16, np.uint16)
    inv_s = _c(inv_s, np.float32)
    n, H = x.shape
    return np.float32(_load().oracle_clip_threshold(n, H, _ptr(x), _ptr(inv_s),
                                                    float(np.float32(percentile))))


def percentile_rank(p: float, N: int) -> int:
    """1-based rank of the nearest-rank percentile p (float32 p, as the ABI)."""
    return int(_load().oracle_percentile_rank(float(np.float32(p)), int(N)))


def expert_rows(rows, ids, sorted_, qx, sx, cal, want_acc1: bool = True, want_h: bool = True,
                fmt: int = FMT_INT8):
    """Expert FFN for the permuted rows listed in `rows` (sorted positions).
    acc1 is int32 for INT8 codes and the exact fp64 sums for FP8 codes."""
    rows = _c(rows, np.int32)
    ids = _c(ids, np.int32)
    T, k = ids.shape
    sorted_ = _c(sorted_, np.int32)
    qx, sx = _c(qx, np.int8), _c(sx, np.float32)
    q_gu, sw_gu = _c(cal["q_gu"], np.int8), _c(cal["sw_gu"], np.float32)
    q_d, sw_d = _c(cal["q_d"], np.int8), _c(cal["sw_d"], np.float32)
    E, F2, H = q_gu.shape
    F = F2 // 2
    n = rows.shape[0]
    acc1 = np.empty((n, 2 * F), np.int32) if want_acc1 and fmt == FMT_INT8 else None
    acc1f = np.empty((n, 2 * F), np.float64) if want_acc1 and fmt == FMT_FP8 else None
    h = np.empty((n, F), np.float32) if want_h else None
    qh = np.empty((n, F), np.int8)
    sh = np.empty(n, np.float32)
    y = np.empty((n, H), np.float64)
    _load().oracle_expert_rows(n, _ptr(rows), H, F, k, _ptr(ids), _ptr(sorted_), _ptr(qx), _ptr(sx),
                               _ptr(q_gu), _ptr(sw_gu), _ptr(q_d), _ptr(sw_d), int(fmt),
                               _ptr(acc1), _ptr(acc1f), _ptr(h), _ptr(qh), _ptr(sh), _ptr(y))
    return dict(acc1=acc1 if fmt == FMT_INT8 else acc1f, h=h, qh=qh, sh=sh, y=y)


def combine(tokens, w, row_of, y, y_row_index=None, want_exact: bool = False):
    """Gate-weighted sum for the listed tokens; returns bf16 bits [n][H], or
    (bits, the fp64 sums before rounding) with want_exact."""
    w = _c(w, np.float32)
    T, k = w.shape
    row_of = _c(row_of, np.int32)
    y = _c(y, np.float64)
    H = y.shape[1]
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else tok.shape[0]
    yri = None if y_row_index is None else _c(y_row_index, np.int64)
    out = np.empty((n, H), np.uint16)
    exact = np.empty((n, H), np.float64) if want_exact else None
    _load().oracle_combine(n, _ptr(tok), H, k, _ptr(w), _ptr(row_of), _ptr(yri), _ptr(y), _ptr(out),
                           _ptr(exact))
    return (out, exact) if want_exact else out


def forward(x_bf16, cal, k: int, logits=None, ids=None, w=None, capacity_factor: float = 0.0,
            want_acc1: bool = True, want_h: bool = True, clip: float = 0.0,
            sat_percentile: float = 0.0, fmt: int = FMT_INT8):
    """The whole layer on the CPU. Returns a dict of every stage's output
    ("out_exact": the combine's fp64 sums before the rounding to bf16)."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    q_gu, sw_gu = _c(cal["q_gu"], np.int8), _c(cal["sw_gu"], np.float32)
    q_d, sw_d = _c(cal["q_d"], np.int8), _c(cal["sw_d"], np.float32)
    inv_s = _c(cal["inv_s"], np.float32)
    E, F2, _ = q_gu.shape
    F = F2 // 2
    A = T * k
    lg = None if logits is None else _c(logits, np.float32)
    ids_in = None if ids is None else _c(ids, np.int32)
    w_in = None if w is None else _c(w, np.float32)
    if lg is None:
        assert ids_in is not None and w_in is not None
    o = dict(ids=np.empty((T, k), np.int32), w=np.empty((T, k), np.float32),
             counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
             sorted=np.full(max(A, 1), -1, np.int32), row_of=np.empty((T, k), np.int32),
             qx=np.empty((T, H), np.int8), sx=np.empty(T, np.float32),
             acc1=np.empty((A, 2 * F), np.int32) if want_acc1 and fmt == FMT_INT8 else None,
             acc1f=np.empty((A, 2 * F), np.float64) if want_acc1 and fmt == FMT_FP8 else None,
             h=np.empty((A, F), np.float32) if want_h else None,
             qh=np.empty((max(A, 1), F), np.int8), sh=np.empty(max(A, 1), np.float32),
             y=np.empty((max(A, 1), H), np.float64), out=np.empty((T, H), np.uint16),
             out_exact=np.empty((T, H), np.float64))
    kept = _load().oracle_forward(
        T, H, F, E, k, _ptr(x), _ptr(lg), _ptr(ids_in), _ptr(w_in), float(capacity_factor),
        _ptr(q_gu), _ptr(sw_gu), _ptr(q_d), _ptr(sw_d), _ptr(inv_s), float(clip),
        float(np.float32(sat_percentile)), int(fmt), _ptr(o["ids"]), _ptr(o["w"]),
        _ptr(o["counts"]), _ptr(o["offsets"]), _ptr(o["sorted"]), _ptr(o["row_of"]), _ptr(o["qx"]),
        _ptr(o["sx"]), _ptr(o["acc1"]), _ptr(o["acc1f"]), _ptr(o["h"]), _ptr(o["qh"]),
        _ptr(o["sh"]), _ptr(o["y"]), _ptr(o["out"]), _ptr(o["out_exact"]))
    kept = int(kept)
    o["kept"] = kept
    o["sorted"] = o["sorted"][:kept]
    o["qh"], o["sh"], o["y"] = o["qh"][:kept], o["sh"][:kept], o["y"][:kept]
    if fmt == FMT_FP8:
        o["acc1"] = o.pop("acc1f")
    else:
        o.pop("acc1f")
    if o["acc1"] is not None:
        o["acc1"] = o["acc1"][:kept]
    if o["h"] is not None:
        o["h"] = o["h"][:kept]
    return o
