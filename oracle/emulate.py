"""Precision-emulating model of the flash and baseline attention algorithms --
TEST INFRASTRUCTURE ONLY (see emulate.c for the model and its source).

Formats are named "f64" (no rounding), "f32", "tf32", "f16", "bf16", or given
as a tuple (p, emin, emax); fmt_bits(p) is p significant bits with the
exponent range of fp32 and bf16 (the mantissa-width sweep).
"""
import ctypes

import numpy as np

from . import _load, _f64

FORMATS = {
    "f64": (0, 0, 0),
    "f32": (24, -126, 127),
    "tf32": (11, -126, 127),
    "f16": (11, -14, 15),
    "bf16": (8, -126, 127),
}


def fmt_bits(p):
    return (int(p), -126, 127)


class _Fmt(ctypes.Structure):
    _fields_ = [("p", ctypes.c_int), ("emin", ctypes.c_int), ("emax", ctypes.c_int)]


class _Cfg(ctypes.Structure):
    _fields_ = [("acc", _Fmt), ("pfmt", _Fmt), ("state", _Fmt), ("out", _Fmt),
                ("bc", ctypes.c_long), ("order", ctypes.c_int), ("kv_outer", ctypes.c_int)]


def _fmt(f):
    return _Fmt(*(FORMATS[f] if isinstance(f, str) else tuple(int(x) for x in f)))


_ready = False


def _lib():
    global _ready
    lib = _load()
    if not _ready:
        L, D, I = ctypes.c_long, ctypes.c_double, ctypes.c_int
        P = ctypes.POINTER
        lib.emu_round.argtypes = [D, I, I, I]
        lib.emu_round.restype = D
        lib.emu_flash_rows.argtypes = [P(D), P(D), P(D), L, L, L, L, D, I, P(_Cfg), P(L), L, P(D)]
        lib.emu_flash_rows.restype = I
        lib.emu_baseline_rows.argtypes = [P(D), P(D), P(D), L, L, L, L, D, I, P(_Fmt), P(_Fmt), P(_Fmt),
                                          P(L), L, P(D)]
        lib.emu_baseline_rows.restype = I
        _ready = True
    return lib


def round_fmt(x, fmt):
    """Element-wise rounding of float64 values to a format (slow; small arrays)."""
    f = FORMATS[fmt] if isinstance(fmt, str) else fmt
    lib = _lib()
    a = np.asarray(x, dtype=np.float64)
    return np.array([lib.emu_round(float(t), *f) for t in a.ravel()]).reshape(a.shape)


def _rows(rows):
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.ctypes.data_as(ctypes.POINTER(ctypes.c_long))


def flash_rows(q, k, v, scale, rows, causal=False, acc="f32", p="bf16", state="f32", out="f32",
               bc=64, order=0, kv_outer=False):
    """Emulated flash forward on selected rows; returns [len(rows), d]."""
    B, H, N, d = q.shape
    q, qp = _f64(q); k, kp = _f64(k); v, vp = _f64(v)
    r, rp = _rows(rows)
    o = np.zeros((r.size, d))
    cfg = _Cfg(_fmt(acc), _fmt(p), _fmt(state), _fmt(out), int(bc), int(order), int(bool(kv_outer)))
    rc = _lib().emu_flash_rows(qp, kp, vp, B, H, N, d, float(scale), int(bool(causal)), ctypes.byref(cfg),
                               rp, r.size, o.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc:
        raise ValueError("emu_flash_rows: bad arguments")
    return o


def baseline_rows(q, k, v, scale, rows, causal=False, acc="f32", store="bf16", out="f32"):
    """Emulated baseline attention (S and P stored in `store`) on selected rows."""
    B, H, N, d = q.shape
    q, qp = _f64(q); k, kp = _f64(k); v, vp = _f64(v)
    r, rp = _rows(rows)
    o = np.zeros((r.size, d))
    a, s, u = _fmt(acc), _fmt(store), _fmt(out)
    rc = _lib().emu_baseline_rows(qp, kp, vp, B, H, N, d, float(scale), int(bool(causal)), ctypes.byref(a),
                                  ctypes.byref(s), ctypes.byref(u), rp, r.size,
                                  o.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc:
        raise ValueError("emu_baseline_rows: bad arguments")
    return o
