"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  The HIP library never imports, links or calls it, and it
never imports anything from the HIP side.  See oracle.c for what each routine
computes and which passage of the pages it follows.

All arrays are numpy float64, C-contiguous; q, k, v are [B, H, N, d];
mask is a [B, N] uint8 array (non-zero = padded key) or None.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_D = ctypes.POINTER(ctypes.c_double)
_U8 = ctypes.POINTER(ctypes.c_ubyte)
_L = ctypes.POINTER(ctypes.c_long)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        L, D, I = ctypes.c_long, ctypes.c_double, ctypes.c_int
        lib.oracle_attn_f64.argtypes = [_D, _D, _D, _D, _D, L, L, L, L, D, I, _U8]
        lib.oracle_attn_rows_f64.argtypes = [_D, _D, _D, L, L, L, L, D, I, _U8, _L, L, _D, _D]
        lib.oracle_attn_blocked_f64.argtypes = [_D, _D, _D, _D, _D, L, L, L, L, D, I, _U8, L, I]
        lib.oracle_attn_blocked_kvouter_f64.argtypes = [_D, _D, _D, _D, _D, L, L, L, L, D, I, _U8, L, I]
        lib.oracle_row_softmax_f64.argtypes = [_D, _D, L, L, _D, _D]
        lib.oracle_row_blocked_f64.argtypes = [_D, _D, _U8, L, L, L, I, I, _D, _D]
        lib.oracle_attn_kv_f64.argtypes = [_D, _D, _D, _D, _D, L, L, L, L, L, D, I, _U8]
        lib.oracle_attn_bwd_f64.argtypes = [_D, _D, _D, _D, _D, _D, _D, L, L, L, L, D, I, _U8]
        lib.oracle_attn_blockmask_f64.argtypes = [_D, _D, _D, _D, _D, L, L, L, L, D, I, _U8, _U8, L]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_threads.argtypes = [I]
        lib.oracle_set_threads.restype = None
        for f in (lib.oracle_attn_f64, lib.oracle_attn_rows_f64, lib.oracle_attn_blocked_f64,
                  lib.oracle_attn_blocked_kvouter_f64, lib.oracle_row_softmax_f64,
                  lib.oracle_row_blocked_f64, lib.oracle_num_threads, lib.oracle_attn_kv_f64, lib.oracle_attn_bwd_f64, lib.oracle_attn_blockmask_f64):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_D)


def _mask(mask, B, N):
    if mask is None:
        return None, None
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    if m.shape != (B, N):
        raise ValueError("mask must be [B, N]")
    return m, m.ctypes.data_as(_U8)


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments")


def _qkv(q, k, v):
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    return (q, k, v), (qp, kp, vp)


def attn(q, k, v, scale, causal=False, mask=None):
    """Plain definition softmax(scale * q k^T + mask) v in fp64 -> (o, lse)."""
    keep, (qp, kp, vp) = _qkv(q, k, v)
    B, H, N, d = keep[0].shape
    mk, mp = _mask(mask, B, N)
    o = np.empty((B, H, N, d), np.float64)
    lse = np.empty((B, H, N), np.float64)
    _check(_load().oracle_attn_f64(qp, kp, vp, o.ctypes.data_as(_D), lse.ctypes.data_as(_D),
                                   B, H, N, d, float(scale), int(bool(causal)), mp))
    return o, lse


def attn_rows(q, k, v, scale, rows, causal=False, mask=None):
    """Plain definition for flat row indices (b*H + h)*N + i only -> (o[nr, d], lse[nr])."""
    keep, (qp, kp, vp) = _qkv(q, k, v)
    B, H, N, d = keep[0].shape
    mk, mp = _mask(mask, B, N)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((r.size, d), np.float64)
    lse = np.empty((r.size,), np.float64)
    _check(_load().oracle_attn_rows_f64(qp, kp, vp, B, H, N, d, float(scale), int(bool(causal)), mp,
                                        r.ctypes.data_as(_L), r.size, o.ctypes.data_as(_D),
                                        lse.ctypes.data_as(_D)))
    return o, lse


def attn_blocked(q, k, v, scale, bc, order=0, causal=False, mask=None, kv_outer=False):
    """Blocked online-softmax form with key-tile width bc; order 0 ascending, 1 descending."""
    keep, (qp, kp, vp) = _qkv(q, k, v)
    B, H, N, d = keep[0].shape
    mk, mp = _mask(mask, B, N)
    o = np.empty((B, H, N, d), np.float64)
    lse = np.empty((B, H, N), np.float64)
    fn = _load().oracle_attn_blocked_kvouter_f64 if kv_outer else _load().oracle_attn_blocked_f64
    _check(fn(qp, kp, vp, o.ctypes.data_as(_D), lse.ctypes.data_as(_D), B, H, N, d,
              float(scale), int(bool(causal)), mp, int(bc), int(order)))
    return o, lse


def row_softmax(scores, values):
    """Score-level plain softmax-weighted average of value rows -> (out[dv], lse)."""
    s, sp = _f64(scores)
    vals, vp = _f64(values)
    n = s.size
    dv = vals.shape[1] if vals.ndim == 2 else 1
    if vals.size != n * dv:
        raise ValueError("values must be [n, dv]")
    out = np.empty((dv,), np.float64)
    lse = np.empty((1,), np.float64)
    _check(_load().oracle_row_softmax_f64(sp, vp, n, dv, out.ctypes.data_as(_D), lse.ctypes.data_as(_D)))
    return out, float(lse[0])


def row_blocked(scores, values, width, order=0, visible=None, rescale=True):
    """Score-level blocked online form.  rescale=False is the deliberately wrong mutant."""
    s, sp = _f64(scores)
    vals, vp = _f64(values)
    n = s.size
    dv = vals.shape[1] if vals.ndim == 2 else 1
    if vals.size != n * dv:
        raise ValueError("values must be [n, dv]")
    vis = None
    vis_p = None
    if visible is not None:
        vis = np.ascontiguousarray(visible, dtype=np.uint8)
        vis_p = vis.ctypes.data_as(_U8)
    out = np.empty((dv,), np.float64)
    lse = np.empty((1,), np.float64)
    _check(_load().oracle_row_blocked_f64(sp, vp, vis_p, n, dv, int(width), int(order), int(bool(rescale)),
                                          out.ctypes.data_as(_D), lse.ctypes.data_as(_D)))
    return out, float(lse[0])


def attn_kv(q, k, v, scale, causal=False, mask=None):
    """Query block q [B,H,Nq,d] against keys/values [B,H,Nk,d], plain definition;
    causal visibility aligned to the end of the keys (row i sees j <= Nk - Nq + i,
    so with Nq > Nk the first Nq - Nk rows see nothing) -> (o, lse)."""
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    if q.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q [B,H,Nq,d] and k, v [B,H,Nk,d] do not match")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    mk, mp = _mask(mask, B, Nk)
    o = np.empty((B, H, Nq, d), np.float64)
    lse = np.empty((B, H, Nq), np.float64)
    _check(_load().oracle_attn_kv_f64(qp, kp, vp, o.ctypes.data_as(_D), lse.ctypes.data_as(_D),
                                      B, H, Nq, Nk, d, float(scale), int(bool(causal)), mp))
    return o, lse


def attn_bwd(q, k, v, dout, scale, causal=False, mask=None):
    """Gradient of the plain definition w.r.t. q, k, v for the output cotangent
    dout (all [B,H,N,d], fp64) -> (dq, dk, dv)."""
    keep, (qp, kp, vp) = _qkv(q, k, v)
    g, gp = _f64(dout)
    if g.shape != keep[0].shape:
        raise ValueError("dout must match q")
    B, H, N, d = keep[0].shape
    mk, mp = _mask(mask, B, N)
    dq = np.empty((B, H, N, d), np.float64)
    dk = np.empty((B, H, N, d), np.float64)
    dv = np.empty((B, H, N, d), np.float64)
    _check(_load().oracle_attn_bwd_f64(qp, kp, vp, gp, dq.ctypes.data_as(_D), dk.ctypes.data_as(_D),
                                       dv.ctypes.data_as(_D), B, H, N, d, float(scale), int(bool(causal)), mp))
    return dq, dk, dv


def attn_blockmask(q, k, v, scale, block_mask, block=64, causal=False, mask=None):
    """Plain definition with block-sparse visibility: block_mask [B,H,nb,nb]
    (nb = ceil(N / block)), non-zero = the block of pairs is attended."""
    keep, (qp, kp, vp) = _qkv(q, k, v)
    B, H, N, d = keep[0].shape
    nb = (N + block - 1) // block
    bm = np.ascontiguousarray(block_mask, dtype=np.uint8)
    if bm.shape != (B, H, nb, nb):
        raise ValueError(f"block_mask must be [B, H, {nb}, {nb}]")
    mk, mp = _mask(mask, B, N)
    o = np.empty((B, H, N, d), np.float64)
    lse = np.empty((B, H, N), np.float64)
    _check(_load().oracle_attn_blockmask_f64(qp, kp, vp, o.ctypes.data_as(_D), lse.ctypes.data_as(_D), B, H, N, d,
                                             float(scale), int(bool(causal)), mp, bm.ctypes.data_as(_U8), int(block)))
    return o, lse


def num_threads():
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def set_threads(n):
    """Threads of the oracle's parallel loops from now on (timing only)."""
    _load().oracle_set_threads(int(n))
