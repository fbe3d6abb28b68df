"""ctypes wrapper of the C oracle's direct form (``swa_oracle.c``).

Test infrastructure only: loaded by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library.

A problem is any object with the attributes ``batch, heads, head_dim,
extent, padded, window, shift, cyclic`` (3-tuples ordered time, latitude,
longitude) and optionally ``scale`` (None or 0 means 1/sqrt(head_dim)).
"""
import ctypes
import math
import os

import numpy as np

from .build import LIBRARY


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int), ("heads", ctypes.c_int), ("head_dim", ctypes.c_int),
        ("extent", ctypes.c_int * 3), ("padded", ctypes.c_int * 3),
        ("window", ctypes.c_int * 3), ("shift", ctypes.c_int * 3),
        ("cyclic", ctypes.c_int * 3), ("scale", ctypes.c_double),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"oracle library not built: {LIBRARY} (run oracle/build.py)")
        lib = ctypes.CDLL(LIBRARY)
        P = ctypes.POINTER(_Problem)
        lib.swo_forward.argtypes = [P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long,
                                    ctypes.c_void_p, ctypes.c_int]
        lib.swo_forward.restype = ctypes.c_int
        lib.swo_visible.argtypes = [P, ctypes.POINTER(ctypes.c_long), ctypes.POINTER(ctypes.c_long)]
        lib.swo_visible.restype = ctypes.c_int
        lib.swo_local_coord.argtypes = [P, ctypes.c_int, ctypes.c_long]
        lib.swo_local_coord.restype = ctypes.c_long
        lib.swo_check.argtypes = [P]
        lib.swo_check.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_scale(prob) -> float:
    s = getattr(prob, "scale", None)
    return float(s) if s else 1.0 / math.sqrt(prob.head_dim)


def _problem(prob) -> _Problem:
    p = _Problem()
    p.batch, p.heads, p.head_dim = prob.batch, prob.heads, prob.head_dim
    for a in range(3):
        p.extent[a] = prob.extent[a]
        p.padded[a] = prob.padded[a]
        p.window[a] = prob.window[a]
        p.shift[a] = prob.shift[a]
        p.cyclic[a] = int(prob.cyclic[a])
    p.scale = default_scale(prob)
    return p


def check(prob) -> int:
    """0 when the problem is a well-formed tiling, else a nonzero code."""
    return _load().swo_check(ctypes.byref(_problem(prob)))


def _f32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return a


def direct_forward(prob, q, k, v, table, query_index=None, nthreads=0):
    """fp64 output of the direct form.

    q, k, v: arrays [B, T, H, W, heads, head_dim] (any float dtype; converted
    to float32, which is exact for bf16 and fp32 values).  table:
    [2w_t-1, 2w_y-1, 2w_x-1, heads].  query_index: optional 1-D int array of
    flat real-token indices ((b*T + t)*H + y)*W + x.  Returns float64 of shape
    [B, T, H, W, heads, head_dim] when query_index is None, else
    [len(query_index), heads, head_dim], plus the thread count used.
    """
    lib = _load()
    p = _problem(prob)
    if lib.swo_check(ctypes.byref(p)) != 0:
        raise ValueError("malformed problem")
    q, k, v, table = _f32(q), _f32(k), _f32(v), _f32(table)
    B, (T, H, W) = prob.batch, prob.extent
    want = (B, T, H, W, prob.heads, prob.head_dim)
    for name, a in (("q", q), ("k", k), ("v", v)):
        if a.shape != want:
            raise ValueError(f"{name} has shape {a.shape}, expected {want}")
    tshape = (2 * prob.window[0] - 1, 2 * prob.window[1] - 1, 2 * prob.window[2] - 1, prob.heads)
    if table.shape != tshape:
        raise ValueError(f"table has shape {table.shape}, expected {tshape}")
    if query_index is None:
        out = np.empty(want, dtype=np.float64)
        qi_ptr, nq = None, 0
    else:
        qi = np.ascontiguousarray(np.asarray(query_index, dtype=np.int64))
        if qi.ndim != 1 or (qi.size and (qi.min() < 0 or qi.max() >= B * T * H * W)):
            raise ValueError("query_index out of range")
        out = np.empty((qi.size, prob.heads, prob.head_dim), dtype=np.float64)
        qi_ptr, nq = qi.ctypes.data, qi.size
    used = lib.swo_forward(ctypes.byref(p), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                           table.ctypes.data, qi_ptr, nq, out.ctypes.data, int(nthreads))
    if used < 0:
        raise ValueError("oracle rejected the problem")
    return out, used


def visible(prob, qc, kc) -> bool:
    """Direct-form visibility of the key at padded-frame coordinates kc to the
    query at qc (both (t, y, x)); False when either is a pad token."""
    lib = _load()
    p = _problem(prob)
    a = (ctypes.c_long * 3)(*qc)
    b = (ctypes.c_long * 3)(*kc)
    return bool(lib.swo_visible(ctypes.byref(p), a, b))


def local_coord(prob, axis, c) -> int:
    """Window-local coordinate ((c - s) mod P) mod w on one axis."""
    return int(_load().swo_local_coord(ctypes.byref(_problem(prob)), axis, c))
