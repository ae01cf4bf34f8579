"""Brute-force fp64 CPU oracle for neighborhood attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package. It shares no code with the GPU library (``fwd_bwd_amd``)
and imports nothing from it; both sides only see the same seeded inputs.

The arithmetic lives in ``na_oracle.c`` (plain C + OpenMP, every sum in
double). This module only builds it, loads it with ctypes and marshals numpy
arrays. Source of the method: the NATTEN issue "Backward pass is very slow
towards much tokens and large kernels" (SHI-Labs/NATTEN #161) -- its benchmark
script (token-major [B, (T,) H, W, heads, head_dim] tensors, per-axis
kernel_size, dilation, loss = output.sum()) and the maintainer's profiler
tables (ComputeDelta, AGRAD, QGRAD, KGRAD, VGRAD).

Every function here is pinned by a CPU test against something other than
itself (dense softmax attention from torch, finite differences, exact
identities, brute-force window properties); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "na_oracle.c")
_LIB = os.path.join(_HERE, "libna_oracle.so")


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle's C source into a shared library (gcc, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("extent", ctypes.c_int64 * 3),
        ("kernel", ctypes.c_int64 * 3),
        ("dilation", ctypes.c_int64 * 3),
        ("scale", ctypes.c_double),
    ]


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(_Problem)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_window_start.argtypes = [ctypes.c_int64] * 4
    lib.oracle_window_start.restype = ctypes.c_int64
    lib.oracle_na_fwd.argtypes = [P, dp, dp, dp, ctypes.c_int64, ip, dp, dp]
    lib.oracle_na_fwd.restype = None
    lib.oracle_na_weights.argtypes = [P, dp, dp, ctypes.c_int64, ip, dp, ip]
    lib.oracle_na_weights.restype = None
    lib.oracle_na_bwd.argtypes = [P, dp, dp, dp, dp, ctypes.c_int64, ip, dp, dp, dp]
    lib.oracle_na_bwd.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(_LIB)
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_load().oracle_num_threads())


def window_start(L: int, k: int, d: int, x: int) -> int:
    """First key coordinate (absolute) of the window of coordinate x on one axis."""
    return int(_load().oracle_window_start(L, k, d, x))


def _as3(v, ndim, fill):
    v = (v,) * ndim if np.isscalar(v) else tuple(int(a) for a in v)
    if len(v) != ndim:
        raise ValueError(f"expected {ndim} values, got {v}")
    return (fill,) * (3 - ndim) + v


def _problem(shape, kernel, dilation, scale):
    """shape is the token-major tensor shape [B, (T,) H, W, heads, D]."""
    ndim = len(shape) - 3
    if ndim not in (2, 3):
        raise ValueError("expected a 2D or 3D token grid")
    B, heads, D = shape[0], shape[-2], shape[-1]
    ext = (1,) * (3 - ndim) + tuple(shape[1:-2])
    p = _Problem()
    p.batch, p.heads, p.head_dim = B, heads, D
    p.extent[:] = ext
    p.kernel[:] = _as3(kernel, ndim, 1)
    p.dilation[:] = _as3(dilation, ndim, 1)
    p.scale = float(D ** -0.5 if scale is None else scale)
    for a in range(3):
        L, k, d = p.extent[a], p.kernel[a], p.dilation[a]
        if d < 1 or k < 1 or L < 1:
            raise ValueError("extent, kernel and dilation must be >= 1")
        if k > L // d:  # the smallest residue class holds floor(L / d) positions
            raise ValueError(f"kernel {k} does not fit extent {L} at dilation {d}")
    return p


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _f64(a):
    a = np.asarray(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _sel(sel):
    if sel is None:
        return 0, None
    s = np.ascontiguousarray(np.asarray(sel, dtype=np.int64).ravel())
    return s.size, s


def na_fwd(q, k, v, kernel, dilation=1, scale=None, sel=None, lib=None):
    """Forward. Returns (out, lse) as float64.

    Without ``sel`` the results have the full shapes [B,(T,)H,W,heads,D] and
    [B,(T,)H,W,heads]. With ``sel`` (flat ids of (b, token, head) in
    token-major order) they are [n, D] and [n].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    p = _problem(q.shape, kernel, dilation, scale)
    n, s = _sel(sel)
    if s is None:
        out = np.empty(q.shape, np.float64)
        lse = np.empty(q.shape[:-1], np.float64)
    else:
        out = np.empty((n, q.shape[-1]), np.float64)
        lse = np.empty((n,), np.float64)
    (lib or _load()).oracle_na_fwd(ctypes.byref(p), _dptr(q), _dptr(k), _dptr(v), n,
                          None if s is None else _iptr(s), _dptr(out), _dptr(lse))
    return out, lse


def na_weights(q, k, kernel, dilation=1, scale=None, sel=None, lib=None):
    """Attention weights of each (selected) query over its window.

    Returns (weights [n, K], key_tokens [n, K]) with K = prod(kernel), in the
    window's row-major offset order; key_tokens are token indices within the
    batch element.
    """
    q, k = _f64(q), _f64(k)
    p = _problem(q.shape, kernel, dilation, scale)
    n, s = _sel(sel)
    if s is None:
        n_all = int(np.prod(q.shape[:-1]))
    else:
        n_all = n
    K = int(np.prod(list(p.kernel)))
    w = np.empty((n_all, K), np.float64)
    keys = np.empty((n_all, K), np.int64)
    (lib or _load()).oracle_na_weights(ctypes.byref(p), _dptr(q), _dptr(k), n,
                              None if s is None else _iptr(s), _dptr(w), _iptr(keys))
    return w, keys


def na_bwd(q, k, v, dout, kernel, dilation=1, scale=None, sel=None, want=("dq", "dk", "dv"),
           lib=None):
    """Backward of sum(out * dout). Returns (dq, dk, dv) as float64 (None where not wanted).

    Shapes follow ``na_fwd``: full tensors, or [n, D] for the selected units
    (for dk/dv the selected unit is the key).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    p = _problem(q.shape, kernel, dilation, scale)
    n, s = _sel(sel)
    shape = q.shape if s is None else (n, q.shape[-1])
    res = {name: (np.empty(shape, np.float64) if name in want else None)
           for name in ("dq", "dk", "dv")}
    (lib or _load()).oracle_na_bwd(ctypes.byref(p), _dptr(q), _dptr(k), _dptr(v), _dptr(dout), n,
                          None if s is None else _iptr(s),
                          *(None if res[nm] is None else _dptr(res[nm]) for nm in ("dq", "dk", "dv")))
    return res["dq"], res["dk"], res["dv"]


class Bound:
    """The oracle's functions bound to one compiled library (the default build
    unless a path is given). Lets a check run against another build of the
    same source, e.g. one with a deliberately planted mistake."""

    def __init__(self, path=None):
        self.lib = _load() if path is None else _bind(path)

    def window_start(self, L, k, d, x):
        return int(self.lib.oracle_window_start(L, k, d, x))

    def na_fwd(self, *a, **kw):
        return na_fwd(*a, lib=self.lib, **kw)

    def na_weights(self, *a, **kw):
        return na_weights(*a, lib=self.lib, **kw)

    def na_bwd(self, *a, **kw):
        return na_bwd(*a, lib=self.lib, **kw)
