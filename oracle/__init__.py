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
    lib.oracle_na_qk.argtypes = [P, dp, dp, ctypes.c_double, ctypes.c_int64, ip, dp]
    lib.oracle_na_qk.restype = None
    lib.oracle_na_av.argtypes = [P, dp, dp, ctypes.c_double, ctypes.c_int64, ip, dp]
    lib.oracle_na_av.restype = None
    lib.oracle_na_av_inverse.argtypes = [P, dp, dp, ctypes.c_double, ctypes.c_int64, ip, dp]
    lib.oracle_na_av_inverse.restype = None
    lib.oracle_na_qk_rpb.argtypes = [P, dp, dp, ctypes.c_double, dp, ctypes.c_int64, ip, dp]
    lib.oracle_na_qk_rpb.restype = None
    lib.oracle_na_rpb_grad.argtypes = [P, dp, dp]
    lib.oracle_na_rpb_grad.restype = None
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


# ----------------------------------------------------------------------------- unfused ops
# The unfused formulation of the benchmark script (method = 'unfused'): na*_qk,
# a softmax over the window axis, na*_av, on head-major tensors
# [B, heads, (T,) H, W, C] (C = head_dim, or K = prod(kernel) for the attention
# array). The C oracle works token-major; these wrappers only move the heads
# axis (and translate selected unit ids) around the call. Selected units are
# flat ids of (b, head, token) in head-major order.

def _to_tm(x):
    """[B, heads, (T,) H, W, C] -> [B, (T,) H, W, heads, C]."""
    return np.ascontiguousarray(np.moveaxis(_f64(x), 1, -2))


def _to_hm(x):
    return np.ascontiguousarray(np.moveaxis(x, -2, 1))


def _sel_tm(sel, shape_hm):
    """Head-major unit ids -> token-major unit ids."""
    n, s = _sel(sel)
    if s is None:
        return n, None
    heads = shape_hm[1]
    tokens = int(np.prod(shape_hm[2:-1]))
    b, rest = np.divmod(s, heads * tokens)
    h, tok = np.divmod(rest, tokens)
    return n, np.ascontiguousarray((b * tokens + tok) * heads + h, dtype=np.int64)


def _problem_hm(shape_hm, kernel, dilation, head_dim):
    tm = (shape_hm[0],) + tuple(shape_hm[2:-1]) + (shape_hm[1], head_dim)
    return _problem(tm, kernel, dilation, 1.0)


def rpb_shape(kernel, heads):
    """Shape of a relative positional bias table: [heads, 2k-1 per axis]."""
    return (heads,) + tuple(2 * int(k) - 1 for k in kernel)


def na_qk(a, b, kernel, dilation=1, alpha=1.0, sel=None, rpb=None, lib=None):
    """attn[x, j] = alpha * <a_x, b_{N(x)_j}> (the script's na*_qk times alpha),
    plus rpb[head][offset of the key from the query] when a bias table is given
    (shape rpb_shape(kernel, heads)).

    a, b: [B, heads, (T,) H, W, D]. Returns [B, heads, (T,) H, W, K], or [n, K]
    for the selected query units.
    """
    a_tm, b_tm = _to_tm(a), _to_tm(b)
    p = _problem_hm(a.shape, kernel, dilation, a.shape[-1])
    K = int(np.prod(list(p.kernel)))
    n, s = _sel_tm(sel, a.shape)
    units = n if s is not None else int(np.prod(a.shape[:-1]))
    attn = np.empty((units, K), np.float64)
    if rpb is None:
        (lib or _load()).oracle_na_qk(ctypes.byref(p), _dptr(a_tm), _dptr(b_tm), float(alpha), n,
                                      None if s is None else _iptr(s), _dptr(attn))
    else:
        rp = _f64(rpb)
        if rp.shape != rpb_shape(kernel if not np.isscalar(kernel) else (kernel,) * (a.ndim - 3),
                                 a.shape[1]):
            raise ValueError("rpb must have shape rpb_shape(kernel, heads)")
        (lib or _load()).oracle_na_qk_rpb(ctypes.byref(p), _dptr(a_tm), _dptr(b_tm), float(alpha),
                                          _dptr(rp), n, None if s is None else _iptr(s),
                                          _dptr(attn))
    if s is not None:
        return attn
    return _to_hm(attn.reshape(a_tm.shape[:-1] + (K,)))


def na_av(attn, b, kernel, dilation=1, alpha=1.0, sel=None, lib=None):
    """out_x = alpha * sum_j attn[x, j] b_{N(x)_j} (the script's na*_av times alpha).

    attn: [B, heads, (T,) H, W, K]; b: [B, heads, (T,) H, W, D]. Returns the
    shape of b, or [n, D] for the selected query units.
    """
    at_tm, b_tm = _to_tm(attn), _to_tm(b)
    p = _problem_hm(b.shape, kernel, dilation, b.shape[-1])
    if attn.shape[:-1] != b.shape[:-1] or attn.shape[-1] != int(np.prod(list(p.kernel))):
        raise ValueError("attn must be [B, heads, (T,) H, W, prod(kernel)]")
    n, s = _sel_tm(sel, b.shape)
    out = np.empty(b_tm.shape if s is None else (n, b.shape[-1]), np.float64)
    (lib or _load()).oracle_na_av(ctypes.byref(p), _dptr(at_tm), _dptr(b_tm), float(alpha), n,
                                  None if s is None else _iptr(s), _dptr(out))
    return out if s is not None else _to_hm(out)


def na_av_inverse(attn, a, kernel, dilation=1, alpha=1.0, sel=None, lib=None):
    """out_y = alpha * sum over the queries x whose window holds y of attn[x, j] a_x.

    The map behind the gradients of the keys of na*_qk and of the values of
    na*_av (KGRAD, VGRAD). Shapes as in na_av; selected units are keys.
    """
    at_tm, a_tm = _to_tm(attn), _to_tm(a)
    p = _problem_hm(a.shape, kernel, dilation, a.shape[-1])
    if attn.shape[:-1] != a.shape[:-1] or attn.shape[-1] != int(np.prod(list(p.kernel))):
        raise ValueError("attn must be [B, heads, (T,) H, W, prod(kernel)]")
    n, s = _sel_tm(sel, a.shape)
    out = np.empty(a_tm.shape if s is None else (n, a.shape[-1]), np.float64)
    (lib or _load()).oracle_na_av_inverse(ctypes.byref(p), _dptr(at_tm), _dptr(a_tm),
                                          float(alpha), n, None if s is None else _iptr(s),
                                          _dptr(out))
    return out if s is not None else _to_hm(out)


def rpb_grad(dattn, kernel, dilation=1, lib=None):
    """Gradient of the bias table: for every head and relative offset, the sum
    of dattn over all batch elements, queries and window entries at that
    offset. dattn: [B, heads, (T,) H, W, K]. Returns rpb_shape(kernel, heads)."""
    at_tm = _to_tm(dattn)
    kern = (kernel,) * (dattn.ndim - 3) if np.isscalar(kernel) else tuple(kernel)
    p = _problem_hm(dattn.shape, kern, dilation, 1)
    out = np.empty(rpb_shape(kern, dattn.shape[1]), np.float64)
    (lib or _load()).oracle_na_rpb_grad(ctypes.byref(p), _dptr(at_tm), _dptr(out))
    return out


def softmax(x):
    """Softmax over the last (window) axis, as the script's F.softmax(attn, dim=-1):
    exp(x - max) / sum exp(x - max), in float64. A row whose entries are all
    -inf (every key masked out) gets zero weights."""
    x = _f64(x)
    m = np.max(x, axis=-1, keepdims=True)
    dead = np.isneginf(m)
    e = np.exp(x - np.where(dead, 0.0, m))
    s = np.sum(e, axis=-1, keepdims=True)
    return np.where(dead, 0.0, e / np.where(dead, 1.0, s))


def mask_scores(attn, mask):
    """Masked windows (the issue's requester masks the result of na3d_qk to get
    per-frame window sizes): score entries whose mask is 0 become -inf, so the
    window softmax gives them zero weight. mask: [(T,) H, W, K] per token,
    shared by every batch element and head (broadcast)."""
    attn = _f64(attn)
    return np.where(np.asarray(mask) != 0, attn, -np.inf)


def frame_window_mask(grid, kernel, frame_kernel):
    """Mask [T, H, W, K] keeping, for every query of frame t, only the keys
    whose frame lies in the window of size frame_kernel[t] around t (the same
    centered-and-shifted rule along T), inside the kernel[0]-frame window the
    scores are computed over: the requester's time kernel that varies per
    frame. Undilated grids."""
    T, H, W = grid
    kt, kh, kw = kernel
    mask = np.zeros((T, H, W, kt * kh * kw), np.uint8)
    for t in range(T):
        s_max = window_start(T, kt, 1, t)
        s_own = window_start(T, int(frame_kernel[t]), 1, t)
        for it in range(kt):
            f = s_max + it
            if s_own <= f < s_own + int(frame_kernel[t]):
                mask[t, :, :, it * kh * kw:(it + 1) * kh * kw] = 1
    return mask


def outer_window_mask(grid, kernel, outer_kernel, dilation=1):
    """Mask [*grid, K] (K = prod(kernel), window entries in row-major order)
    restricting windows along the outermost axis (H on 2D grids, T on 3D
    ones): a query at coordinate x0 along that axis keeps only the keys whose
    coordinate there lies in the window of size outer_kernel[x0] around x0 --
    the same centered-and-shifted rule, inside x0's residue class -- among the
    kernel[0] positions its scores are computed over. outer_kernel[x0] = 0
    masks every key of the query. The requester's per-frame time kernel is
    the 3D case."""
    grid, kernel = tuple(int(g) for g in grid), tuple(int(k) for k in kernel)
    dil = _as3(dilation, len(grid), 1)[3 - len(grid):]
    L0, k0, d0 = grid[0], kernel[0], int(dil[0])
    rest = int(np.prod(kernel[1:]))
    mask = np.zeros(grid + (k0 * rest,), np.uint8)
    for x0 in range(L0):
        fk = int(outer_kernel[x0])
        if fk == 0:
            continue
        s_max = window_start(L0, k0, d0, x0)
        s_own = window_start(L0, fk, d0, x0)
        for i0 in range(k0):
            f = s_max + d0 * i0
            if s_own <= f < s_own + d0 * fk:
                mask[x0, ..., i0 * rest:(i0 + 1) * rest] = 1
    return mask


def window_mask_from_indices(grid, kernel, indices, dilation=1):
    """The requester's other form of a per-query window (an index tensor of
    the attended tokens, for na3d_qk) as a mask of the window entries:
    indices [*grid, m] lists, per query token, flat token indices (row-major
    over the grid) of the keys it attends to, -1 for an unused slot. Returns
    (mask [*grid, prod(kernel)] uint8, bad [*grid] int32): a listed token that
    lies in the query's window sets the entry of its place there (per axis,
    (coordinate - window start) / dilation, entries row-major over the axes);
    bad counts the slots that hold neither -1 nor a token of the query's
    window. Plain loops over queries, slots and axes."""
    grid, kernel = tuple(int(g) for g in grid), tuple(int(k) for k in kernel)
    nd = len(grid)
    dil = _as3(dilation, nd, 1)[3 - nd:]
    idx = np.asarray(indices, dtype=np.int64)
    mask = np.zeros(grid + (int(np.prod(kernel)),), np.uint8)
    bad = np.zeros(grid, np.int32)
    ntok = int(np.prod(grid))
    for x in np.ndindex(*grid):
        starts = [window_start(grid[a], kernel[a], int(dil[a]), x[a]) for a in range(nd)]
        for y in idx[x]:
            y = int(y)
            if y == -1:
                continue
            if not 0 <= y < ntok:
                bad[x] += 1
                continue
            yc = np.unravel_index(y, grid)
            place = []
            for a in range(nd):
                rel = int(yc[a]) - starts[a]
                if rel < 0 or rel % int(dil[a]) or rel // int(dil[a]) >= kernel[a]:
                    break
                place.append(rel // int(dil[a]))
            if len(place) < nd:
                bad[x] += 1
                continue
            mask[x + (int(np.ravel_multi_index(place, kernel)),)] = 1
    return mask, bad


def softmax_bwd(p, dp):
    """Backward of the window softmax: dS = P * (dP - sum_j P dP) over the last axis."""
    p, dp = _f64(p), _f64(dp)
    return p * (dp - np.sum(p * dp, axis=-1, keepdims=True))


def unfused_fwd(q, k, v, kernel, dilation=1, scale=None, rpb=None, mask=None, lib=None):
    """The unfused forward on head-major tensors: P = softmax(scale * na_qk(q, k)
    [+ rpb], masked), out = na_av(P, v). Returns (P, out)."""
    scale = q.shape[-1] ** -0.5 if scale is None else scale
    s = na_qk(q, k, kernel, dilation, scale, rpb=rpb, lib=lib)
    if mask is not None:
        s = mask_scores(s, mask)
    P = softmax(s)
    return P, na_av(P, v, kernel, dilation, 1.0, lib=lib)


def unfused_bwd(q, k, v, P, dout, kernel, dilation=1, scale=None, want_rpb=False, lib=None):
    """Backward of sum(out * dout) through the unfused ops (AGRAD, softmax
    backward, QGRAD, KGRAD, VGRAD). Returns (dq, dk, dv), and the bias
    gradient as a fourth value when want_rpb."""
    scale = q.shape[-1] ** -0.5 if scale is None else scale
    dP = na_qk(dout, v, kernel, dilation, 1.0, lib=lib)             # AGRAD
    dv = na_av_inverse(P, dout, kernel, dilation, 1.0, lib=lib)      # VGRAD
    dS = softmax_bwd(P, dP)
    dq = na_av(dS, k, kernel, dilation, scale, lib=lib)              # QGRAD
    dk = na_av_inverse(dS, q, kernel, dilation, scale, lib=lib)      # KGRAD
    if want_rpb:
        return dq, dk, dv, rpb_grad(dS, kernel, dilation, lib=lib)
    return dq, dk, dv


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

    def na_qk(self, *a, **kw):
        return na_qk(*a, lib=self.lib, **kw)

    def na_av(self, *a, **kw):
        return na_av(*a, lib=self.lib, **kw)

    def na_av_inverse(self, *a, **kw):
        return na_av_inverse(*a, lib=self.lib, **kw)

    def rpb_grad(self, *a, **kw):
        return rpb_grad(*a, lib=self.lib, **kw)

    def unfused_fwd(self, *a, **kw):
        return unfused_fwd(*a, lib=self.lib, **kw)

    def unfused_bwd(self, *a, **kw):
        return unfused_bwd(*a, lib=self.lib, **kw)
