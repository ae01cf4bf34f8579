"""Thin ctypes binding of libna (include/na.h): argument marshalling only.

Every step of neighborhood attention runs in the library's HIP kernels; this
module allocates the output tensors with torch (device memory and the current
stream are the only things torch provides), passes raw pointers, and turns a
non-OK status into an exception. There is no fallback: if libna.so is missing
or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libna.so")

NA_OK = 0
NA_ERR_INVALID_ARG = 1
NA_ERR_UNSUPPORTED = 2
NA_ERR_WORKSPACE = 3
NA_ERR_HIP = 4

NA_F32 = 0
NA_BF16 = 1
NA_F16 = 2

NA_BWD_GATHER = 0
NA_BWD_KVPARALLEL = 1
VARIANTS = {"gather": NA_BWD_GATHER, "kvparallel": NA_BWD_KVPARALLEL}

# every symbol include/na.h declares
EXPORTS = ("na_check_problem", "na_fwd", "na_bwd_workspace_bytes", "na_bwd", "na_bwd_dq",
           "na_bwd_dkdv", "na_status_string", "na_window_start", "na_inverse_window",
           "na_qk", "na_av", "na_av_inverse", "na_softmax", "na_softmax_bwd", "na_unfused_fwd",
           "na_unfused_bwd", "na_rpb_grad_workspace_bytes", "na_rpb_grad", "na_qk_softmax",
           "na_qk_softmax_bwd", "na_source_sha256", "na_bwd_noalloc", "na_fwd_framed",
           "na_bwd_framed", "na_fwd_masked", "na_bwd_masked", "na_window_mask_from_indices")

# rows (batch * tokens * heads) the static delta array of na_bwd_noalloc holds
NOALLOC_MAX_ROWS = 8388608


class NaProblem(ctypes.Structure):
    """Mirror of na_problem."""
    _fields_ = [
        ("ndim", ctypes.c_int64),
        ("dtype", ctypes.c_int64),
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("extent", ctypes.c_int64 * 3),
        ("kernel", ctypes.c_int64 * 3),
        ("dilation", ctypes.c_int64 * 3),
        ("scale", ctypes.c_double),
    ]


class NaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libna.so (built in-tree by fwd_bwd_amd.build); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run fwd_bwd_amd.build.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, P = ctypes.c_void_p, ctypes.POINTER(NaProblem)
        i64 = ctypes.c_int64
        lib.na_check_problem.argtypes = [P]
        lib.na_check_problem.restype = ctypes.c_int
        lib.na_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp]
        lib.na_fwd.restype = ctypes.c_int
        lib.na_bwd_workspace_bytes.argtypes = [P, ctypes.c_int32, ctypes.c_int32]
        lib.na_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.na_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                               ctypes.c_int32, ctypes.c_int32, vp]
        lib.na_bwd.restype = ctypes.c_int
        lib.na_bwd_dq.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.na_bwd_dq.restype = ctypes.c_int
        lib.na_bwd_dkdv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.na_bwd_dkdv.restype = ctypes.c_int
        lib.na_status_string.argtypes = [ctypes.c_int]
        lib.na_status_string.restype = ctypes.c_char_p
        lib.na_source_sha256.argtypes = []
        lib.na_source_sha256.restype = ctypes.c_char_p
        lib.na_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.na_bwd_noalloc.restype = ctypes.c_int
        lib.na_fwd_framed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        lib.na_fwd_framed.restype = ctypes.c_int
        lib.na_bwd_framed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                      ctypes.c_int32, ctypes.c_int32, vp, vp]
        lib.na_bwd_framed.restype = ctypes.c_int
        lib.na_fwd_masked.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        lib.na_fwd_masked.restype = ctypes.c_int
        lib.na_bwd_masked.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                      ctypes.c_int32, ctypes.c_int32, vp, vp]
        lib.na_bwd_masked.restype = ctypes.c_int
        lib.na_window_mask_from_indices.argtypes = [P, vp, ctypes.c_int32, vp, vp, vp]
        lib.na_window_mask_from_indices.restype = ctypes.c_int
        lib.na_window_start.argtypes = [i64, i64, i64, i64]
        lib.na_window_start.restype = i64
        lib.na_inverse_window.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64),
                                          ctypes.POINTER(i64)]
        lib.na_inverse_window.restype = ctypes.c_int
        dbl = ctypes.c_double
        lib.na_qk.argtypes = [P, vp, vp, dbl, vp, vp, vp, vp]
        lib.na_qk_softmax.argtypes = [P, vp, vp, dbl, vp, vp, vp, vp]
        lib.na_qk_softmax.restype = ctypes.c_int
        lib.na_qk_softmax_bwd.argtypes = [P, vp, vp, vp, vp, vp]
        lib.na_qk_softmax_bwd.restype = ctypes.c_int
        lib.na_rpb_grad_workspace_bytes.argtypes = [P]
        lib.na_rpb_grad_workspace_bytes.restype = ctypes.c_size_t
        lib.na_rpb_grad.argtypes = [P, vp, vp, vp, ctypes.c_size_t, vp]
        lib.na_rpb_grad.restype = ctypes.c_int
        lib.na_av.argtypes = [P, vp, vp, dbl, vp, vp]
        lib.na_av_inverse.argtypes = [P, vp, vp, dbl, vp, vp]
        lib.na_softmax.argtypes = [P, vp, vp, vp]
        lib.na_softmax_bwd.argtypes = [P, vp, vp, vp, vp]
        lib.na_unfused_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.na_unfused_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
        for name in ("na_qk", "na_av", "na_av_inverse", "na_softmax", "na_softmax_bwd",
                     "na_unfused_fwd", "na_unfused_bwd"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(status: int):
    if status != NA_OK:
        raise NaError(status, load().na_status_string(status).decode())


def _tuple(v: Union[int, Sequence[int]], n: int) -> Tuple[int, ...]:
    if isinstance(v, int):
        return (v,) * n
    v = tuple(int(a) for a in v)
    if len(v) != n:
        raise ValueError(f"expected {n} values, got {v}")
    return v


_DTYPES = {torch.float32: NA_F32, torch.bfloat16: NA_BF16, torch.float16: NA_F16}


def make_problem(shape: Sequence[int], dtype: torch.dtype, kernel_size, dilation=1,
                 scale: Optional[float] = None) -> NaProblem:
    """na_problem for a token-major tensor shape [B, (T,) H, W, heads, head_dim]."""
    ndim = len(shape) - 3
    if ndim not in (2, 3):
        raise ValueError(f"expected [B, (T,) H, W, heads, head_dim], got shape {tuple(shape)}")
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    p = NaProblem()
    p.ndim = ndim
    p.dtype = _DTYPES[dtype]
    p.batch, p.heads, p.head_dim = int(shape[0]), int(shape[-2]), int(shape[-1])
    ext = tuple(int(s) for s in shape[1:-2])
    ks, ds = _tuple(kernel_size, ndim), _tuple(dilation, ndim)
    for a in range(3):
        p.extent[a] = ext[a] if a < ndim else 0
        p.kernel[a] = ks[a] if a < ndim else 0
        p.dilation[a] = ds[a] if a < ndim else 0
    p.scale = float(shape[-1] ** -0.5 if scale is None else scale)
    return p


def check_problem(p: NaProblem) -> int:
    return int(load().na_check_problem(ctypes.byref(p)))


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _check_tensors(ref: torch.Tensor, *ts: torch.Tensor):
    for t in ts:
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v (and out, dout) must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (token-major layout)")
    if ref.device.type != "cuda":
        raise ValueError("tensors must live on the GPU")


def _check_buf(t: torch.Tensor, name: str, shape, dtype: torch.dtype, device: torch.device):
    """A caller-supplied output or workspace buffer: the C ABI cannot see sizes,
    so a wrong one would be written out of bounds; reject it here."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(ws: torch.Tensor, need: int, device: torch.device):
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {need}")


def na_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kernel_size, dilation=1,
           scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Fused NA forward. Returns (out, lse); lse is fp32 [B,(T,)H,W,heads]."""
    _check_tensors(q, k, v)
    p = make_problem(q.shape, q.dtype, kernel_size, dilation, scale)
    if out is None:
        out = torch.empty_like(q)
    _check_buf(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    _check_buf(lse, "lse", q.shape[:-1], torch.float32, q.device)
    _check(load().na_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                         _stream_handle(q.device)))
    return out, lse


def bwd_workspace_bytes(p: NaProblem, variant: int, kv_splits: int = 0) -> int:
    return int(load().na_bwd_workspace_bytes(ctypes.byref(p), variant, kv_splits))


def na_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
           dout: torch.Tensor, lse: torch.Tensor, kernel_size, dilation=1,
           scale: Optional[float] = None, variant: str = "gather",
           workspace: Optional[torch.Tensor] = None,
           grads: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
           kv_splits: int = 0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Fused NA backward of sum(out * dout). Returns (dq, dk, dv). kv_splits
    (KV-parallel only): 0 = float atomics into one accumulator; S >= 1 = at most
    S accumulator copies, bitwise reproducible."""
    _check_tensors(q, k, v, out, dout)
    if lse.dtype != torch.float32 or lse.shape != q.shape[:-1] or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 tensor of shape q.shape[:-1]")
    p = make_problem(q.shape, q.dtype, kernel_size, dilation, scale)
    vid = VARIANTS[variant]
    if kv_splits < 0:
        raise ValueError("kv_splits must be >= 0")
    need = bwd_workspace_bytes(p, vid, kv_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_buf(g, name, q.shape, q.dtype, q.device)
    _check(load().na_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                         _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), vid, kv_splits,
                         _stream_handle(q.device)))
    return dq, dk, dv


def na_bwd_dq(q, k, v, out, dout, lse, kernel_size, dilation=1, scale=None, dq=None, delta=None):
    """Query half of the gather backward: returns (dq, delta)."""
    _check_tensors(q, k, v, out, dout)
    _check_buf(lse, "lse", q.shape[:-1], torch.float32, q.device)
    p = make_problem(q.shape, q.dtype, kernel_size, dilation, scale)
    if dq is None:
        dq = torch.empty_like(q)
    _check_buf(dq, "dq", q.shape, q.dtype, q.device)
    if delta is None:
        delta = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    _check_buf(delta, "delta", q.shape[:-1], torch.float32, q.device)
    _check(load().na_bwd_dq(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                            _ptr(lse), _ptr(dq), _ptr(delta), _stream_handle(q.device)))
    return dq, delta


def na_bwd_dkdv(q, k, v, dout, lse, delta, kernel_size, dilation=1, scale=None, dk=None, dv=None):
    """Key half of the gather backward: returns (dk, dv)."""
    _check_tensors(q, k, v, dout)
    _check_buf(lse, "lse", q.shape[:-1], torch.float32, q.device)
    _check_buf(delta, "delta", q.shape[:-1], torch.float32, q.device)
    p = make_problem(q.shape, q.dtype, kernel_size, dilation, scale)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    _check_buf(dk, "dk", q.shape, q.dtype, q.device)
    _check_buf(dv, "dv", q.shape, q.dtype, q.device)
    _check(load().na_bwd_dkdv(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                              _ptr(delta), _ptr(dk), _ptr(dv), _stream_handle(q.device)))
    return dk, dv


def na_bwd_noalloc(q, k, v, out, dout, lse, kernel_size, dilation=1, scale=None, grads=None):
    """The gather backward with its delta rows in the library's static device
    array instead of a workspace (the C entry point allocates nothing; pass
    grads to allocate nothing here either). Returns (dq, dk, dv)."""
    _check_tensors(q, k, v, out, dout)
    _check_buf(lse, "lse", q.shape[:-1], torch.float32, q.device)
    p = make_problem(q.shape, q.dtype, kernel_size, dilation, scale)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_buf(g, name, q.shape, q.dtype, q.device)
    _check(load().na_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                 _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _stream_handle(q.device)))
    return dq, dk, dv


def _check_frame(frame_kernel: torch.Tensor, q: torch.Tensor):
    """Per-coordinate window sizes along the outermost grid axis: int32, one
    per coordinate (q.shape[1]), on q's device, contiguous."""
    if (not isinstance(frame_kernel, torch.Tensor) or frame_kernel.dtype != torch.int32
            or tuple(frame_kernel.shape) != (q.shape[1],) or frame_kernel.device != q.device
            or not frame_kernel.is_contiguous()):
        raise ValueError(f"frame_kernel must be a contiguous int32 tensor of shape ({q.shape[1]},) "
                         f"on {q.device}")
    return _ptr(frame_kernel)


def na_fwd_framed(q, k, v, frame_kernel, kernel_size, dilation=1, scale=None, out=None, lse=None):
    """na_fwd with windows restricted along the outermost axis (T on 3D grids,
    H on 2D grids) to frame_kernel[x0] positions around each query's x0."""
    _check_tensors(q, k, v)
    fp = _check_frame(frame_kernel, q)
    p = make_problem(q.shape, q.dtype, kernel_size, dilation, scale)
    if out is None:
        out = torch.empty_like(q)
    _check_buf(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    _check_buf(lse, "lse", q.shape[:-1], torch.float32, q.device)
    _check(load().na_fwd_framed(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                fp, _stream_handle(q.device)))
    return out, lse


def na_bwd_framed(q, k, v, out, dout, lse, frame_kernel, kernel_size, dilation=1, scale=None,
                  variant="gather", kv_splits=0, workspace=None, grads=None):
    """na_bwd with the windows of na_fwd_framed. Returns (dq, dk, dv)."""
    _check_tensors(q, k, v, out, dout)
    _check_buf(lse, "lse", q.shape[:-1], torch.float32, q.device)
    fp = _check_frame(frame_kernel, q)
    p = make_problem(q.shape, q.dtype, kernel_size, dilation, scale)
    vid = VARIANTS[variant]
    if kv_splits < 0:
        raise ValueError("kv_splits must be >= 0")
    need = bwd_workspace_bytes(p, vid, kv_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_buf(g, name, q.shape, q.dtype, q.device)
    _check(load().na_bwd_framed(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(workspace), workspace.numel() * workspace.element_size(), vid,
                                kv_splits, fp, _stream_handle(q.device)))
    return dq, dk, dv


def _check_window_mask(mask: torch.Tensor, q: torch.Tensor, kernel_size):
    """Window mask of the masked entry points: contiguous uint8
    [(T,) H, W, prod(kernel)] (token-major grid order), on q's device."""
    ks = _tuple(kernel_size, q.dim() - 3)
    K = 1
    for k in ks:
        K *= int(k)
    want = tuple(q.shape[1:-2]) + (K,)
    if (not isinstance(mask, torch.Tensor) or mask.dtype != torch.uint8
            or tuple(mask.shape) != want or mask.device != q.device or not mask.is_contiguous()):
        raise ValueError(f"mask must be a contiguous uint8 tensor of shape {want} on {q.device}")
    return _ptr(mask)


def na_fwd_masked(q, k, v, mask, kernel_size, dilation=1, scale=None, out=None, lse=None):
    """na_fwd with an arbitrary set of each query's window keys masked
    (mask[(t,) h, w, j] == 0 drops the j-th key of the window of token (t, h, w))."""
    _check_tensors(q, k, v)
    mp = _check_window_mask(mask, q, kernel_size)
    p = make_problem(q.shape, q.dtype, kernel_size, dilation, scale)
    if out is None:
        out = torch.empty_like(q)
    _check_buf(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    _check_buf(lse, "lse", q.shape[:-1], torch.float32, q.device)
    _check(load().na_fwd_masked(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                mp, _stream_handle(q.device)))
    return out, lse


def na_bwd_masked(q, k, v, out, dout, lse, mask, kernel_size, dilation=1, scale=None,
                  variant="gather", kv_splits=0, workspace=None, grads=None):
    """na_bwd with the windows of na_fwd_masked. Returns (dq, dk, dv)."""
    _check_tensors(q, k, v, out, dout)
    _check_buf(lse, "lse", q.shape[:-1], torch.float32, q.device)
    mp = _check_window_mask(mask, q, kernel_size)
    p = make_problem(q.shape, q.dtype, kernel_size, dilation, scale)
    vid = VARIANTS[variant]
    if kv_splits < 0:
        raise ValueError("kv_splits must be >= 0")
    need = bwd_workspace_bytes(p, vid, kv_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_buf(g, name, q.shape, q.dtype, q.device)
    _check(load().na_bwd_masked(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(workspace), workspace.numel() * workspace.element_size(), vid,
                                kv_splits, mp, _stream_handle(q.device)))
    return dq, dk, dv


def na_window_mask_from_indices(indices: torch.Tensor, kernel_size, dilation=1, mask=None,
                                bad=None, check: bool = True):
    """Window mask of na_fwd_masked / na_bwd_masked from an index tensor of
    attended tokens: indices is a contiguous int64 tensor [(T,) H, W, m] on the
    GPU, per query token m flat token indices ((t * H + h) * W + w) of keys in
    its window, -1 for an unused slot. Returns (mask, bad): mask uint8
    [(T,) H, W, prod(kernel)], bad int32 [(T,) H, W] = the query's slots that
    hold neither -1 nor a token of its window. With check (the default) a
    nonzero bad raises ValueError (reading it back synchronizes the stream)."""
    if (not isinstance(indices, torch.Tensor) or indices.dtype != torch.int64
            or indices.dim() not in (3, 4) or not indices.is_contiguous()
            or indices.device.type != "cuda"):
        raise ValueError("indices must be a contiguous int64 CUDA tensor [(T,) H, W, m]")
    grid = tuple(indices.shape[:-1])
    m = int(indices.shape[-1])
    if m > 2 ** 31 - 1:
        raise ValueError("too many slots per query")
    p = make_problem((1,) + grid + (1, 16), torch.float32, kernel_size, dilation)
    K = 1
    for k in p.kernel[:p.ndim]:
        K *= int(k)
    if mask is None:
        mask = torch.empty(grid + (K,), dtype=torch.uint8, device=indices.device)
    _check_buf(mask, "mask", grid + (K,), torch.uint8, indices.device)
    if bad is None:
        bad = torch.empty(grid, dtype=torch.int32, device=indices.device)
    _check_buf(bad, "bad", grid, torch.int32, indices.device)
    _check(load().na_window_mask_from_indices(ctypes.byref(p), _ptr(indices), m, _ptr(mask),
                                              _ptr(bad), _stream_handle(indices.device)))
    if check:
        wrong = torch.nonzero(bad)
        if wrong.numel():
            first = tuple(int(c) for c in wrong[0])
            raise ValueError(f"{wrong.shape[0]} query tokens list tokens outside their window "
                             f"(first: {first}, {int(bad[first])} slots)")
    return mask, bad


def source_sha256() -> str:
    """sha256 of the sources the loaded library was built from."""
    return load().na_source_sha256().decode()


def window_start(extent: int, kernel: int, dilation: int, x: int) -> int:
    return int(load().na_window_start(extent, kernel, dilation, x))


def inverse_window(extent: int, kernel: int, dilation: int, y: int) -> Tuple[int, int]:
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(load().na_inverse_window(extent, kernel, dilation, y, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


class NeighborhoodAttention(torch.autograd.Function):
    """Autograd wrapper: forward = na_fwd, backward = na_bwd (gather variant)."""

    @staticmethod
    def forward(ctx, q, k, v, kernel_size, dilation, scale):
        # views (e.g. q, k, v split from one fused projection) become contiguous
        # copies here, and the backward gets those same copies
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out, lse = na_fwd(q, k, v, kernel_size, dilation, scale)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.cfg = (kernel_size, dilation, scale)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        dq, dk, dv = na_bwd(q, k, v, out, dout.contiguous(), lse, *ctx.cfg)
        return dq, dk, dv, None, None, None


def neighborhood_attention(q, k, v, kernel_size, dilation=1, scale=None):
    """Differentiable fused NA on token-major [B, (T,) H, W, heads, head_dim] tensors."""
    return NeighborhoodAttention.apply(q, k, v, kernel_size, dilation, scale)


# ----------------------------------------------------------------------------- unfused ops
# Head-major tensors [B, heads, (T,) H, W, head_dim] and fp32 attention arrays
# [B, heads, (T,) H, W, K], as the benchmark script's unfused method uses them.

def make_problem_hm(shape: Sequence[int], head_dim: int, kernel_size, dilation=1,
                    scale: Optional[float] = None) -> NaProblem:
    """fp32 na_problem for a head-major shape [B, heads, (T,) H, W, C] (C is
    head_dim for vectors, K for attention arrays; head_dim is given apart)."""
    ndim = len(shape) - 3
    tm = (shape[0],) + tuple(shape[2:-1]) + (shape[1], head_dim)
    if ndim not in (2, 3):
        raise ValueError(f"expected [B, heads, (T,) H, W, C], got shape {tuple(shape)}")
    return make_problem(tm, torch.float32, kernel_size, dilation, scale)


def _window_size(kernel_size, ndim):
    n = 1
    for k in _tuple(kernel_size, ndim):
        n *= k
    return n


def _check_hm(*ts: torch.Tensor):
    for t in ts:
        if t.dtype != torch.float32:
            raise ValueError("the unfused ops take fp32 tensors")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (head-major layout)")
        if t.device.type != "cuda":
            raise ValueError("tensors must live on the GPU")


def _check_hm_buf(t, name: str, shape, ref: torch.Tensor):
    """A caller-supplied fp32 buffer of the unfused ops: right shape, on ref's device."""
    _check_hm(t)
    if tuple(t.shape) != tuple(shape) or t.device != ref.device:
        raise ValueError(f"{name} must be an fp32 tensor of shape {tuple(shape)} on {ref.device}")


def _attn_like(x: torch.Tensor, K: int) -> torch.Tensor:
    return torch.empty(x.shape[:-1] + (K,), dtype=torch.float32, device=x.device)


def rpb_shape(kernel_size, heads: int, ndim: int) -> Tuple[int, ...]:
    """Shape of a relative positional bias table: [heads, 2k - 1 per axis]."""
    return (heads,) + tuple(2 * k - 1 for k in _tuple(kernel_size, ndim))


def _check_rpb(rpb, kernel_size, heads, ndim, ref):
    if rpb is None:
        return None
    _check_hm(rpb)
    if tuple(rpb.shape) != rpb_shape(kernel_size, heads, ndim) or rpb.device != ref.device:
        raise ValueError(f"rpb must be an fp32 tensor of shape {rpb_shape(kernel_size, heads, ndim)}")
    return _ptr(rpb)


def _check_mask(mask, ref, K):
    """A window mask: uint8 [(T,) H, W, K] per token, on the device of ref."""
    if mask is None:
        return None
    if mask.dtype != torch.uint8 or not mask.is_contiguous() or mask.device != ref.device:
        raise ValueError("mask must be a contiguous uint8 tensor on the tensors' device")
    if tuple(mask.shape) != tuple(ref.shape[2:-1]) + (K,):
        raise ValueError(f"mask must have shape {tuple(ref.shape[2:-1]) + (K,)}")
    return _ptr(mask)


def na_qk(a: torch.Tensor, b: torch.Tensor, kernel_size, dilation=1, alpha: float = 1.0,
          attn: Optional[torch.Tensor] = None, rpb: Optional[torch.Tensor] = None,
          mask: Optional[torch.Tensor] = None) -> torch.Tensor:
    """attn[x, j] = alpha * <a_x, b_{N(x)_j}> [+ rpb[head, offset]], -inf where the
    window mask is 0 (na*_qk, QKRPB; AGRAD with a = dout, b = v)."""
    _check_hm(a, b)
    ndim = a.dim() - 3
    K = _window_size(kernel_size, ndim)
    p = make_problem_hm(a.shape, a.shape[-1], kernel_size, dilation)
    if b.shape != a.shape:
        raise ValueError("a and b must share their shape")
    rp = _check_rpb(rpb, kernel_size, a.shape[1], ndim, a)
    mp = _check_mask(mask, a, K)
    if attn is None:
        attn = _attn_like(a, K)
    _check_hm_buf(attn, "attn", a.shape[:-1] + (K,), a)
    _check(load().na_qk(ctypes.byref(p), _ptr(a), _ptr(b), float(alpha), rp, mp, _ptr(attn),
                        _stream_handle(a.device)))
    return attn


def na_qk_softmax(a: torch.Tensor, b: torch.Tensor, kernel_size, dilation=1, alpha: float = 1.0,
                  probs: Optional[torch.Tensor] = None, rpb: Optional[torch.Tensor] = None,
                  mask: Optional[torch.Tensor] = None) -> torch.Tensor:
    """softmax(na_qk(a, b, alpha, rpb, mask)) over the window axis."""
    _check_hm(a, b)
    ndim = a.dim() - 3
    K = _window_size(kernel_size, ndim)
    if b.shape != a.shape:
        raise ValueError("a and b must share their shape")
    p = make_problem_hm(a.shape, a.shape[-1], kernel_size, dilation)
    rp = _check_rpb(rpb, kernel_size, a.shape[1], ndim, a)
    mp = _check_mask(mask, a, K)
    if probs is None:
        probs = _attn_like(a, K)
    _check_hm_buf(probs, "probs", a.shape[:-1] + (K,), a)
    _check(load().na_qk_softmax(ctypes.byref(p), _ptr(a), _ptr(b), float(alpha), rp, mp,
                                _ptr(probs), _stream_handle(a.device)))
    return probs


def na_qk_softmax_bwd(dout: torch.Tensor, v: torch.Tensor, probs: torch.Tensor, kernel_size,
                      dilation=1, dscores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dS = probs * (dP - rowsum(probs * dP)) with dP = na_qk(dout, v)."""
    _check_hm(dout, v, probs)
    K = _window_size(kernel_size, dout.dim() - 3)
    if probs.shape != dout.shape[:-1] + (K,) or v.shape != dout.shape:
        raise ValueError("probs must be [B, heads, (T,) H, W, prod(kernel_size)], v like dout")
    p = make_problem_hm(dout.shape, dout.shape[-1], kernel_size, dilation)
    if dscores is None:
        dscores = _attn_like(dout, K)
    _check_hm_buf(dscores, "dscores", dout.shape[:-1] + (K,), dout)
    _check(load().na_qk_softmax_bwd(ctypes.byref(p), _ptr(dout), _ptr(v), _ptr(probs),
                                    _ptr(dscores), _stream_handle(dout.device)))
    return dscores


def na_rpb_grad(dscores: torch.Tensor, kernel_size, dilation=1,
                drpb: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of the bias table from dscores [B, heads, (T,) H, W, K]."""
    _check_hm(dscores)
    ndim = dscores.dim() - 3
    p = make_problem_hm(dscores.shape, 16, kernel_size, dilation)
    need = int(load().na_rpb_grad_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dscores.device)
    _check_workspace(workspace, need, dscores.device)
    if drpb is None:
        drpb = torch.empty(rpb_shape(kernel_size, dscores.shape[1], ndim), dtype=torch.float32,
                           device=dscores.device)
    _check_hm_buf(drpb, "drpb", rpb_shape(kernel_size, dscores.shape[1], ndim), dscores)
    _check(load().na_rpb_grad(ctypes.byref(p), _ptr(dscores), _ptr(drpb), _ptr(workspace),
                              workspace.numel() * workspace.element_size(),
                              _stream_handle(dscores.device)))
    return drpb


def na_av(attn: torch.Tensor, b: torch.Tensor, kernel_size, dilation=1, alpha: float = 1.0,
          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out_x = alpha * sum_j attn[x, j] b_{N(x)_j} (na*_av; QGRAD with attn = dS, b = k)."""
    _check_hm(attn, b)
    K = _window_size(kernel_size, b.dim() - 3)
    if attn.shape != b.shape[:-1] + (K,):
        raise ValueError("attn must be [B, heads, (T,) H, W, prod(kernel_size)]")
    p = make_problem_hm(b.shape, b.shape[-1], kernel_size, dilation)
    if out is None:
        out = torch.empty_like(b)
    _check_hm_buf(out, "out", b.shape, b)
    _check(load().na_av(ctypes.byref(p), _ptr(attn), _ptr(b), float(alpha), _ptr(out),
                        _stream_handle(b.device)))
    return out


def na_av_inverse(attn: torch.Tensor, a: torch.Tensor, kernel_size, dilation=1,
                  alpha: float = 1.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out_y = alpha * sum over the queries x whose window holds y of attn[x, j] a_x
    (KGRAD with attn = dS, a = q; VGRAD with attn = P, a = dout)."""
    _check_hm(attn, a)
    K = _window_size(kernel_size, a.dim() - 3)
    if attn.shape != a.shape[:-1] + (K,):
        raise ValueError("attn must be [B, heads, (T,) H, W, prod(kernel_size)]")
    p = make_problem_hm(a.shape, a.shape[-1], kernel_size, dilation)
    if out is None:
        out = torch.empty_like(a)
    _check_hm_buf(out, "out", a.shape, a)
    _check(load().na_av_inverse(ctypes.byref(p), _ptr(attn), _ptr(a), float(alpha), _ptr(out),
                                _stream_handle(a.device)))
    return out


def na_softmax(attn: torch.Tensor, kernel_size, dilation=1,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Softmax of attn over its window axis (out may be attn itself)."""
    _check_hm(attn)
    p = make_problem_hm(attn.shape, 16, kernel_size, dilation)
    if attn.shape[-1] != _window_size(kernel_size, attn.dim() - 3):
        raise ValueError("the last axis of attn must hold prod(kernel_size) entries")
    if out is None:
        out = torch.empty_like(attn)
    _check_hm_buf(out, "out", attn.shape, attn)
    _check(load().na_softmax(ctypes.byref(p), _ptr(attn), _ptr(out), _stream_handle(attn.device)))
    return out


def na_softmax_bwd(probs: torch.Tensor, dprobs: torch.Tensor, kernel_size, dilation=1,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """probs * (dprobs - rowsum(probs * dprobs)) over the window axis (out may be dprobs)."""
    _check_hm(probs, dprobs)
    if probs.shape != dprobs.shape:
        raise ValueError("probs and dprobs must share their shape")
    p = make_problem_hm(probs.shape, 16, kernel_size, dilation)
    if probs.shape[-1] != _window_size(kernel_size, probs.dim() - 3):
        raise ValueError("the last axis must hold prod(kernel_size) entries")
    if out is None:
        out = torch.empty_like(probs)
    _check_hm_buf(out, "out", probs.shape, probs)
    _check(load().na_softmax_bwd(ctypes.byref(p), _ptr(probs), _ptr(dprobs), _ptr(out),
                                 _stream_handle(probs.device)))
    return out


def na_unfused_fwd(q, k, v, kernel_size, dilation=1, scale: Optional[float] = None,
                   probs: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   rpb: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None):
    """Unfused forward on head-major fp32 tensors: returns (probs, out)."""
    _check_hm(q, k, v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must share their shape")
    K = _window_size(kernel_size, q.dim() - 3)
    p = make_problem_hm(q.shape, q.shape[-1], kernel_size, dilation, scale)
    rp = _check_rpb(rpb, kernel_size, q.shape[1], q.dim() - 3, q)
    mp = _check_mask(mask, q, K)
    if probs is None:
        probs = _attn_like(q, K)
    if out is None:
        out = torch.empty_like(q)
    _check_hm_buf(probs, "probs", q.shape[:-1] + (K,), q)
    _check_hm_buf(out, "out", q.shape, q)
    _check(load().na_unfused_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), rp, mp,
                                 _ptr(probs), _ptr(out), _stream_handle(q.device)))
    return probs, out


def na_unfused_bwd(q, k, v, probs, dout, kernel_size, dilation=1, scale: Optional[float] = None,
                   dscores: Optional[torch.Tensor] = None, grads=None, want_rpb: bool = False,
                   workspace: Optional[torch.Tensor] = None):
    """Unfused backward of sum(out * dout): returns (dq, dk, dv), and the bias
    gradient as a fourth value when want_rpb."""
    _check_hm(q, k, v, probs, dout)
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout must share their shape")
    K = _window_size(kernel_size, q.dim() - 3)
    if probs.shape != q.shape[:-1] + (K,):
        raise ValueError("probs must be [B, heads, (T,) H, W, prod(kernel_size)]")
    p = make_problem_hm(q.shape, q.shape[-1], kernel_size, dilation, scale)
    if dscores is None:
        dscores = _attn_like(q, K)
    _check_hm_buf(dscores, "dscores", q.shape[:-1] + (K,), q)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_hm_buf(g, name, q.shape, q)
    drpb, ws_ptr, ws_n = None, None, 0
    if want_rpb:
        need = int(load().na_rpb_grad_workspace_bytes(ctypes.byref(p)))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _check_workspace(workspace, need, q.device)
        drpb = torch.empty(rpb_shape(kernel_size, q.shape[1], q.dim() - 3), dtype=torch.float32,
                           device=q.device)
        ws_ptr, ws_n = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(load().na_unfused_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(probs),
                                 _ptr(dout), _ptr(dscores), _ptr(dq), _ptr(dk), _ptr(dv),
                                 None if drpb is None else _ptr(drpb), ws_ptr, ws_n,
                                 _stream_handle(q.device)))
    return (dq, dk, dv, drpb) if want_rpb else (dq, dk, dv)
