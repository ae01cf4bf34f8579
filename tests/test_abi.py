"""CPU-only checks of the C ABI (include/na.h): the library loads, exports every
declared symbol, validates problems on the host, and its window helpers match
brute force. No call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

import oracle
from fwd_bwd_amd import na

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "na.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(na.lib_path()):
        from fwd_bwd_amd import build
        build.build()
    return na.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(na_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_matches_binding_list():
    assert declared_functions() == sorted(na.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", na.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for s in range(5):
        assert lib.na_status_string(s).decode().startswith("NA_")


def _p(shape=(1, 16, 16, 2, 16), dtype=None, kernel=(3, 3), dil=1, scale=None):
    import torch
    return na.make_problem(shape, dtype or torch.float32, kernel, dil, scale)


def test_check_problem_accepts_workloads():
    from fwd_bwd_amd.inputs import WORKLOADS
    for w in WORKLOADS.values():
        p = na.make_problem(w.shape, w.dtype, w.kernel, w.dilation, w.scale)
        assert na.check_problem(p) == na.NA_OK, w.name


@pytest.mark.parametrize("mutate,expect", [
    (lambda p: setattr(p, "ndim", 4), na.NA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "ndim", 1), na.NA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "dtype", 7), na.NA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "batch", 0), na.NA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "heads", 0), na.NA_ERR_INVALID_ARG),
    (lambda p: p.kernel.__setitem__(0, 0), na.NA_ERR_INVALID_ARG),
    (lambda p: p.kernel.__setitem__(1, 17), na.NA_ERR_INVALID_ARG),
    (lambda p: p.dilation.__setitem__(0, 0), na.NA_ERR_INVALID_ARG),
    (lambda p: p.dilation.__setitem__(0, 6), na.NA_ERR_INVALID_ARG),   # 16 // 6 = 2 < 3
    (lambda p: p.extent.__setitem__(1, 0), na.NA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "scale", float("nan")), na.NA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "scale", float("inf")), na.NA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "head_dim", 24), na.NA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "head_dim", 128), na.NA_ERR_UNSUPPORTED),
])
def test_check_problem_rejects(mutate, expect):
    p = _p()
    assert na.check_problem(p) == na.NA_OK
    mutate(p)
    assert na.check_problem(p) == expect


def test_dilated_kernel_limit():
    p = _p(shape=(1, 9, 16, 1, 16), kernel=(3, 3), dil=(3, 1))   # 9 // 3 = 3: fits
    assert na.check_problem(p) == na.NA_OK
    p = _p(shape=(1, 8, 16, 1, 16), kernel=(3, 3), dil=(3, 1))   # class of 2 < 3
    assert na.check_problem(p) == na.NA_ERR_INVALID_ARG


def test_fwd_bwd_reject_null_pointers_before_launch(lib):
    p = _p()
    fake = ctypes.c_void_p(1 << 20)
    args = [fake] * 5
    for i in range(5):
        a = list(args)
        a[i] = None
        assert lib.na_fwd(ctypes.byref(p), *a, None) == na.NA_ERR_INVALID_ARG
    # misaligned
    mis = ctypes.c_void_p((1 << 20) + 4)
    assert lib.na_fwd(ctypes.byref(p), mis, fake, fake, fake, fake, None) == na.NA_ERR_INVALID_ARG
    ws = na.bwd_workspace_bytes(p, na.NA_BWD_GATHER)
    bargs = [fake] * 9
    for i in range(9):
        a = list(bargs)
        a[i] = None
        assert lib.na_bwd(ctypes.byref(p), *a, fake, ws, 0, 0, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_bwd(ctypes.byref(p), *bargs, None, ws, 0, 0, None) == na.NA_ERR_WORKSPACE
    assert lib.na_bwd(ctypes.byref(p), *bargs, fake, ws - 1, 0, 0, None) == na.NA_ERR_WORKSPACE
    assert lib.na_bwd(ctypes.byref(p), *bargs, fake, ws, 5, 0, None) == na.NA_ERR_INVALID_ARG
    # a KV-parallel workspace grows with kv_splits
    wk = na.bwd_workspace_bytes(p, na.NA_BWD_KVPARALLEL, 3)
    assert lib.na_bwd(ctypes.byref(p), *bargs, fake, wk - 1, 1, 3, None) == na.NA_ERR_WORKSPACE
    bad = _p(kernel=(3, 19))
    assert lib.na_fwd(ctypes.byref(bad), *args, None) == na.NA_ERR_INVALID_ARG


def test_workspace_bytes():
    p = _p(shape=(2, 16, 16, 2, 16))
    rows = 2 * 256 * 2
    g = na.bwd_workspace_bytes(p, na.NA_BWD_GATHER)
    kv = na.bwd_workspace_bytes(p, na.NA_BWD_KVPARALLEL)
    assert g >= rows * 4 and g % 256 == 0
    assert kv >= g + rows * 16 * 4 and kv % 256 == 0
    assert na.bwd_workspace_bytes(p, 9) == 0


def test_window_helpers_match_oracle_and_brute_force(lib):
    for L in range(1, 21):
        for d in range(1, 4):
            if L // d < 1:
                continue
            for k in range(1, L // d + 1):
                for x in range(L):
                    s = na.window_start(L, k, d, x)
                    assert s == oracle.window_start(L, k, d, x), (L, k, d, x)
                for y in range(L):
                    # brute force: every query whose window contains y
                    att = [x for x in range(L) if x % d == y % d and
                           y in range(oracle.window_start(L, k, d, x),
                                      oracle.window_start(L, k, d, x) + d * k, d)]
                    first, last = na.inverse_window(L, k, d, y)
                    assert att == list(range(first, last + 1, d)), (L, k, d, y)
    assert na.window_start(5, 6, 1, 0) == -1
    with pytest.raises(na.NaError):
        na.inverse_window(5, 6, 1, 0)


# ----------------------------------------------------------------------------- unfused ops

def _hm_problem(shape=(2, 2, 16, 16, 16), kernel=(3, 3), dil=1):
    return na.make_problem_hm(shape, shape[-1], kernel, dil)


def test_unfused_entry_points_validate_on_host(lib):
    """Argument errors of the unfused ops come back before anything is launched."""
    p = _hm_problem()
    fake = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 4)
    # null / misaligned operands, non-finite alpha, misaligned bias table
    assert lib.na_qk(ctypes.byref(p), None, fake, 1.0, None, None, fake, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_qk(ctypes.byref(p), fake, fake, 1.0, None, None, mis, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_qk(ctypes.byref(p), fake, fake, float("nan"), None, None, fake, None) == \
        na.NA_ERR_INVALID_ARG
    assert lib.na_qk(ctypes.byref(p), fake, fake, 1.0, mis, None, fake, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_av(ctypes.byref(p), fake, None, 1.0, fake, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_av_inverse(ctypes.byref(p), fake, fake, 1.0, None, None) == na.NA_ERR_INVALID_ARG
    # the unfused ops are fp32 only
    b16 = _hm_problem()
    b16.dtype = na.NA_BF16
    assert lib.na_qk(ctypes.byref(b16), fake, fake, 1.0, None, None, fake, None) == na.NA_ERR_UNSUPPORTED
    # head_dim outside {16, 32, 64}: unsupported for the contractions
    odd = _hm_problem(shape=(1, 2, 16, 16, 24))
    assert lib.na_av(ctypes.byref(odd), fake, fake, 1.0, fake, None) == na.NA_ERR_UNSUPPORTED
    bad = _hm_problem(kernel=(3, 17))
    assert lib.na_softmax(ctypes.byref(bad), fake, fake, None) == na.NA_ERR_INVALID_ARG
    # the bias gradient needs its workspace
    need = lib.na_rpb_grad_workspace_bytes(ctypes.byref(p))
    assert lib.na_rpb_grad(ctypes.byref(p), fake, fake, None, need, None) == na.NA_ERR_WORKSPACE
    assert lib.na_rpb_grad(ctypes.byref(p), fake, fake, fake, need - 1, None) == na.NA_ERR_WORKSPACE
    args = [fake] * 9
    assert lib.na_unfused_bwd(ctypes.byref(p), *args, fake, fake, need - 1, None) == na.NA_ERR_WORKSPACE


def test_rpb_workspace_bytes(lib):
    # (batch 2 x heads 2) planes x one chunk of 256 tokens x (2*3-1)^2 offsets, fp32
    assert lib.na_rpb_grad_workspace_bytes(ctypes.byref(_hm_problem())) == 2 * 2 * 1 * 25 * 4
    # 3D, 3 chunks of a 600-token plane, offsets 5 * 9 * 9
    p = _hm_problem(shape=(1, 3, 4, 10, 15, 32), kernel=(3, 5, 5))
    assert lib.na_rpb_grad_workspace_bytes(ctypes.byref(p)) == 3 * 3 * 5 * 9 * 9 * 4
    assert na.rpb_shape((3, 5, 5), 3, 3) == (3, 5, 9, 9)


@pytest.mark.parametrize("extent,kernel,expect", [
    (40, 16, na.NA_OK),            # windows up to 16 fit every extent
    (33, 16, na.NA_OK),
    (33, 17, na.NA_ERR_UNSUPPORTED),  # a border walk of 34 points
    (64, 17, na.NA_OK),
    (100, 23, na.NA_ERR_UNSUPPORTED),
    (30, 23, na.NA_OK),            # class extents below 33 always fit
])
def test_window_limit(lib, extent, kernel, expect):
    """Windows whose walk near a border exceeds the kernels' 32-bit validity
    masks are rejected on the host, by na_check_problem and by the entry points."""
    p = _p(shape=(1, extent, 48, 1, 32), kernel=(kernel, 3))
    assert na.check_problem(p) == expect
    if expect != na.NA_OK:
        fake = ctypes.c_void_p(4096)
        assert lib.na_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, None) == expect


def test_source_hash_matches_tree(lib):
    from fwd_bwd_amd import build
    assert na.source_sha256() == build.source_sha256()


def test_noalloc_rejects_problems_beyond_its_array(lib):
    """na_bwd_noalloc keeps delta in a static array of NA_NOALLOC_MAX_ROWS rows:
    larger problems are refused on the host, before any HIP call."""
    assert na.NOALLOC_MAX_ROWS == 1 << 23
    p = _p(shape=(1, 1024, 1024, 9, 16), kernel=(3, 3))   # 9 * 2^20 rows
    fake = ctypes.c_void_p(4096)
    args = [ctypes.byref(p)] + [fake] * 9 + [None]
    assert lib.na_bwd_noalloc(*args) == na.NA_ERR_WORKSPACE
    p = _p(shape=(1, 1024, 1024, 8, 16), kernel=(3, 3))   # exactly 2^23 rows: accepted sizes
    assert na.check_problem(p) == na.NA_OK
    bad = [ctypes.byref(p)] + [fake] * 8 + [None, None]   # dv missing
    assert lib.na_bwd_noalloc(*bad) == na.NA_ERR_INVALID_ARG


def test_workspace_bytes_per_variant_and_copies(lib):
    """Gather: the delta rows; KV-parallel: delta plus max(kv_splits, 1) fp32
    accumulators, each region 256-byte aligned; a negative kv_splits is 0."""
    p = _p(shape=(2, 13, 17, 3, 32), kernel=(3, 5))
    rows = 2 * 13 * 17 * 3
    r256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    delta, acc = r256(rows * 4), rows * 32 * 4
    assert na.bwd_workspace_bytes(p, na.NA_BWD_GATHER, 0) == delta
    assert na.bwd_workspace_bytes(p, na.NA_BWD_GATHER, 5) == delta
    assert na.bwd_workspace_bytes(p, na.NA_BWD_KVPARALLEL, 0) == delta + r256(acc)
    assert na.bwd_workspace_bytes(p, na.NA_BWD_KVPARALLEL, 1) == delta + r256(acc)
    assert na.bwd_workspace_bytes(p, na.NA_BWD_KVPARALLEL, 4) == delta + r256(4 * acc)
    assert na.bwd_workspace_bytes(p, na.NA_BWD_KVPARALLEL, -1) == 0
    fake = ctypes.c_void_p(4096)
    args = [ctypes.byref(p)] + [fake] * 9 + [fake, ctypes.c_size_t(1 << 40), na.NA_BWD_KVPARALLEL,
                                             -1, None]
    assert lib.na_bwd(*args) == na.NA_ERR_INVALID_ARG


def test_masked_entry_points_reject_a_null_mask(lib):
    """The window mask of the masked entry points is a byte array: a null
    pointer is refused before any launch, after the problem itself."""
    p = _p()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.na_fwd_masked(ctypes.byref(p), *[fake] * 5, None, None) == na.NA_ERR_INVALID_ARG
    ws = na.bwd_workspace_bytes(p, na.NA_BWD_GATHER)
    assert lib.na_bwd_masked(ctypes.byref(p), *[fake] * 9, fake, ws, 0, 0, None,
                             None) == na.NA_ERR_INVALID_ARG
    bad = _p(kernel=(3, 19))
    assert lib.na_fwd_masked(ctypes.byref(bad), *[fake] * 5, fake, None) == na.NA_ERR_INVALID_ARG
    # misaligned tensors and a short workspace are refused as for na_fwd / na_bwd
    mis = ctypes.c_void_p((1 << 20) + 4)
    assert lib.na_fwd_masked(ctypes.byref(p), mis, *[fake] * 4, fake, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_bwd_masked(ctypes.byref(p), *[fake] * 9, fake, 0, 0, 0, fake,
                             None) == na.NA_ERR_WORKSPACE


def test_framed_entry_points_reject_bad_frame_pointers(lib):
    """The per-coordinate window sizes of the framed entry points are an int32
    device array: a null or misaligned pointer is refused before any launch."""
    p = _p()
    fake = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 2)
    for fr in (None, mis):
        assert lib.na_fwd_framed(ctypes.byref(p), *[fake] * 5, fr, None) == na.NA_ERR_INVALID_ARG
        ws = na.bwd_workspace_bytes(p, na.NA_BWD_GATHER)
        assert lib.na_bwd_framed(ctypes.byref(p), *[fake] * 9, fake, ws, 0, 0, fr,
                                 None) == na.NA_ERR_INVALID_ARG
    # the problem is validated first
    bad = _p(kernel=(3, 19))
    assert lib.na_fwd_framed(ctypes.byref(bad), *[fake] * 5, fake, None) == na.NA_ERR_INVALID_ARG


def test_window_mask_checks_of_the_binding():
    """The binding refuses a window mask of the wrong shape, dtype or layout
    (the C ABI cannot see its size) before any call."""
    import torch
    q = torch.zeros((1, 4, 6, 7, 2, 16))
    good = torch.ones((4, 6, 7, 3 * 5 * 5), dtype=torch.uint8)
    assert na._check_window_mask(good, q, (3, 5, 5)) == good.data_ptr()
    for bad in (torch.ones((4, 6, 7, 74), dtype=torch.uint8),       # K of another window
                torch.ones((4, 6, 7, 75), dtype=torch.int32),       # not bytes
                torch.ones((4, 7, 6, 75), dtype=torch.uint8),       # grid axes swapped
                torch.ones((75, 4, 6, 7), dtype=torch.uint8).permute(1, 2, 3, 0),  # strided
                None):
        with pytest.raises(ValueError):
            na._check_window_mask(bad, q, (3, 5, 5))


def test_index_mask_entry_point_rejects_bad_arguments_on_the_host(lib):
    """na_window_mask_from_indices reads only the grid fields of the problem
    and refuses a malformed grid, a negative slot count and null or misaligned
    pointers before any launch; the binding refuses indices that are not a
    contiguous int64 GPU tensor."""
    import torch
    fake = ctypes.c_void_p(1 << 20)
    p = _p()
    f = lib.na_window_mask_from_indices
    assert f(ctypes.byref(p), fake, -1, fake, fake, None) == na.NA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), None, 4, fake, fake, None) == na.NA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), fake, 4, None, fake, None) == na.NA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), fake, 4, fake, None, None) == na.NA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 4), 4, fake, fake,
             None) == na.NA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), fake, 4, fake, ctypes.c_void_p((1 << 20) + 2),
             None) == na.NA_ERR_INVALID_ARG
    for bad in (_p(kernel=(3, 17)), _p(kernel=(3, 9), dil=(1, 2)), _p(kernel=(0, 3))):
        assert f(ctypes.byref(bad), fake, 4, fake, fake, None) == na.NA_ERR_INVALID_ARG
    assert f(None, fake, 4, fake, fake, None) == na.NA_ERR_INVALID_ARG
    for idx in (torch.zeros((6, 7, 3), dtype=torch.int32), torch.zeros((6, 7, 3), dtype=torch.int64),
                torch.zeros((3, 6, 7), dtype=torch.int64).permute(1, 2, 0)):
        with pytest.raises(ValueError):
            na.na_window_mask_from_indices(idx, (3, 3))
