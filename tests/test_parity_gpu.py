"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs.

Bar (per output tensor Y in {out, lse, dq, dk, dv}):
    max |Y_gpu - Y_oracle| / max |Y_oracle| <= 1e-4 for fp32, 2e-2 for bf16.
Small cases are compared element by element on every output; the full-size
workloads are compared on sampled (b, token, head) units that include the grid
corners and borders.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from fwd_bwd_amd import na
from fwd_bwd_amd.inputs import WORKLOADS, make_inputs, make_random

pytestmark = pytest.mark.gpu

# fp16: outputs are rounded to binary16 (relative step 2^-11 ~ 4.9e-4) after fp32
# accumulation; four rounding steps of the largest output is the bar.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 2e-3}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    na.load()   # raises if the HIP library is not built: there is no fallback


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    return err / scale if scale > 0 else err


def np64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


# backward variants under test: (na_bwd variant, kv_splits); "kvdet" is the
# KV-parallel backward with bounded, bitwise-reproducible accumulator copies
VARIANTS = {"gather": ("gather", 0), "kvparallel": ("kvparallel", 0), "kvdet": ("kvparallel", 2)}


def gpu_run(q, k, v, dout, kernel, dil, scale, variant="gather"):
    dev = torch.device("cuda:0")
    qd, kd, vd, dd = (t.to(dev) for t in (q, k, v, dout))
    out, lse = na.na_fwd(qd, kd, vd, kernel, dil, scale)
    var, splits = VARIANTS[variant]
    dq, dk, dv = na.na_bwd(qd, kd, vd, out, dd, lse, kernel, dil, scale, variant=var,
                           kv_splits=splits)
    torch.cuda.synchronize()
    return {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def oracle_full(q, k, v, dout, kernel, dil, scale):
    args = [np64(t) for t in (q, k, v)]
    out, lse = oracle.na_fwd(*args, kernel, dil, scale)
    dq, dk, dv = oracle.na_bwd(*args, np64(dout), kernel, dil, scale)
    return {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def compare(got, ref, dtype, label):
    tol = TOL[dtype]
    errs = {}
    for name in ref:
        errs[name] = rel_err(np64(got[name]), ref[name])
    say(label, {k: f"{v:.2e}" for k, v in errs.items()})
    for name, e in errs.items():
        assert e <= tol, (label, name, e)
    return errs


# ----------------------------------------------------------------------------- small cases
# shapes span several wave tiles (8x8 per wave) with ragged tails, both dtypes,
# all head dims, dilation, batch > 1, k = 1, kernel = grid, windows of even size.
SMALL = [
    # (shape [B,(T,)H,W,h,D], kernel, dilation, dtype)
    ((1, 16, 16, 2, 16), (3, 3), 1, torch.float32),
    ((1, 19, 23, 2, 32), (5, 7), 1, torch.float32),
    ((2, 13, 17, 3, 16), (3, 3), (2, 3), torch.float32),
    ((1, 20, 20, 1, 64), (9, 9), 1, torch.float32),
    ((1, 7, 9, 2, 32), (7, 9), 1, torch.float32),        # kernel = grid: dense attention
    ((1, 11, 10, 2, 32), (1, 1), 1, torch.float32),      # k = 1
    ((1, 12, 11, 1, 16), (4, 2), 1, torch.float32),      # even kernels
    ((1, 3, 5, 1, 16), (3, 5), 1, torch.float32),        # grid smaller than a wave tile
    ((1, 5, 11, 13, 2, 32), (3, 5, 5), 1, torch.float32),
    ((1, 6, 9, 10, 2, 16), (3, 3, 3), (2, 1, 2), torch.float32),
    ((2, 4, 9, 8, 1, 64), (3, 3, 3), 1, torch.float32),
    ((1, 19, 23, 2, 32), (5, 7), 1, torch.bfloat16),
    ((1, 6, 10, 9, 2, 32), (5, 7, 7), 1, torch.bfloat16),
    ((2, 26, 27, 2, 64), (5, 5), 2, torch.bfloat16),
    # several 16 x 16 tiles with ragged tails (register-resident kernels; for
    # k = 9 the tiles at the grid border take the split dk/dv kernel)
    ((1, 40, 37, 2, 32), (9, 9), 1, torch.float32),
    ((1, 35, 33, 2, 16), (5, 5), (1, 2), torch.float32),
    ((1, 3, 37, 35, 1, 32), (3, 5, 5), 1, torch.float32),
    ((1, 7, 18, 20, 2, 16), (5, 3, 3), (1, 2, 1), torch.float32),
    # longer inverse walks at the borders: 3D walk 4 whose border tiles need 5
    # (split kernel), 2D head_dim 16 with k = 9 (split kernel for walks 6, 7),
    # 2D k = 7 (a border launch of walk 5), batch 2
    ((1, 5, 40, 36, 1, 32), (3, 7, 7), 1, torch.float32),
    ((1, 34, 35, 2, 16), (9, 9), 1, torch.float32),
    ((2, 33, 30, 1, 32), (7, 7), 1, torch.float32),
    # border tiles by class next to interior tiles: a longer inverse walk along
    # H only, along W only, and along both (corners), each its own launch
    ((1, 64, 56, 1, 32), (9, 9), 1, torch.float32),
    ((1, 64, 56, 1, 32), (9, 9), 1, torch.float16),
    ((1, 4, 48, 40, 1, 32), (3, 5, 5), 1, torch.float32),
    # the same on grids with several planes and a 7-wide window (walk 6 at the
    # border, one workgroup per CU)
    ((1, 3, 64, 56, 1, 32), (3, 7, 7), 1, torch.float32),
    ((1, 3, 64, 56, 1, 32), (3, 7, 7), 1, torch.bfloat16),
    # degenerate shapes: a 3D grid of one plane (k_t = 1), a window spanning the
    # whole extent along one axis only, a dilation that leaves every residue
    # class exactly one window long
    ((1, 1, 40, 37, 2, 32), (1, 9, 9), 1, torch.float32),
    ((1, 9, 30, 1, 32), (9, 5), 1, torch.float32),
    ((1, 18, 18, 1, 16), (3, 3), 6, torch.float32),
    # fp16: 2D, 3D, dilation, every head_dim (head_dim 16: the fp32 kernels after
    # conversion; 32 and 64: the 16-bit MFMA kernels)
    ((1, 19, 23, 2, 32), (5, 7), 1, torch.float16),
    ((1, 5, 18, 20, 2, 16), (3, 5, 5), 1, torch.float16),
    ((2, 26, 27, 2, 64), (5, 5), 2, torch.float16),
    ((1, 40, 37, 2, 32), (9, 9), 1, torch.float16),
    # 16-bit MFMA kernels: 2D with several tiles and ragged tails, 3D, dilation
    ((1, 40, 37, 2, 32), (9, 9), 1, torch.bfloat16),
    ((1, 3, 37, 35, 1, 32), (3, 5, 5), 1, torch.float16),
    ((1, 5, 40, 36, 1, 32), (3, 7, 7), 1, torch.bfloat16),
    ((1, 35, 33, 2, 32), (5, 5), (1, 2), torch.float16),
    # 16-bit MFMA kernels with wider slab rows: up to 32 points (k = 13, 17 and a
    # 3D 11 x 11 window) and up to 48 (k = 21; inverse walks up to 44 columns)
    ((1, 44, 41, 2, 32), (13, 13), 1, torch.bfloat16),
    ((1, 40, 38, 1, 64), (17, 15), 1, torch.float16),
    ((1, 3, 30, 29, 1, 32), (3, 11, 11), 1, torch.float16),
    ((1, 50, 48, 1, 32), (21, 21), 1, torch.bfloat16),
    ((1, 46, 49, 1, 64), (19, 21), 1, torch.float16),
    # 16-bit MFMA kernels on the degenerate and dilated shapes: dilation along
    # T and H of a 3D grid, kernel = grid (dense attention), k = 1, even kernels
    ((1, 6, 20, 18, 2, 32), (3, 5, 5), (2, 2, 1), torch.bfloat16),
    ((1, 7, 9, 2, 32), (7, 9), 1, torch.bfloat16),
    ((1, 11, 10, 2, 64), (1, 1), 1, torch.float16),
    ((1, 12, 11, 1, 32), (4, 2), 1, torch.float16),
]


def _id(c):
    shape, k, d, dt = c
    return f"{'x'.join(map(str, shape))}-k{'x'.join(map(str, k))}-d{d}-{str(dt)[6:]}"


@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
@pytest.mark.parametrize("variant", ["gather", "kvparallel", "kvdet"])
def test_small_cases_match_oracle(case, variant):
    shape, kernel, dil, dtype = case
    say("case", _id(case), variant)
    q, k, v, dout = make_random(shape, dtype, seed=zlib.crc32(_id(case).encode()) % 1000)
    scale = shape[-1] ** -0.5
    got = gpu_run(q, k, v, dout, kernel, dil, scale, variant)
    ref = oracle_full(q, k, v, dout, kernel, dil, scale)
    compare(got, ref, dtype, f"{_id(case)} {variant}")


# Scales other than head_dim^-0.5 (the ABI takes any finite one): negative
# (the 16-bit forward flips the queries' signs then), zero (uniform weights,
# dq = dk = 0 exactly), large (peaked softmax: the lazy rescaling of the
# 16-bit forward and the per-plane rescale of the fp32 one take many steps)
# and tiny, on one case of each kernel family: fp32 register-resident 2D and
# 3D, the fp32 split kernels (head_dim 64), the 16-bit MFMA kernels at head_dim
# 32 (2D, 3D) and 64 (dilated).
SCALE_CASES = [
    ((1, 40, 37, 2, 32), (9, 9), 1, torch.float32),
    ((1, 3, 37, 35, 1, 32), (3, 5, 5), 1, torch.float32),
    ((1, 20, 20, 1, 64), (9, 9), 1, torch.float32),
    ((1, 40, 37, 2, 32), (9, 9), 1, torch.bfloat16),
    ((1, 3, 37, 35, 1, 32), (3, 5, 5), 1, torch.float16),
    ((2, 26, 27, 2, 64), (5, 5), 2, torch.float16),
]


@pytest.mark.parametrize("scale", [-0.7, 0.0, 2.5, 1e-3])
@pytest.mark.parametrize("case", SCALE_CASES, ids=[_id(c) for c in SCALE_CASES])
def test_other_scales_match_oracle(case, scale):
    shape, kernel, dil, dtype = case
    say("case", _id(case), "scale", scale)
    q, k, v, dout = make_random(shape, dtype, seed=zlib.crc32(_id(case).encode()) % 1000 + 7)
    got = gpu_run(q, k, v, dout, kernel, dil, scale, "gather")
    ref = oracle_full(q, k, v, dout, kernel, dil, scale)
    errs = compare(got, ref, dtype, f"{_id(case)} scale {scale}")
    if scale == 0.0:
        # uniform weights over each window: lse = log(window size), no q / k gradient
        assert np.all(np64(got["dq"]) == 0) and np.all(np64(got["dk"]) == 0)
        assert errs["lse"] <= 1e-6


def test_kvparallel_with_a_negative_scale():
    shape, kernel, dil, dtype = (2, 14, 15, 2, 32), (5, 7), (1, 2), torch.float32
    q, k, v, dout = make_random(shape, dtype, seed=19)
    for variant in ("kvparallel", "kvdet"):
        got = gpu_run(q, k, v, dout, kernel, dil, -0.4, variant)
        ref = oracle_full(q, k, v, dout, kernel, dil, -0.4)
        compare(got, ref, dtype, f"negative scale {variant}")


def test_first_workload_full_and_dout_ones():
    """The 16x16 fp32 workload, every output, dout = ones as in the issue's script."""
    w = WORKLOADS["2d_16x16_k3_h2_d16_f32"]
    q, k, v, dout = make_inputs(w, seed=0)
    for variant in ("gather", "kvparallel"):
        got = gpu_run(q, k, v, dout, w.kernel, w.dilation, w.the_scale, variant)
        ref = oracle_full(q, k, v, dout, w.kernel, w.dilation, w.the_scale)
        compare(got, ref, w.dtype, f"{w.name} {variant}")


def test_gather_backward_is_deterministic():
    shape, kernel = (1, 4, 21, 19, 2, 32), (3, 5, 5)
    q, k, v, dout = (t.cuda() for t in make_random(shape, torch.float32, seed=11))
    out, lse = na.na_fwd(q, k, v, kernel)
    a = na.na_bwd(q, k, v, out, dout, lse, kernel)
    b = na.na_bwd(q, k, v, out, dout, lse, kernel)
    out2, lse2 = na.na_fwd(q, k, v, kernel)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_split_entry_points_equal_na_bwd():
    shape, kernel = (1, 17, 18, 2, 32), (5, 5)
    q, k, v, dout = (t.cuda() for t in make_random(shape, torch.float32, seed=12))
    out, lse = na.na_fwd(q, k, v, kernel)
    dq, dk, dv = na.na_bwd(q, k, v, out, dout, lse, kernel)
    dq2, delta = na.na_bwd_dq(q, k, v, out, dout, lse, kernel)
    dk2, dv2 = na.na_bwd_dkdv(q, k, v, dout, lse, delta, kernel)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    ref_delta = (dout.double() * out.double()).sum(-1)
    assert torch.allclose(delta.double(), ref_delta, rtol=1e-5, atol=1e-5)


def test_kvparallel_matches_gather():
    shape, kernel, dil = (2, 14, 15, 2, 32), (5, 7), (1, 2)
    q, k, v, dout = (t.cuda() for t in make_random(shape, torch.float32, seed=13))
    out, lse = na.na_fwd(q, k, v, kernel, dil)
    a = na.na_bwd(q, k, v, out, dout, lse, kernel, dil, variant="gather")
    b = na.na_bwd(q, k, v, out, dout, lse, kernel, dil, variant="kvparallel")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert rel_err(np64(x), np64(y)) < 1e-5


@pytest.mark.parametrize("case", [((1, 40, 37, 2, 32), (9, 9), 1, torch.float32),
                                  ((1, 5, 21, 19, 2, 32), (3, 5, 5), 1, torch.float32),
                                  ((2, 26, 27, 2, 64), (5, 5), 2, torch.bfloat16)],
                         ids=lambda c: _id(c))
def test_kvparallel_with_copies_is_bitwise_reproducible(case):
    """kv_splits >= 1: exact per-tile sums and ordered copies give the same
    bits on every run, for any number of copies, and match the gather."""
    shape, kernel, dil, dtype = case
    q, k, v, dout = (t.cuda() for t in make_random(shape, dtype, seed=16))
    out, lse = na.na_fwd(q, k, v, kernel, dil)
    ref = na.na_bwd(q, k, v, out, dout, lse, kernel, dil)
    for splits in (1, 3, 64):
        a = na.na_bwd(q, k, v, out, dout, lse, kernel, dil, variant="kvparallel", kv_splits=splits)
        b = na.na_bwd(q, k, v, out, dout, lse, kernel, dil, variant="kvparallel", kv_splits=splits)
        torch.cuda.synchronize()
        for name, x, y, r in zip(("dq", "dk", "dv"), a, b, ref):
            assert torch.equal(x, y), (splits, name)
            assert rel_err(np64(x), np64(r)) <= TOL[dtype], (splits, name)


def test_autograd_wrapper():
    shape, kernel = (1, 10, 12, 2, 16), (3, 5)
    q, k, v, dout = make_random(shape, torch.float32, seed=14)
    qd, kd, vd = (t.cuda().requires_grad_() for t in (q, k, v))
    o = na.neighborhood_attention(qd, kd, vd, kernel)
    o.backward(dout.cuda())
    ref = oracle_full(q, k, v, dout, kernel, 1, shape[-1] ** -0.5)
    got = {"out": o, "dq": qd.grad, "dk": kd.grad, "dv": vd.grad}
    compare(got, {n: ref[n] for n in got}, torch.float32, "autograd")


def test_autograd_on_views_of_a_fused_projection():
    """q, k, v as non-contiguous views of one [.., 3, heads, D] projection: the
    forward makes contiguous copies and the backward must use the same ones."""
    shape, kernel = (1, 10, 12, 2, 32), (3, 5)
    g = torch.Generator().manual_seed(15)
    qkv = torch.randn(shape[:-2] + (3,) + shape[-2:], generator=g)
    dout = torch.randn(shape, generator=g)
    x = qkv.cuda().requires_grad_()
    q, k, v = x.unbind(-3)
    assert not q.is_contiguous()
    o = na.neighborhood_attention(q, k, v, kernel)
    o.backward(dout.cuda())
    ref = oracle_full(*(t.contiguous() for t in qkv.unbind(-3)), dout, kernel, 1,
                      shape[-1] ** -0.5)
    got = {"out": o, "dq": x.grad[..., 0, :, :], "dk": x.grad[..., 1, :, :],
           "dv": x.grad[..., 2, :, :]}
    compare(got, {n: ref[n] for n in got}, torch.float32, "autograd on views")


# ----------------------------------------------------------------------------- full-size workloads

def _axis_strata(n, k, d, rng):
    """Coordinates along one axis, one per stratum: every coordinate of the two
    border bands (width k*d: where windows are shifted and inverse windows are
    irregular, the keys of the border-class launches), then one interior
    coordinate per residue mod 16*d (every position inside a tile of up to 16
    along the axis, in every dilation class)."""
    b = min(n, k * d)
    lo, hi = list(range(b)), list(range(max(b, n - b), n))
    inner = [c for c in range(b, n - b)]
    m = 16 * d
    mid = []
    for r in range(m):
        cs = [c for c in inner if c % m == r]
        if cs:
            mid.append(int(rng.choice(cs)))
    return lo, mid, hi


def sample_units(w, n_random=96, seed=0):
    """Flat (b, token, head) ids, stratified so that every launch and tile class
    contributes: for each axis, every coordinate of both border bands and one
    interior coordinate per tile residue (other axes random); two units in
    each of the 3^ndim border/interior region combinations (corners, edges,
    faces, interior); plus random units. Batch elements and heads are dealt
    round-robin, so each of them appears."""
    rng = np.random.default_rng(seed)
    grid = tuple(w.grid)
    strata = [_axis_strata(n, k, d, rng) for n, k, d in zip(grid, w.kernel, w.dilation)]
    pts = []
    for a, (lo, mid, hi) in enumerate(strata):
        for c in lo + mid + hi:
            p = [int(rng.integers(0, n)) for n in grid]
            p[a] = c
            pts.append(tuple(p))
    import itertools
    for combo in itertools.product(range(3), repeat=len(grid)):
        for _ in range(2):
            p = []
            for a, r in enumerate(combo):
                band = strata[a][r] or strata[a][1] or strata[a][0]
                p.append(int(rng.choice(band)))
            pts.append(tuple(p))
    ntok = int(np.prod(grid))
    ids = []
    for i, p in enumerate(pts):
        tok = int(np.ravel_multi_index(p, grid))
        b = i % w.batch
        h = (i // w.batch) % w.heads
        ids.append((b * ntok + tok) * w.heads + h)
    total = w.batch * ntok * w.heads
    ids.extend(rng.integers(0, total, n_random).tolist())
    return np.array(sorted(set(ids)), np.int64)


FULL = ["2d_1024x1024_k9_h8_d32_f32", "3d_16x256x256_k3x5x5_h8_d32_f32",
        "3d_b2_8x128x128_k5x7x7_h8_d32_bf16", "2d_b4_512x512_k13_d2_h4_d64_bf16",
        "2d_1024x1024_k9_h8_d32_f16", "3d_16x256x256_k3x5x5_h8_d32_f16"]


FULL_CASES = [(n, "gather") for n in FULL] + [("2d_1024x1024_k9_h8_d32_f32", "kvdet"),
                                              ("2d_1024x1024_k9_h8_d32_f32", "kvparallel"),
                                              ("3d_16x256x256_k3x5x5_h8_d32_f32", "kvdet"),
                                              ("2d_b4_512x512_k13_d2_h4_d64_bf16", "kvdet")]


@pytest.mark.parametrize("name,variant", FULL_CASES, ids=[f"{n}-{v}" for n, v in FULL_CASES])
def test_full_workload_sampled(name, variant):
    w = WORKLOADS[name]
    say("full workload", name, variant)
    q, k, v, dout = make_inputs(w, seed=0)
    got = gpu_run(q, k, v, dout, w.kernel, w.dilation, w.the_scale, variant)
    sel = sample_units(w)
    D = w.head_dim
    args = [np64(t) for t in (q, k, v)]
    o_ref, l_ref = oracle.na_fwd(*args, w.kernel, w.dilation, w.the_scale, sel=sel)
    dq_ref, dk_ref, dv_ref = oracle.na_bwd(*args, np64(dout), w.kernel, w.dilation, w.the_scale,
                                           sel=sel)
    pick = lambda t: np64(t).reshape(-1, D)[sel]  # noqa: E731
    got_s = {"out": pick(got["out"]), "lse": np64(got["lse"]).reshape(-1)[sel],
             "dq": pick(got["dq"]), "dk": pick(got["dk"]), "dv": pick(got["dv"])}
    ref_s = {"out": o_ref, "lse": l_ref, "dq": dq_ref, "dk": dk_ref, "dv": dv_ref}
    compare(got_s, ref_s, w.dtype, f"{name} sampled({sel.size})")
    # properties that hold at any size, checked on the whole tensors
    axes = tuple(range(1, 1 + w.ndim))
    dv_sum = got["dv"].double().sum(axes)
    do_sum = torch.as_tensor(dout).double().sum(axes).to(dv_sum.device)
    assert rel_err(dv_sum.cpu().numpy(), do_sum.cpu().numpy()) < TOL[w.dtype]
    # sum over keys of dk is 0 for every (b, head, channel): the rows of dS sum
    # to zero because delta = rowsum(dO o O) = sum_j P_j dP_j. Rounding of the
    # stored dk adds up like a random walk, so the bound is tol * ||dk||_2.
    dk = got["dk"].double()
    dk_sum = dk.sum(axes).abs()
    dk_l2 = dk.square().sum(axes).sqrt()
    assert bool((dk_sum <= TOL[w.dtype] * dk_l2).all()), float((dk_sum / dk_l2).max())
    assert torch.isfinite(got["dq"]).all() and torch.isfinite(got["dk"]).all()
