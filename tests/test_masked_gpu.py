"""GPU parity of the fused entry points with arbitrary window masks
(na_fwd_masked / na_bwd_masked): per query token, any subset of its window's
keys. The reference is the oracle's masked unfused path (scores of dropped
keys set to -inf before the window softmax) with the same mask, on the same
seeded inputs; lse is the log-sum-exp of the oracle's masked scores.

Bar as for the unmasked parity tests (per tensor, max abs error over max abs
reference value): 1e-4 fp32, 2e-2 bf16, 2e-3 fp16. A query that keeps no key
must give a zero output and lse = -inf.
"""
import itertools
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from fwd_bwd_amd import na
from fwd_bwd_amd.inputs import make_random

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 2e-3}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    na.load()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    fin = np.isfinite(ref)
    scale = np.max(np.abs(ref[fin])) if fin.any() else 1.0
    return float(np.max(np.abs(got[fin] - ref[fin])) / scale) if fin.any() else 0.0


# (shape [B, (T,) H, W, heads, D], kernel, dilation, dtype)
CASES = [
    ((1, 40, 37, 2, 32), (9, 9), 1, torch.float32),
    ((2, 19, 23, 2, 16), (5, 7), (2, 1), torch.float32),
    ((1, 5, 11, 13, 2, 32), (3, 5, 5), 1, torch.float32),
    ((1, 6, 20, 18, 2, 32), (5, 3, 3), 1, torch.bfloat16),
    ((1, 26, 27, 2, 64), (7, 5), 1, torch.float16),
    ((1, 6, 9, 10, 1, 64), (3, 3, 3), (2, 1, 2), torch.float32),
    # the register-resident fp32 kernels with the mask: every square walk of
    # the interior tiles (3 x 3 to 9 x 9 windows, head_dim 16 and 32, dilation,
    # a 3D grid with head_dim 16), border tiles on the general kernels
    ((1, 21, 19, 2, 16), (3, 3), 1, torch.float32),
    ((1, 26, 27, 2, 32), (5, 5), (1, 2), torch.float32),
    ((2, 35, 33, 1, 32), (7, 7), 1, torch.float32),
    ((1, 4, 18, 20, 2, 16), (3, 3, 3), 1, torch.float32),
    ((1, 7, 12, 13, 2, 32), (3, 3, 3), (2, 1, 2), torch.float32),   # dilation along T and W
    # 16-bit tensors with head_dim 32 on the same register-resident kernels
    # (converted while staged): 2D interior walk 5 with border walks 6 and 7,
    # 2D 7 x 7 with its border classes, 3D walk 4 (masked border kernel) with
    # longer border walks, 3D with dilation
    ((1, 40, 37, 2, 32), (9, 9), 1, torch.bfloat16),
    ((2, 35, 33, 1, 32), (7, 7), 1, torch.float16),
    ((1, 6, 20, 18, 1, 32), (5, 7, 7), 1, torch.bfloat16),
    ((1, 7, 12, 13, 2, 32), (3, 3, 3), (2, 1, 2), torch.float16),
]


def _id(c):
    shape, k, d, dt = c
    return f"{'x'.join(map(str, shape))}-k{'x'.join(map(str, k))}-d{d}-{str(dt)[6:]}"


def random_mask(shape, kernel, seed, density=0.7):
    """A mask [(T,) H, W, K]: each window key kept with the given density,
    the middle token of the grid dropping every key."""
    grid = tuple(shape[1:-2])
    K = int(np.prod(kernel))
    rng = np.random.default_rng(seed)
    m = (rng.random(grid + (K,)) < density).astype(np.uint8)
    m[tuple(g // 2 for g in grid)] = 0
    return m


def reference(q, k, v, dout, kernel, dil, scale, mask):
    hm = lambda t: np.moveaxis(np64(t), -2, 1)  # noqa: E731  token-major -> head-major
    tm = lambda x: np.moveaxis(x, 1, -2)        # noqa: E731
    Q, K, V, DO = (hm(t) for t in (q, k, v, dout))
    P, out = oracle.unfused_fwd(Q, K, V, kernel, dil, scale, mask=mask)
    dq, dk, dv = oracle.unfused_bwd(Q, K, V, P, DO, kernel, dil, scale)
    s = oracle.mask_scores(oracle.na_qk(Q, K, kernel, dil, scale), mask)
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.max(s, axis=-1, keepdims=True)
        lse = np.squeeze(m, -1) + np.log(np.sum(np.exp(s - np.where(np.isneginf(m), 0, m)), -1))
    lse = np.where(np.all(np.isneginf(s), -1), -np.inf, lse)
    return {"out": tm(out), "lse": np.moveaxis(lse, 1, -1), "dq": tm(dq), "dk": tm(dk),
            "dv": tm(dv)}


def run_masked(q, k, v, dout, mask, kernel, dil, scale, variant, splits):
    dev = torch.device("cuda:0")
    qd, kd, vd, dd = (t.to(dev) for t in (q, k, v, dout))
    md = torch.from_numpy(mask).to(dev)
    out, lse = na.na_fwd_masked(qd, kd, vd, md, kernel, dil, scale)
    dq, dk, dv = na.na_bwd_masked(qd, kd, vd, out, dd, lse, md, kernel, dil, scale,
                                  variant=variant, kv_splits=splits)
    torch.cuda.synchronize()
    return {"out": np64(out), "lse": np64(lse), "dq": np64(dq), "dk": np64(dk), "dv": np64(dv)}


@pytest.mark.parametrize("variant", [("gather", 0), ("kvparallel", 0), ("kvparallel", 2)],
                         ids=["gather", "kvparallel", "kvdet"])
@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_masked_matches_oracle(case, variant):
    shape, kernel, dil, dtype = case
    seed = zlib.crc32(_id(case).encode()) % 991
    say("masked", _id(case), variant)
    q, k, v, dout = make_random(shape, dtype, seed=seed)
    mask = random_mask(shape, kernel, seed)
    scale = shape[-1] ** -0.5
    got = run_masked(q, k, v, dout, mask, kernel, dil, scale, *variant)
    ref = reference(q, k, v, dout, kernel, dil, scale, mask)
    errs = {n: rel_err(got[n], ref[n]) for n in ref}
    say("  ", {n: f"{e:.2e}" for n, e in errs.items()})
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)
    # a query that keeps no key: zero output, lse -inf; everything else finite
    dead = np.all(mask == 0, axis=-1)
    assert np.array_equal(np.isneginf(got["lse"]),
                          np.broadcast_to(dead[None, ..., None], got["lse"].shape))
    assert np.all(got["out"][:, dead] == 0)
    for n in ("dq", "dk", "dv"):
        assert np.all(np.isfinite(got[n])), n


@pytest.mark.parametrize("case", [CASES[0], CASES[3]], ids=[_id(CASES[0]), _id(CASES[3])])
def test_all_ones_mask_equals_unmasked(case):
    """Keeping every key gives the unmasked function (the masked entry points
    run other kernels, so within the parity bar rather than bitwise)."""
    shape, kernel, dil, dtype = case
    q, k, v, dout = (t.cuda() for t in make_random(shape, dtype, seed=29))
    ones = torch.ones(tuple(shape[1:-2]) + (int(np.prod(kernel)),), dtype=torch.uint8,
                      device="cuda")
    o1, l1 = na.na_fwd(q, k, v, kernel, dil)
    g1 = na.na_bwd(q, k, v, o1, dout, l1, kernel, dil)
    o2, l2 = na.na_fwd_masked(q, k, v, ones, kernel, dil)
    g2 = na.na_bwd_masked(q, k, v, o2, dout, l2, ones, kernel, dil)
    torch.cuda.synchronize()
    for name, x, y in zip(("out", "lse", "dq", "dk", "dv"), (o1, l1) + tuple(g1),
                          (o2, l2) + tuple(g2)):
        assert rel_err(np64(y), np64(x)) <= TOL[dtype], name


def test_masked_gather_is_deterministic():
    shape, kernel, dil, dtype = CASES[2]
    q, k, v, dout = (t.cuda() for t in make_random(shape, dtype, seed=31))
    mask = torch.from_numpy(random_mask(shape, kernel, 31)).cuda()
    o1, l1 = na.na_fwd_masked(q, k, v, mask, kernel, dil)
    o2, l2 = na.na_fwd_masked(q, k, v, mask, kernel, dil)
    g1 = na.na_bwd_masked(q, k, v, o1, dout, l1, mask, kernel, dil)
    g2 = na.na_bwd_masked(q, k, v, o1, dout, l1, mask, kernel, dil)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def test_mask_at_an_odd_address_matches_the_aligned_one():
    """The register-resident kernels read the mask in aligned dwords and take
    only 4-byte aligned masks; a mask starting at an odd byte goes to the
    general kernels. Both give the same function."""
    shape, kernel, dil, dtype = CASES[0]
    q, k, v, dout = (t.cuda() for t in make_random(shape, dtype, seed=37))
    m = torch.from_numpy(random_mask(shape, kernel, 37))
    store = torch.zeros(m.numel() + 1, dtype=torch.uint8, device="cuda")
    odd = store[1:].view(m.shape)
    odd.copy_(m.cuda())
    assert odd.data_ptr() % 4 != 0 and odd.is_contiguous()
    aligned = m.cuda().contiguous()
    res = []
    for mk in (aligned, odd):
        o, l = na.na_fwd_masked(q, k, v, mk, kernel, dil)
        g = na.na_bwd_masked(q, k, v, o, dout, l, mk, kernel, dil)
        res.append((o, l) + tuple(g))
    torch.cuda.synchronize()
    for name, x, y in zip(("out", "lse", "dq", "dk", "dv"), res[0], res[1]):
        assert rel_err(np64(y), np64(x)) <= TOL[dtype], name


# ---------------------------------------------------------------------------
# Index tensors of attended tokens (na_window_mask_from_indices): the mask
# bytes and the per-query counts of invalid slots are integer results, so the
# bar is bitwise equality with the oracle's window_mask_from_indices.

def window_tokens(grid, kernel, dil, x):
    """Flat indices of the tokens of query x's window (oracle window starts)."""
    axes = [[oracle.window_start(grid[a], kernel[a], dil[a], x[a]) + dil[a] * j
             for j in range(kernel[a])] for a in range(len(grid))]
    return [int(np.ravel_multi_index(c, grid)) for c in itertools.product(*axes)]


def random_indices(grid, kernel, dil, seed, invalid=False):
    """Per query token a random subset of its window's tokens, shuffled, one
    repeated, the rest of its m slots -1; the middle token lists nothing. With
    invalid, every seventh query also lists tokens outside its window, off
    the grid and below -1."""
    r = np.random.default_rng(seed)
    K, toks = int(np.prod(kernel)), int(np.prod(grid))
    idx = np.full(tuple(grid) + (K + 4,), -1, np.int64)
    for n, x in enumerate(np.ndindex(*grid)):
        if x == tuple(g // 2 for g in grid):
            continue
        win = window_tokens(grid, kernel, dil, x)
        keep = [t for t in win if r.random() < 0.6] or [win[-1]]
        slots = keep + [keep[0]]
        if invalid and n % 7 == 0:
            inside = set(win)
            outside = [t for t in range(toks) if t not in inside]
            slots += [toks + n, -2 - n] + ([int(r.choice(outside))] if outside else [])
        r.shuffle(slots)
        idx[x][:len(slots)] = slots
    return idx


def _dil(d, nd):
    return (d,) * nd if isinstance(d, int) else tuple(d)


INDEX_CASES = [((40, 37), (9, 9), 1), ((19, 23), (5, 7), (2, 1)), ((5, 11, 13), (3, 5, 5), 1),
               ((7, 12, 13), (3, 3, 3), (2, 1, 2)), ((4, 9), (1, 3), 1)]


@pytest.mark.parametrize("case", INDEX_CASES, ids=[f"{c[0]}-k{c[1]}-d{c[2]}" for c in INDEX_CASES])
def test_index_mask_matches_oracle(case):
    grid, kernel, dil = case
    dil = _dil(dil, len(grid))
    say("index mask", grid, kernel, dil)
    idx = random_indices(grid, kernel, dil, seed=len(grid) * 100 + kernel[-1], invalid=True)
    want_mask, want_bad = oracle.window_mask_from_indices(grid, kernel, idx, dil)
    assert want_bad.any()
    mask, bad = na.na_window_mask_from_indices(torch.from_numpy(idx).cuda(), kernel, dil,
                                               check=False)
    torch.cuda.synchronize()
    assert np.array_equal(mask.cpu().numpy(), want_mask)
    assert np.array_equal(bad.cpu().numpy(), want_bad)
    with pytest.raises(ValueError):
        na.na_window_mask_from_indices(torch.from_numpy(idx).cuda(), kernel, dil)


def test_index_mask_into_an_odd_address_and_no_slots():
    """The mask may start at any byte (the clearing kernel then stores bytes);
    zero slots per query drop every key."""
    grid, kernel = (19, 23), (5, 7)
    idx = torch.from_numpy(random_indices(grid, kernel, (1, 1), seed=3)).cuda()
    want, _ = na.na_window_mask_from_indices(idx, kernel)
    store = torch.full((want.numel() + 1,), 7, dtype=torch.uint8, device="cuda")
    odd = store[1:].view(want.shape)
    na.na_window_mask_from_indices(idx, kernel, mask=odd)
    torch.cuda.synchronize()
    assert odd.data_ptr() % 2 == 1 and torch.equal(odd, want) and int(store[0]) == 7
    none = torch.empty(grid + (0,), dtype=torch.int64, device="cuda")
    m0, b0 = na.na_window_mask_from_indices(none, kernel)
    torch.cuda.synchronize()
    assert not m0.any() and not b0.any()


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[7]],
                         ids=[_id(CASES[0]), _id(CASES[2]), _id(CASES[7])])
def test_indices_through_the_masked_kernels_match_oracle(case):
    """Index tensor -> mask (GPU) -> na_fwd_masked / na_bwd_masked (GPU)
    against the oracle's masked reference with the oracle's mask from the
    same indices."""
    shape, kernel, dil, dtype = case
    grid = tuple(shape[1:-2])
    d = _dil(dil, len(grid))
    seed = zlib.crc32(_id(case).encode()) % 997
    say("indices through masked kernels", _id(case))
    idx = random_indices(grid, kernel, d, seed)
    omask, _ = oracle.window_mask_from_indices(grid, kernel, idx, d)
    q, k, v, dout = make_random(shape, dtype, seed=seed)
    mask, _ = na.na_window_mask_from_indices(torch.from_numpy(idx).cuda(), kernel, dil)
    qd, kd, vd, dd = (t.cuda() for t in (q, k, v, dout))
    scale = shape[-1] ** -0.5
    out, lse = na.na_fwd_masked(qd, kd, vd, mask, kernel, dil, scale)
    dq, dk, dv = na.na_bwd_masked(qd, kd, vd, out, dd, lse, mask, kernel, dil, scale)
    torch.cuda.synchronize()
    got = {"out": np64(out), "lse": np64(lse), "dq": np64(dq), "dk": np64(dk), "dv": np64(dv)}
    ref = reference(q, k, v, dout, kernel, dil, scale, omask)
    for n in ref:
        assert rel_err(got[n], ref[n]) <= TOL[dtype], n
    assert np.array_equal(np.isneginf(got["lse"][0, ..., 0]), ~omask.any(-1))


def test_index_mask_at_the_3d_workload_size():
    """The 3D grid of the 16 x 256 x 256, 3 x 5 x 5 workload (about 1M query
    tokens, 75 slots each): every query lists its whole window in order except
    the key at place (token mod 75), which it replaces by -1, so the mask is
    all ones but that byte. Window starts per axis from the oracle; the
    indices are built on the GPU."""
    grid, kernel = (16, 256, 256), (3, 5, 5)
    K = 75
    dev = torch.device("cuda:0")
    axes = []
    for a in range(3):
        st = torch.tensor([oracle.window_start(grid[a], kernel[a], 1, x) for x in range(grid[a])],
                          device=dev)
        axes.append(st[:, None] + torch.arange(kernel[a], device=dev)[None, :])   # [L, k]
    t = axes[0][:, None, None, :, None, None]
    h = axes[1][None, :, None, None, :, None]
    w = axes[2][None, None, :, None, None, :]
    idx = ((t * grid[1] + h) * grid[2] + w).reshape(grid + (K,)).contiguous()
    drop = torch.arange(idx[..., 0].numel(), device=dev).reshape(grid) % K
    idx.scatter_(-1, drop[..., None], -1)
    mask, bad = na.na_window_mask_from_indices(idx, kernel)
    torch.cuda.synchronize()
    want = torch.ones_like(mask)
    want.scatter_(-1, drop[..., None], 0)
    assert not bad.any()
    assert torch.equal(mask, want)
    del idx, mask, want
    torch.cuda.empty_cache()
