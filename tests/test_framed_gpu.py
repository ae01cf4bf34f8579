"""GPU parity of the fused kernels with windows restricted along the outermost
axis (na_fwd_framed / na_bwd_framed): the requester's per-frame time kernel on
3D grids, a per-row window on 2D grids. The reference is the oracle's masked
unfused path (scores outside the restricted windows set to -inf before the
window softmax) with the mask from oracle.outer_window_mask, on the same
seeded inputs; lse is the log-sum-exp of the oracle's masked scores.

Bar as for the unmasked parity tests (per tensor, max abs error over max abs
reference value): 1e-4 fp32, 2e-2 bf16, 2e-3 fp16. A query whose window is
masked away entirely must give a zero output and lse = -inf.
"""
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


# (shape [B, (T,) H, W, heads, D], kernel, dilation, dtype, sizes along the outermost axis)
CASES = [
    # the unfused path's per-frame cases, now through the fused kernels
    ((1, 6, 20, 18, 2, 32), (5, 3, 3), 1, torch.float32, [1, 3, 3, 5, 5, 5]),
    ((1, 5, 11, 13, 2, 32), (3, 5, 5), 1, torch.float32, [1, 1, 3, 3, 3]),
    ((1, 4, 9, 8, 1, 64), (3, 3, 3), 1, torch.float32, [3, 1, 1, 3]),      # split kernels
    ((1, 6, 20, 18, 2, 32), (5, 3, 3), 1, torch.bfloat16, [1, 3, 3, 5, 5, 0]),
    ((2, 5, 11, 13, 2, 64), (3, 5, 5), 1, torch.float16, [3, 1, 2, 3, 1]),
    # per-row windows on 2D grids, one row fully masked; dilation along the axis
    ((1, 40, 37, 2, 32), (9, 9), 1, torch.float32, None),
    ((1, 19, 23, 2, 16), (5, 7), (2, 1), torch.float32, None),
    ((1, 26, 27, 2, 64), (7, 5), 1, torch.bfloat16, None),
]


def _sizes(case):
    shape, kernel, dil, dtype, fk = case
    if fk is not None:
        return fk
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    fk = rng.integers(1, kernel[0] + 1, shape[1]).tolist()
    fk[shape[1] // 2] = 0
    return fk


def _id(c):
    shape, k, d, dt, _ = c
    return f"{'x'.join(map(str, shape))}-k{'x'.join(map(str, k))}-d{d}-{str(dt)[6:]}"


def reference(q, k, v, dout, kernel, dil, scale, fk):
    hm = lambda t: np.moveaxis(np64(t), -2, 1)  # noqa: E731  token-major -> head-major
    tm = lambda x: np.moveaxis(x, 1, -2)        # noqa: E731
    Q, K, V, DO = (hm(t) for t in (q, k, v, dout))
    mask = oracle.outer_window_mask(q.shape[1:-2], kernel, fk, dil)
    P, out = oracle.unfused_fwd(Q, K, V, kernel, dil, scale, mask=mask)
    dq, dk, dv = oracle.unfused_bwd(Q, K, V, P, DO, kernel, dil, scale)
    s = oracle.mask_scores(oracle.na_qk(Q, K, kernel, dil, scale), mask)
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.max(s, axis=-1, keepdims=True)
        lse = np.squeeze(m, -1) + np.log(np.sum(np.exp(s - np.where(np.isneginf(m), 0, m)), -1))
    lse = np.where(np.all(np.isneginf(s), -1), -np.inf, lse)
    return {"out": tm(out), "lse": np.moveaxis(lse, 1, -1), "dq": tm(dq), "dk": tm(dk),
            "dv": tm(dv)}, mask


@pytest.mark.parametrize("variant", [("gather", 0), ("kvparallel", 2)], ids=["gather", "kvdet"])
@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_framed_matches_masked_oracle(case, variant):
    shape, kernel, dil, dtype, _ = case
    fk = _sizes(case)
    say("framed", _id(case), fk, variant)
    q, k, v, dout = make_random(shape, dtype, seed=zlib.crc32(_id(case).encode()) % 997)
    scale = shape[-1] ** -0.5
    dev = torch.device("cuda:0")
    qd, kd, vd, dd = (t.to(dev) for t in (q, k, v, dout))
    frames = torch.tensor(fk, dtype=torch.int32, device=dev)
    out, lse = na.na_fwd_framed(qd, kd, vd, frames, kernel, dil, scale)
    dq, dk, dv = na.na_bwd_framed(qd, kd, vd, out, dd, lse, frames, kernel, dil, scale,
                                  variant=variant[0], kv_splits=variant[1])
    torch.cuda.synchronize()
    ref, mask = reference(q, k, v, dout, kernel, dil, scale, fk)
    got = {"out": np64(out), "lse": np64(lse), "dq": np64(dq), "dk": np64(dk), "dv": np64(dv)}
    errs = {n: rel_err(got[n], ref[n]) for n in ref}
    say("  ", {n: f"{e:.2e}" for n, e in errs.items()})
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)
    # fully masked queries: zero output, lse -inf; everything else finite
    dead = np.all(mask == 0, axis=-1)                       # [(T,) H, W]
    assert np.array_equal(np.isneginf(got["lse"]), np.broadcast_to(
        dead[None, ..., None], got["lse"].shape))
    assert np.all(got["out"][:, dead] == 0)
    for n in ("dq", "dk", "dv"):
        assert np.all(np.isfinite(got[n])), n


def test_full_frames_equal_unrestricted():
    """frame_kernel = kernel[0] everywhere changes nothing (bitwise)."""
    shape, kernel = (1, 5, 21, 19, 2, 32), (3, 5, 5)
    q, k, v, dout = (t.cuda() for t in make_random(shape, torch.float32, seed=23))
    frames = torch.full((shape[1],), kernel[0], dtype=torch.int32, device="cuda")
    o1, l1 = na.na_fwd(q, k, v, kernel)
    o2, l2 = na.na_fwd_framed(q, k, v, frames, kernel)
    g1 = na.na_bwd(q, k, v, o1, dout, l1, kernel)
    g2 = na.na_bwd_framed(q, k, v, o2, dout, l2, frames, kernel)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)
