"""GPU parity of the unfused ops (na_qk, window softmax, na_av, the inverse
sum and their forward / backward compositions), through the C ABI, against
the fp64 CPU oracle on the same seeded head-major inputs.

Bar: max |Y_gpu - Y_oracle| / max |Y_oracle| <= 1e-4 per output (fp32).
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

TOL = 1e-4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    na.load()


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


def check(got, ref, label, tol=TOL):
    errs = {n: rel_err(np64(got[n]), ref[n]) for n in ref}
    say(label, {n: f"{e:.2e}" for n, e in errs.items()})
    for n, e in errs.items():
        assert e <= tol, (label, n, e)


# (head-major shape [B, heads, (T,) H, W, D], kernel, dilation)
SMALL = [
    ((1, 2, 16, 16, 16), (3, 3), 1),
    ((1, 2, 19, 23, 32), (5, 7), 1),
    ((2, 3, 13, 17, 16), (3, 3), (2, 3)),
    ((1, 1, 20, 20, 64), (9, 9), 1),
    ((1, 2, 7, 9, 32), (7, 9), 1),           # kernel = grid
    ((1, 2, 11, 10, 32), (1, 1), 1),         # k = 1
    ((1, 1, 12, 11, 16), (4, 2), 1),         # even kernels
    ((1, 2, 40, 37, 32), (9, 9), 1),
    ((1, 2, 35, 33, 16), (5, 5), (1, 2)),
    ((1, 1, 70, 68, 32), (9, 9), 1),
    ((1, 2, 5, 11, 13, 32), (3, 5, 5), 1),
    ((1, 2, 6, 9, 10, 16), (3, 3, 3), (2, 1, 2)),
    ((1, 1, 3, 37, 35, 32), (3, 5, 5), 1),
    ((1, 1, 5, 40, 36, 32), (3, 7, 7), 1),
    ((2, 1, 4, 9, 8, 64), (3, 3, 3), 1),
]


def _id(c):
    shape, k, d = c
    return f"{'x'.join(map(str, shape))}-k{'x'.join(map(str, k))}-d{d}"


def _seed(c):
    return zlib.crc32(_id(c).encode()) % 1000


@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
def test_unfused_fwd_bwd_matches_oracle(case):
    shape, kernel, dil = case
    say("case", _id(case))
    q, k, v, dout = make_random(shape, torch.float32, seed=_seed(case))
    scale = shape[-1] ** -0.5
    dev = torch.device("cuda:0")
    qd, kd, vd, dd = (t.to(dev) for t in (q, k, v, dout))
    probs, out = na.na_unfused_fwd(qd, kd, vd, kernel, dil, scale)
    dq, dk, dv = na.na_unfused_bwd(qd, kd, vd, probs, dd, kernel, dil, scale)
    torch.cuda.synchronize()
    args = [np64(t) for t in (q, k, v)]
    P, o = oracle.unfused_fwd(*args, kernel, dil, scale)
    gq, gk, gv = oracle.unfused_bwd(*args, P, np64(dout), kernel, dil, scale)
    check({"probs": probs, "out": out, "dq": dq, "dk": dk, "dv": dv},
          {"probs": P, "out": o, "dq": gq, "dk": gk, "dv": gv}, _id(case))


@pytest.mark.parametrize("case", SMALL[:4] + SMALL[10:12], ids=[_id(c) for c in SMALL[:4] + SMALL[10:12]])
def test_unfused_ops_on_arbitrary_operands(case):
    """Each op alone, with alpha != 1 and attention arrays that are not softmax
    rows (seeded normals), so a wrong window position cannot hide behind
    normalization."""
    shape, kernel, dil = case
    say("ops", _id(case))
    K = int(np.prod(kernel))
    a, b, _, _ = make_random(shape, torch.float32, seed=_seed(case) + 1)
    attn, g, _, _ = make_random(shape[:-1] + (K,), torch.float32, seed=_seed(case) + 2)
    dev = torch.device("cuda:0")
    ad, bd, atd, gd = (t.to(dev) for t in (a, b, attn, g))
    s = na.na_qk(ad, bd, kernel, dil, alpha=0.7)
    o = na.na_av(atd, bd, kernel, dil, alpha=-1.3)
    oi = na.na_av_inverse(atd, ad, kernel, dil, alpha=0.4)
    p = na.na_softmax(atd, kernel, dil)
    ds = na.na_softmax_bwd(p, gd, kernel, dil)
    torch.cuda.synchronize()
    A, B, AT, G = (np64(t) for t in (a, b, attn, g))
    Pref = oracle.softmax(AT)
    check({"qk": s, "av": o, "av_inverse": oi, "softmax": p, "softmax_bwd": ds},
          {"qk": oracle.na_qk(A, B, kernel, dil, 0.7),
           "av": oracle.na_av(AT, B, kernel, dil, -1.3),
           "av_inverse": oracle.na_av_inverse(AT, A, kernel, dil, 0.4),
           "softmax": Pref, "softmax_bwd": oracle.softmax_bwd(Pref, G)}, "ops " + _id(case))


def test_softmax_in_place_and_large_rows():
    """In-place softmax / softmax backward, and rows longer than the register
    path holds (K = 441 > 384 entries: the multi-pass kernel)."""
    dev = torch.device("cuda:0")
    for shape, kernel in [((1, 2, 9, 10, 16), (3, 5)), ((1, 1, 22, 23, 16), (21, 21))]:
        K = int(np.prod(kernel))
        x, g, _, _ = make_random(shape[:-1] + (K,), torch.float32, seed=K)
        x = 3.0 * x
        xd, gd = x.to(dev), g.to(dev)
        p = na.na_softmax(xd, kernel)
        xd2 = xd.clone()
        na.na_softmax(xd2, kernel, out=xd2)
        gd2 = gd.clone()
        na.na_softmax_bwd(p, gd2, kernel, out=gd2)
        torch.cuda.synchronize()
        Pref = oracle.softmax(np64(x))
        check({"p": p, "p_inplace": xd2, "ds_inplace": gd2},
              {"p": Pref, "p_inplace": Pref, "ds_inplace": oracle.softmax_bwd(Pref, np64(g))},
              f"softmax K={K}")


def test_unfused_matches_fused_path():
    """The unfused composition and the fused kernels compute the same function
    (same window rule): compared on one 2D and one 3D problem, the fused path
    fed the token-major copies of the same tensors."""
    dev = torch.device("cuda:0")
    for shape, kernel, dil in [((1, 2, 33, 35, 32), (7, 7), 1), ((1, 2, 5, 20, 18, 32), (3, 5, 5), 1)]:
        q, k, v, dout = (t.to(dev) for t in make_random(shape, torch.float32, seed=21))
        probs, out = na.na_unfused_fwd(q, k, v, kernel, dil)
        dq, dk, dv = na.na_unfused_bwd(q, k, v, probs, dout, kernel, dil)
        tm = lambda t: t.movedim(1, -2).contiguous()  # noqa: E731
        out2, lse = na.na_fwd(tm(q), tm(k), tm(v), kernel, dil)
        dq2, dk2, dv2 = na.na_bwd(tm(q), tm(k), tm(v), out2, tm(dout), lse, kernel, dil)
        torch.cuda.synchronize()
        for a, b in ((out, out2), (dq, dq2), (dk, dk2), (dv, dv2)):
            assert rel_err(np64(tm(a)), np64(b)) < 2e-4


def test_unfused_is_deterministic():
    dev = torch.device("cuda:0")
    shape, kernel = (1, 2, 4, 21, 19, 32), (3, 5, 5)
    q, k, v, dout = (t.to(dev) for t in make_random(shape, torch.float32, seed=22))
    p1, o1 = na.na_unfused_fwd(q, k, v, kernel)
    g1 = na.na_unfused_bwd(q, k, v, p1, dout, kernel)
    p2, o2 = na.na_unfused_fwd(q, k, v, kernel)
    g2 = na.na_unfused_bwd(q, k, v, p2, dout, kernel)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(o1, o2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_unfused_rejects_bf16_and_bad_shapes():
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 2, 8, 8, 16), device=dev)
    p = na.make_problem_hm(q.shape, 16, (3, 3))
    p.dtype = na.NA_BF16
    attn = torch.zeros((1, 2, 8, 8, 9), device=dev)
    status = na.load().na_qk(na.ctypes.byref(p), q.data_ptr(), q.data_ptr(), 1.0, None, None,
                             attn.data_ptr(), None)
    assert status == na.NA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        na.na_av(torch.zeros((1, 2, 8, 8, 8), device=dev), q, (3, 3))
    with pytest.raises(na.NaError):
        na.na_qk(q, q, (9, 3))   # window larger than the grid


# ----------------------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", ["2d_1024x1024_k9_h8_d32_f32", "3d_16x256x256_k3x5x5_h8_d32_f32"])
def test_unfused_full_workload_sampled(name):
    """The two fp32 benchmark workloads through the unfused path (head-major
    copies of the benchmark's inputs, launched as bench.py launches them),
    checked at sampled units: attention rows against softmax(scale * na_qk)
    of the oracle, out and the gradients against the oracle's fused functions
    (equal to the unfused composition by the oracle's own pins)."""
    from fwd_bwd_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    say("unfused full workload", name)
    q, k, v, dout = make_inputs(w, seed=0)
    dev = torch.device("cuda:0")
    hm = lambda t: t.movedim(-2, 1).contiguous().to(dev)  # noqa: E731
    qd, kd, vd, dd = (hm(t) for t in (q, k, v, dout))
    probs, out = na.na_unfused_fwd(qd, kd, vd, w.kernel, w.dilation, w.the_scale)
    dq, dk, dv = na.na_unfused_bwd(qd, kd, vd, probs, dd, w.kernel, w.dilation, w.the_scale)
    torch.cuda.synchronize()
    # sampled units: head-major ids (b, head, token), grid corners and edges plus random ones
    import itertools
    rng = np.random.default_rng(0)
    ntok = int(np.prod(w.grid))
    pts = sorted(set(itertools.product(*[(0, 1, g // 2, g - 2, g - 1) for g in w.grid])))
    ids = [((i % w.batch) * w.heads + (i * 7) % w.heads) * ntok + int(np.ravel_multi_index(p, w.grid))
           for i, p in enumerate(pts)]
    ids += rng.integers(0, w.batch * w.heads * ntok, 64).tolist()
    sel_hm = np.array(sorted(set(ids)), np.int64)
    b, rest = np.divmod(sel_hm, w.heads * ntok)
    h, tok = np.divmod(rest, ntok)
    sel_tm = (b * ntok + tok) * w.heads + h
    D = w.head_dim
    pick = lambda t, c: np64(t.reshape(-1, c)[torch.as_tensor(sel_hm, device=t.device)])  # noqa: E731
    Q, K_, V, DO = (np64(t) for t in (q, k, v, dout))
    qm, km = np.moveaxis(Q, -2, 1), np.moveaxis(K_, -2, 1)
    P_ref = oracle.softmax(oracle.na_qk(qm, km, w.kernel, w.dilation, w.the_scale, sel=sel_hm))
    o_ref, _ = oracle.na_fwd(Q, K_, V, w.kernel, w.dilation, w.the_scale, sel=sel_tm)
    g_ref = oracle.na_bwd(Q, K_, V, DO, w.kernel, w.dilation, w.the_scale, sel=sel_tm)
    check({"probs": pick(probs, w.window), "out": pick(out, D), "dq": pick(dq, D),
           "dk": pick(dk, D), "dv": pick(dv, D)},
          {"probs": P_ref, "out": o_ref, "dq": g_ref[0], "dk": g_ref[1], "dv": g_ref[2]},
          f"unfused {name} sampled({sel_hm.size})")


# ----------------------------------------------------------------------------- relative positional bias

RPB_CASES = [((1, 2, 19, 23, 32), (5, 7), 1), ((2, 3, 13, 17, 16), (3, 3), (2, 3)),
             ((1, 2, 40, 37, 32), (9, 9), 1), ((1, 1, 20, 20, 64), (9, 9), 1),
             ((1, 2, 5, 11, 13, 32), (3, 5, 5), 1), ((1, 2, 6, 9, 10, 16), (3, 3, 3), (2, 1, 2))]


@pytest.mark.parametrize("case", RPB_CASES, ids=[_id(c) for c in RPB_CASES])
def test_unfused_with_rpb_matches_oracle(case):
    """Scores plus a relative positional bias (register-tiled and plain score
    kernels), the whole unfused forward and backward with it, and the bias
    gradient, against the oracle."""
    shape, kernel, dil = case
    say("rpb", _id(case))
    q, k, v, dout = make_random(shape, torch.float32, seed=_seed(case) + 5)
    ndim = len(shape) - 3
    g = torch.Generator(device="cpu").manual_seed(_seed(case) + 6)
    rpb = torch.randn(na.rpb_shape(kernel, shape[1], ndim), generator=g)
    scale = shape[-1] ** -0.5
    dev = torch.device("cuda:0")
    qd, kd, vd, dd, rd = (t.to(dev) for t in (q, k, v, dout, rpb))
    s = na.na_qk(qd, kd, kernel, dil, alpha=0.8, rpb=rd)
    probs, out = na.na_unfused_fwd(qd, kd, vd, kernel, dil, scale, rpb=rd)
    dq, dk, dv, drpb = na.na_unfused_bwd(qd, kd, vd, probs, dd, kernel, dil, scale, want_rpb=True)
    torch.cuda.synchronize()
    Q, K_, V, DO, RP = (np64(t) for t in (q, k, v, dout, rpb))
    P, o = oracle.unfused_fwd(Q, K_, V, kernel, dil, scale, rpb=RP)
    gq, gk, gv, gr = oracle.unfused_bwd(Q, K_, V, P, DO, kernel, dil, scale, want_rpb=True)
    check({"qk_rpb": s, "probs": probs, "out": out, "dq": dq, "dk": dk, "dv": dv, "drpb": drpb},
          {"qk_rpb": oracle.na_qk(Q, K_, kernel, dil, 0.8, rpb=RP), "probs": P, "out": o,
           "dq": gq, "dk": gk, "dv": gv, "drpb": gr}, "rpb " + _id(case))


def test_rpb_grad_of_arbitrary_scores_and_determinism():
    """na_rpb_grad alone on seeded normals (not a softmax gradient), twice:
    equal to the oracle and bitwise equal between runs."""
    dev = torch.device("cuda:0")
    for shape, kernel, dil in [((2, 3, 33, 35, 16), (7, 5), (1, 2)), ((1, 2, 6, 20, 18, 32), (3, 5, 5), 1)]:
        K = int(np.prod(kernel))
        x, _, _, _ = make_random(shape[:-1] + (K,), torch.float32, seed=31)
        xd = x.to(dev)
        a = na.na_rpb_grad(xd, kernel, dil)
        b = na.na_rpb_grad(xd, kernel, dil)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        check({"drpb": a}, {"drpb": oracle.rpb_grad(np64(x), kernel, dil)}, f"rpb_grad {shape}")


# ----------------------------------------------------------------------------- masked windows

MASK_CASES = [((1, 2, 6, 20, 18, 32), (5, 3, 3), [1, 3, 3, 5, 5, 5]),   # register-tiled
              ((1, 2, 5, 11, 13, 32), (3, 5, 5), [1, 1, 3, 3, 3]),
              ((1, 1, 4, 9, 8, 64), (3, 3, 3), [3, 1, 1, 3])]            # plain kernels


@pytest.mark.parametrize("case", MASK_CASES, ids=[f"{c[0]}-k{c[1]}" for c in MASK_CASES])
def test_unfused_masked_windows_match_oracle(case):
    """Per-frame time windows (the requester's masked na3d_qk): scores masked to
    -inf outside each frame's own window, then the whole unfused forward and
    backward, against the oracle; one query fully masked (zero weights)."""
    shape, kernel, frame_k = case
    say("mask", shape, kernel, frame_k)
    q, k, v, dout = make_random(shape, torch.float32, seed=41)
    mask = oracle.frame_window_mask(shape[2:-1], kernel, frame_k)
    mask[1, 2, 3, :] = 0
    scale = shape[-1] ** -0.5
    dev = torch.device("cuda:0")
    qd, kd, vd, dd = (t.to(dev) for t in (q, k, v, dout))
    md = torch.from_numpy(mask).to(dev)
    s = na.na_qk(qd, kd, kernel, 1, alpha=scale, mask=md)
    probs, out = na.na_unfused_fwd(qd, kd, vd, kernel, 1, scale, mask=md)
    dq, dk, dv = na.na_unfused_bwd(qd, kd, vd, probs, dd, kernel, 1, scale)
    torch.cuda.synchronize()
    Q, K_, V, DO = (np64(t) for t in (q, k, v, dout))
    P, o = oracle.unfused_fwd(Q, K_, V, kernel, 1, scale, mask=mask)
    gq, gk, gv = oracle.unfused_bwd(Q, K_, V, P, DO, kernel, 1, scale)
    s_ref = oracle.mask_scores(oracle.na_qk(Q, K_, kernel, 1, scale), mask)
    s_gpu = np64(s)
    assert np.array_equal(np.isneginf(s_gpu), np.isneginf(s_ref))
    fin = np.isfinite(s_ref)
    check({"scores": s_gpu[fin], "probs": probs, "out": out, "dq": dq, "dk": dk, "dv": dv},
          {"scores": s_ref[fin], "probs": P, "out": o, "dq": gq, "dk": gk, "dv": gv},
          f"mask {shape}")
    assert torch.all(probs[:, :, 1, 2, 3] == 0) and torch.all(out[:, :, 1, 2, 3] == 0)


# ----------------------------------------------------------------------------- softmax fused into the score kernels

SMX_CASES = [((1, 2, 40, 37, 32), (9, 9), 1), ((2, 3, 13, 17, 16), (3, 3), (2, 3)),
             ((1, 2, 19, 23, 32), (5, 5), 1), ((1, 2, 5, 11, 13, 32), (3, 5, 5), 1)]


@pytest.mark.parametrize("case", SMX_CASES, ids=[_id(c) for c in SMX_CASES])
def test_qk_softmax_and_its_backward(case):
    """The window softmax taken inside the score kernel (single-plane grids;
    3D grids run the two ops in turn), with a bias and a mask, and AGRAD with
    the softmax backward in one kernel, against the oracle."""
    shape, kernel, dil = case
    say("qk_softmax", _id(case))
    ndim = len(shape) - 3
    a, b, g, _ = make_random(shape, torch.float32, seed=_seed(case) + 9)
    gen = torch.Generator(device="cpu").manual_seed(_seed(case) + 10)
    rpb = torch.randn(na.rpb_shape(kernel, shape[1], ndim), generator=gen)
    K = int(np.prod(kernel))
    mask = (torch.rand(shape[2:-1] + (K,), generator=gen) > 0.2).to(torch.uint8)
    mask[(0,) * ndim] = 0                      # one query with every entry masked
    dev = torch.device("cuda:0")
    ad, bd, gd, rd, md = (t.to(dev) for t in (a, b, g, rpb, mask))
    p = na.na_qk_softmax(ad, bd, kernel, dil, alpha=0.6, rpb=rd, mask=md)
    p2 = na.na_qk_softmax(ad, bd, kernel, dil, alpha=0.6)
    ds = na.na_qk_softmax_bwd(gd, bd, p2, kernel, dil)
    torch.cuda.synchronize()
    A, B, G, RP = (np64(t) for t in (a, b, g, rpb))
    P_ref = oracle.softmax(oracle.mask_scores(oracle.na_qk(A, B, kernel, dil, 0.6, rpb=RP),
                                              mask.numpy()))
    P2_ref = oracle.softmax(oracle.na_qk(A, B, kernel, dil, 0.6))
    dS_ref = oracle.softmax_bwd(np64(p2), oracle.na_qk(G, B, kernel, dil, 1.0))
    check({"probs": p, "probs_plain": p2, "dscores": ds},
          {"probs": P_ref, "probs_plain": P2_ref, "dscores": dS_ref}, "qk_softmax " + _id(case))


def test_rpb_softmax_in_the_score_kernel_repeats_bitwise():
    """The score kernel with the window softmax inside reads the bias table its
    workgroup copies to LDS; every wave must see the whole copy (a barrier
    between the copy and the reads). Ten runs on the 9 x 9 case: all bitwise
    equal, and equal to the oracle's probabilities."""
    shape, kernel, dil = (1, 2, 40, 37, 32), (9, 9), 1
    q, k, _, _ = make_random(shape, torch.float32, seed=43)
    g = torch.Generator(device="cpu").manual_seed(44)
    rpb = torch.randn(na.rpb_shape(kernel, shape[1], 2), generator=g)
    dev = torch.device("cuda:0")
    qd, kd, rd = (t.to(dev) for t in (q, k, rpb))
    scale = shape[-1] ** -0.5
    runs = [na.na_qk_softmax(qd, kd, kernel, dil, alpha=scale, rpb=rd) for _ in range(10)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert torch.equal(r, runs[0])
    P, _ = oracle.unfused_fwd(np64(q), np64(k), np64(k), kernel, dil, scale, rpb=np64(rpb))
    check({"probs": runs[0]}, {"probs": P}, "rpb softmax repeats")
