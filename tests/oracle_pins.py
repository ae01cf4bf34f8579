"""Checks that pin the CPU oracle to facts other than itself.

Each check takes a bound oracle (``oracle.Bound``) so the same battery can be
run against the real oracle and against builds with a planted mistake. A
check raises AssertionError when the oracle disagrees with the fact it pins.

The facts (neighborhood attention as described in NATTEN issue #161, "Backward
pass is very slow towards much tokens and large kernels": scores over a window,
softmax over the window, weighted sum of values; backward = the gradients of
that composition):
  * window shape: along each axis exactly k in-bounds keys of the query's own
    residue class, containing the query, centered when that fits and otherwise
    the nearest such run (ties go to the lower start) -- brute force;
  * kernel = whole grid: NA is plain softmax attention, so torch's
    scaled_dot_product_attention (float64, CPU) and its autograd fix out,
    logsumexp and all three gradients;
  * the window weights of every query sum to one and lse lies in
    [max score, max score + ln K];
  * central finite differences of the oracle's own forward fix dq, dk, dv;
  * k = 1: out = v, lse = scale <q, k>, dq = dk = 0, dv = dout;
  * 3D with k_t = 1 is 2D NA applied to every frame;
  * with dilation d, each residue class is an undilated NA on its sub-grid;
  * heads and batch elements are independent (permutation equivariance);
  * sum_y dv_y = sum_x dout_x and sum_y dk_y = 0 per (b, head, channel);
  * mirroring an axis (odd k, d = 1) mirrors every output;
  * the score scale is linear: NA(c q; scale=1) = NA(q; scale=c).
"""
from __future__ import annotations

import itertools

import numpy as np
import torch


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(shape, seed, dout_ones=False):
    r = _rng(seed)
    q, k, v = (r.standard_normal(shape) for _ in range(3))
    dout = np.ones(shape) if dout_ones else r.standard_normal(shape)
    return q, k, v, dout


# --------------------------------------------------------------------------- windows

def check_windows(orc, max_len=18, max_d=3):
    """Brute-force window properties on every small axis."""
    for L in range(1, max_len + 1):
        for d in range(1, max_d + 1):
            n_min = min((L - r + d - 1) // d for r in range(min(d, L)))
            for k in range(1, n_min + 1):
                for x in range(L):
                    s = orc.window_start(L, k, d, x)
                    keys = [s + d * t for t in range(k)]
                    assert all(0 <= y < L for y in keys), (L, k, d, x, keys)
                    assert all(y % d == x % d for y in keys), (L, k, d, x, keys)
                    assert x in keys, (L, k, d, x, keys)
                    # all runs of k consecutive class members that contain x
                    r = x % d
                    n = (L - r + d - 1) // d
                    i = x // d
                    runs = [a for a in range(0, n - k + 1) if a <= i < a + k]
                    # nearest run center to the query; ties go to the lower start
                    best = min(runs, key=lambda a: (abs((a + (k - 1) / 2) - i), a))
                    assert s == r + d * best, (L, k, d, x, s, r + d * best)


# --------------------------------------------------------------------------- dense

def _flat(a, ndim):
    """[B, (T,) H, W, h, D] -> [B, h, N, D]."""
    B, h, D = a.shape[0], a.shape[-2], a.shape[-1]
    return a.reshape(B, -1, h, D).transpose(0, 2, 1, 3)


def check_dense(orc, grid=(4, 5), heads=2, D=3, seed=0, tol=1e-11):
    """kernel = whole grid: compare with torch's dense attention and autograd."""
    shape = (2,) + tuple(grid) + (heads, D)
    q, k, v, dout = _inputs(shape, seed)
    scale = 0.7
    out, lse = orc.na_fwd(q, k, v, grid, 1, scale)
    dq, dk, dv = orc.na_bwd(q, k, v, dout, grid, 1, scale)

    nd = len(grid)
    tq, tk, tv = (torch.tensor(_flat(a, nd), requires_grad=True) for a in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    tlse = torch.logsumexp(scale * (tq @ tk.transpose(-1, -2)), dim=-1)
    to.backward(torch.tensor(_flat(dout, nd)))

    ref = {
        "out": to.detach().numpy(), "lse": tlse.detach().numpy(),
        "dq": tq.grad.numpy(), "dk": tk.grad.numpy(), "dv": tv.grad.numpy(),
    }
    got = {"out": _flat(out, nd), "lse": lse.reshape(2, -1, heads).transpose(0, 2, 1),
           "dq": _flat(dq, nd), "dk": _flat(dk, nd), "dv": _flat(dv, nd)}
    for name in ref:
        err = np.max(np.abs(got[name] - ref[name])) / max(1.0, np.max(np.abs(ref[name])))
        assert err < tol, (name, err)


# --------------------------------------------------------------------------- weights

def check_weights(orc, seed=1):
    for shape, kernel, dil in [((1, 7, 6, 2, 4), (3, 5), 1), ((1, 9, 8, 1, 3), (3, 3), 2),
                               ((1, 4, 6, 6, 2, 3), (3, 3, 5), (1, 2, 1))]:
        q, k, v, _ = _inputs(shape, seed)
        scale = 0.9
        w, keys = orc.na_weights(q, k, kernel, dil, scale)
        assert np.max(np.abs(w.sum(1) - 1.0)) < 1e-12
        assert np.all(w >= 0)
        # every key of a window is distinct
        assert all(len(set(r)) == r.size for r in keys)
        _, lse = orc.na_fwd(q, k, v, kernel, dil, scale)
        # scores reconstructed from the weights: s = lse + log w; max s <= lse <= max s + ln K
        lse = lse.reshape(-1)
        smax = lse + np.log(w.max(1))
        K = w.shape[1]
        assert np.all(lse >= smax - 1e-12) and np.all(lse <= smax + np.log(K) + 1e-12)
        # the weights are the softmax of scale * <q, k_y> over the listed keys
        h = shape[-2]
        qf = q.reshape(-1, shape[-1])
        kf = k.reshape(shape[0], -1, h, shape[-1])
        n_tok = kf.shape[1]
        for u in range(0, qf.shape[0], max(1, qf.shape[0] // 23)):
            b, tok, hh = u // (h * n_tok), (u // h) % n_tok, u % h
            s = scale * kf[b, keys[u], hh] @ qf[u]
            e = np.exp(s - s.max())
            assert np.max(np.abs(e / e.sum() - w[u])) < 1e-12


# --------------------------------------------------------------------------- finite differences

FD_CASES = [
    ((1, 5, 6, 2, 3), (3, 3), 1),
    ((1, 7, 7, 1, 2), (3, 3), 2),
    ((1, 3, 4, 5, 1, 2), (3, 3, 3), 1),
    ((1, 6, 5, 1, 2), (4, 2), 1),
    ((2, 5, 4, 1, 2), (2, 3), (2, 1)),
]


def check_fd(orc, case, seed=2, h=1e-6, tol=2e-7):
    shape, kernel, dil = case
    q, k, v, dout = _inputs(shape, seed)
    scale = 0.8
    dq, dk, dv = orc.na_bwd(q, k, v, dout, kernel, dil, scale)

    def loss(qq, kk, vv):
        out, _ = orc.na_fwd(qq, kk, vv, kernel, dil, scale)
        return float(np.sum(out * dout))

    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        num = np.empty_like(g)
        for idx in np.ndindex(g.shape):
            args = [q.copy(), k.copy(), v.copy()]
            t = {"dq": 0, "dk": 1, "dv": 2}[name]
            args[t][idx] += h
            lp = loss(*args)
            args[t][idx] -= 2 * h
            lm = loss(*args)
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
        assert err < tol, (name, case, err)


# --------------------------------------------------------------------------- special cases

def check_k1(orc, seed=3):
    for shape, kernel in [((2, 4, 5, 3, 4), (1, 1)), ((1, 2, 3, 4, 2, 3), (1, 1, 1))]:
        q, k, v, dout = _inputs(shape, seed)
        scale = 1.3
        out, lse = orc.na_fwd(q, k, v, kernel, 1, scale)
        assert np.max(np.abs(out - v)) < 1e-13
        assert np.max(np.abs(lse - scale * np.sum(q * k, -1))) < 1e-12
        dq, dk, dv = orc.na_bwd(q, k, v, dout, kernel, 1, scale)
        assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
        assert np.max(np.abs(dv - dout)) < 1e-13


def check_kt1(orc, seed=4):
    shape = (1, 3, 6, 6, 2, 3)
    q, k, v, dout = _inputs(shape, seed)
    out3, lse3 = orc.na_fwd(q, k, v, (1, 3, 3), (1, 1, 2))
    g3 = orc.na_bwd(q, k, v, dout, (1, 3, 3), (1, 1, 2))
    for t in range(shape[1]):
        sl = (slice(None), t)
        out2, lse2 = orc.na_fwd(q[sl], k[sl], v[sl], (3, 3), (1, 2))
        g2 = orc.na_bwd(q[sl], k[sl], v[sl], dout[sl], (3, 3), (1, 2))
        assert np.max(np.abs(out3[sl] - out2)) < 1e-13
        assert np.max(np.abs(lse3[sl] - lse2)) < 1e-13
        for a, b in zip(g3, g2):
            assert np.max(np.abs(a[sl] - b)) < 1e-12


def check_dilation(orc, seed=5):
    for shape, kernel, dil in [((1, 9, 9, 2, 3), (3, 3), (2, 3)),
                               ((1, 5, 7, 6, 1, 2), (2, 3, 2), (2, 2, 3))]:
        q, k, v, dout = _inputs(shape, seed)
        out, lse = orc.na_fwd(q, k, v, kernel, dil)
        g = orc.na_bwd(q, k, v, dout, kernel, dil)
        nd = len(kernel)
        for res in itertools.product(*(range(d) for d in dil)):
            sl = (slice(None),) + tuple(slice(r, None, d) for r, d in zip(res, dil))
            o2, l2 = orc.na_fwd(q[sl], k[sl], v[sl], kernel, 1)
            g2 = orc.na_bwd(q[sl], k[sl], v[sl], dout[sl], kernel, 1)
            assert np.max(np.abs(out[sl] - o2)) < 1e-13, (res, nd)
            assert np.max(np.abs(lse[sl] - l2)) < 1e-13
            for a, b in zip(g, g2):
                assert np.max(np.abs(a[sl] - b)) < 1e-12


def check_heads(orc, seed=6):
    shape = (3, 5, 6, 4, 3)
    q, k, v, dout = _inputs(shape, seed)
    perm_h = np.array([2, 0, 3, 1])
    perm_b = np.array([1, 2, 0])
    out, lse = orc.na_fwd(q, k, v, (3, 5))
    g = orc.na_bwd(q, k, v, dout, (3, 5))
    P = lambda a: a[perm_b][..., perm_h, :]  # noqa: E731
    o2, l2 = orc.na_fwd(P(q), P(k), P(v), (3, 5))
    g2 = orc.na_bwd(P(q), P(k), P(v), P(dout), (3, 5))
    assert np.max(np.abs(P(out) - o2)) < 1e-14
    assert np.max(np.abs(lse[perm_b][..., perm_h] - l2)) < 1e-14
    for a, b in zip(g, g2):
        assert np.max(np.abs(P(a) - b)) < 1e-13


def check_sums(orc, seed=7):
    for shape, kernel, dil in [((2, 6, 7, 2, 3), (3, 5), 1), ((1, 3, 5, 6, 2, 2), (3, 3, 3), (1, 1, 2))]:
        q, k, v, dout = _inputs(shape, seed)
        dq, dk, dv = orc.na_bwd(q, k, v, dout, kernel, dil)
        axes = tuple(range(1, len(shape) - 2))  # spatial axes
        assert np.max(np.abs(dv.sum(axes) - dout.sum(axes))) < 1e-11
        assert np.max(np.abs(dk.sum(axes))) < 1e-11


def check_reflection(orc, seed=8):
    shape = (1, 4, 7, 6, 2, 3)
    kernel = (3, 5, 3)
    q, k, v, dout = _inputs(shape, seed)
    out, lse = orc.na_fwd(q, k, v, kernel)
    g = orc.na_bwd(q, k, v, dout, kernel)
    for ax in (1, 2, 3):
        F = lambda a: np.flip(a, ax)  # noqa: E731
        o2, l2 = orc.na_fwd(F(q), F(k), F(v), kernel)
        g2 = orc.na_bwd(F(q), F(k), F(v), F(dout), kernel)
        assert np.max(np.abs(F(out) - o2)) < 1e-13, ax
        assert np.max(np.abs(F(lse) - l2)) < 1e-13, ax
        for a, b in zip(g, g2):
            assert np.max(np.abs(F(a) - b)) < 1e-12, ax


def check_scale(orc, seed=9):
    shape = (1, 6, 5, 2, 3)
    q, k, v, dout = _inputs(shape, seed)
    c = 0.37
    o1, l1 = orc.na_fwd(q, k, v, (3, 3), 1, c)
    o2, l2 = orc.na_fwd(c * q, k, v, (3, 3), 1, 1.0)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13
    dq1, dk1, dv1 = orc.na_bwd(q, k, v, dout, (3, 3), 1, c)
    dq2, dk2, dv2 = orc.na_bwd(c * q, k, v, dout, (3, 3), 1, 1.0)
    assert np.max(np.abs(dq1 - c * dq2)) < 1e-12
    assert np.max(np.abs(dk1 - dk2)) < 1e-12 and np.max(np.abs(dv1 - dv2)) < 1e-12


def check_selection(orc, seed=10):
    """Sampled evaluation returns exactly the full evaluation's entries."""
    shape = (2, 5, 6, 3, 4)
    q, k, v, dout = _inputs(shape, seed)
    out, lse = orc.na_fwd(q, k, v, (3, 3), 1)
    dq, dk, dv = orc.na_bwd(q, k, v, dout, (3, 3), 1)
    sel = np.array([0, 7, 31, 59, 100, 179])
    o2, l2 = orc.na_fwd(q, k, v, (3, 3), 1, sel=sel)
    g2 = orc.na_bwd(q, k, v, dout, (3, 3), 1, sel=sel)
    D = shape[-1]
    assert np.array_equal(out.reshape(-1, D)[sel], o2)
    assert np.array_equal(lse.reshape(-1)[sel], l2)
    for a, b in zip((dq, dk, dv), g2):
        assert np.array_equal(a.reshape(-1, D)[sel], b)


# --------------------------------------------------------------------------- unfused ops
# The unfused ops (na_qk, softmax, na_av and the inverse-neighborhood sum
# behind KGRAD / VGRAD) on head-major tensors [B, heads, (T,) H, W, C].

def _hm(shape_tm_grid, heads, C, seed, B=1):
    r = _rng(seed)
    return r.standard_normal((B, heads) + tuple(shape_tm_grid) + (C,))


def check_unfused_dense(orc, seed=11):
    """kernel = whole grid: every window is the whole grid in row-major order,
    so na_qk is alpha * a b^T, na_av is alpha * attn b and the inverse sum is
    alpha * attn^T a (numpy matmul per (batch, head))."""
    for grid in [(4, 5), (2, 3, 4)]:
        B, heads, D = 2, 2, 3
        a = _hm(grid, heads, D, seed, B)
        b = _hm(grid, heads, D, seed + 1, B)
        N = int(np.prod(grid))
        G = _hm(grid, heads, N, seed + 2, B)
        alpha = 0.8
        af, bf, Gf = (x.reshape(B, heads, N, -1) for x in (a, b, G))
        attn = orc.na_qk(a, b, grid, 1, alpha).reshape(B, heads, N, N)
        assert np.max(np.abs(attn - alpha * af @ bf.transpose(0, 1, 3, 2))) < 1e-12
        out = orc.na_av(G, b, grid, 1, alpha).reshape(B, heads, N, D)
        assert np.max(np.abs(out - alpha * Gf @ bf)) < 1e-12
        inv = orc.na_av_inverse(G, a, grid, 1, alpha).reshape(B, heads, N, D)
        assert np.max(np.abs(inv - alpha * Gf.transpose(0, 1, 3, 2) @ af)) < 1e-12


UNFUSED_CASES = [((7, 6), (3, 5), (1, 1)), ((9, 8), (3, 3), (2, 2)), ((5, 10), (4, 3), (1, 3)),
                 ((4, 6, 6), (3, 3, 5), (1, 2, 1)), ((5, 4, 7), (2, 3, 3), (2, 1, 2))]


def check_unfused_adjoint(orc, seed=12):
    """na_av and the inverse sum are the two adjoints of na_qk:
    <na_qk(a, b), G> = <a, na_av(G, b)> = <b, na_av_inverse(G, a)> for every G.
    A wrong window position, a transposed index or a wrong membership in any of
    the three breaks one of the equalities."""
    for i, (grid, kernel, dil) in enumerate(UNFUSED_CASES):
        heads, D = 2, 3
        K = int(np.prod(kernel))
        a = _hm(grid, heads, D, seed + 3 * i)
        b = _hm(grid, heads, D, seed + 3 * i + 1)
        G = _hm(grid, heads, K, seed + 3 * i + 2)
        lhs = np.sum(orc.na_qk(a, b, kernel, dil, 1.3) * G)
        mid = np.sum(a * orc.na_av(G, b, kernel, dil, 1.3))
        rhs = np.sum(b * orc.na_av_inverse(G, a, kernel, dil, 1.3))
        assert abs(lhs - mid) < 1e-10 * max(1.0, abs(lhs)), (grid, kernel, dil, lhs, mid)
        assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(lhs)), (grid, kernel, dil, lhs, rhs)


def check_unfused_matches_fused(orc, seed=13):
    """softmax(scale * na_qk) is the fused path's window weights, na_av of
    them its output, and the five backward ops compose to its gradients (the
    fused functions are pinned on their own by the dense, finite-difference
    and identity checks above)."""
    for i, (grid, kernel, dil) in enumerate(UNFUSED_CASES):
        heads, D = 2, 3
        q, k, v, dout = (_hm(grid, heads, D, seed + 4 * i + j) for j in range(4))
        scale = 0.6
        P, out = orc.unfused_fwd(q, k, v, kernel, dil, scale)
        dq, dk, dv = orc.unfused_bwd(q, k, v, P, dout, kernel, dil, scale)
        tm = lambda x: np.moveaxis(x, 1, -2)
        o_ref, _ = orc.na_fwd(tm(q), tm(k), tm(v), kernel, dil, scale)
        w_ref, _ = orc.na_weights(tm(q), tm(k), kernel, dil, scale)
        g_ref = orc.na_bwd(tm(q), tm(k), tm(v), tm(dout), kernel, dil, scale)
        assert np.max(np.abs(tm(out) - o_ref)) < 1e-12
        assert np.max(np.abs(tm(P).reshape(w_ref.shape) - w_ref)) < 1e-12
        for got, ref in zip((dq, dk, dv), g_ref):
            assert np.max(np.abs(tm(got) - ref)) < 1e-12


def check_softmax(orc, seed=14):
    """The window softmax and its backward against torch (float64, CPU) and its autograd."""
    import oracle as _o   # the numpy softmax is module-level, not per build
    r = _rng(seed)
    x = 4.0 * r.standard_normal((3, 5, 25))
    g = r.standard_normal(x.shape)
    tx = torch.tensor(x, requires_grad=True)
    tp = torch.softmax(tx, dim=-1)
    tp.backward(torch.tensor(g))
    p = _o.softmax(x)
    assert np.max(np.abs(p - tp.detach().numpy())) < 1e-14
    assert np.max(np.abs(_o.softmax_bwd(p, g) - tx.grad.numpy())) < 1e-14
    # large scores: no overflow, rows still sum to one
    big = _o.softmax(x * 300.0)
    assert np.all(np.isfinite(big)) and np.max(np.abs(big.sum(-1) - 1.0)) < 1e-12


def check_unfused_selection(orc, seed=15):
    """Sampled evaluation (head-major unit ids) returns the full evaluation's rows."""
    grid, kernel, dil = (5, 6), (3, 3), (1, 2)
    heads, D, K = 3, 4, 9
    a = _hm(grid, heads, D, seed, B=2)
    b = _hm(grid, heads, D, seed + 1, B=2)
    G = _hm(grid, heads, K, seed + 2, B=2)
    sel = np.array([0, 7, 31, 59, 100, 179])
    full = [orc.na_qk(a, b, kernel, dil, 0.5), orc.na_av(G, b, kernel, dil, 0.5),
            orc.na_av_inverse(G, a, kernel, dil, 0.5)]
    part = [orc.na_qk(a, b, kernel, dil, 0.5, sel=sel), orc.na_av(G, b, kernel, dil, 0.5, sel=sel),
            orc.na_av_inverse(G, a, kernel, dil, 0.5, sel=sel)]
    for f, p in zip(full, part):
        assert np.array_equal(f.reshape(-1, f.shape[-1])[sel], p)


# --------------------------------------------------------------------------- relative positional bias

def check_rpb_worked_examples(orc):
    """q = k = 0 so the scores are the bias alone, bias values 10 + index:
    worked out by hand from the reading (offset key - query in class units,
    stored at offset + k - 1) for a 1 x 5 row with k = 3 (windows shifted at
    both ends) and a 1 x 6 row at dilation 2 (two classes of three)."""
    rpb = np.array([10., 11, 12, 13, 14]).reshape(1, 1, 5)
    z = np.zeros((1, 1, 1, 5, 1))
    got = orc.na_qk(z, z, (1, 3), 1, 1.0, rpb=rpb)[0, 0, 0]
    want = [[12, 13, 14], [11, 12, 13], [11, 12, 13], [11, 12, 13], [10, 11, 12]]
    assert np.array_equal(got, np.array(want, float)), got
    z = np.zeros((1, 1, 1, 6, 1))
    got = orc.na_qk(z, z, (1, 3), (1, 2), 1.0, rpb=rpb)[0, 0, 0]
    want = [[12, 13, 14], [12, 13, 14], [11, 12, 13], [11, 12, 13], [10, 11, 12], [10, 11, 12]]
    assert np.array_equal(got, np.array(want, float)), got


def check_rpb_adjoint(orc, seed=16):
    """Adding the bias and its gradient are adjoint maps:
    <qk(a, b, rpb) - qk(a, b), G> = <rpb, rpb_grad(G)> for every rpb and G, and
    a zero table adds nothing."""
    import oracle as _o
    for i, (grid, kernel, dil) in enumerate(UNFUSED_CASES):
        heads, D = 2, 3
        K = int(np.prod(kernel))
        a = _hm(grid, heads, D, seed + 3 * i)
        b = _hm(grid, heads, D, seed + 3 * i + 1)
        G = _hm(grid, heads, K, seed + 3 * i + 2)
        rpb = _rng(seed + i).standard_normal(_o.rpb_shape(kernel, heads))
        base = orc.na_qk(a, b, kernel, dil, 0.9)
        assert np.array_equal(orc.na_qk(a, b, kernel, dil, 0.9, rpb=np.zeros_like(rpb)), base)
        lhs = np.sum((orc.na_qk(a, b, kernel, dil, 0.9, rpb=rpb) - base) * G)
        rhs = np.sum(rpb * orc.rpb_grad(G, kernel, dil))
        assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(lhs)), (grid, kernel, dil, lhs, rhs)


def check_rpb_fd(orc, seed=17, h=1e-6, tol=2e-7):
    """Central finite differences of sum(out * dout) through the unfused forward
    with a bias fix the bias gradient of the unfused backward."""
    import oracle as _o
    for grid, kernel, dil in [((5, 6), (3, 3), (1, 2)), ((3, 4, 5), (3, 3, 3), 1)]:
        heads, D = 2, 3
        q, k, v, dout = (_hm(grid, heads, D, seed + j) for j in range(4))
        rpb = 0.5 * _rng(seed).standard_normal(_o.rpb_shape(kernel, heads))
        P, _ = orc.unfused_fwd(q, k, v, kernel, dil, 0.7, rpb=rpb)
        g = orc.unfused_bwd(q, k, v, P, dout, kernel, dil, 0.7, want_rpb=True)[3]
        flat = rpb.reshape(-1)
        for idx in _rng(seed + 1).choice(flat.size, 6, replace=False):
            vals = []
            for sgn in (1, -1):
                r2 = flat.copy()
                r2[idx] += sgn * h
                _, o2 = orc.unfused_fwd(q, k, v, kernel, dil, 0.7, rpb=r2.reshape(rpb.shape))
                vals.append(np.sum(o2 * dout))
            fd = (vals[0] - vals[1]) / (2 * h)
            assert abs(fd - g.reshape(-1)[idx]) < tol * max(1.0, abs(fd)), (grid, idx, fd)


# --------------------------------------------------------------------------- masked windows

def check_masked_windows(orc, seed=18):
    """Masking the scores of a larger window down to a smaller one gives
    neighborhood attention with the smaller window (windows of the same
    centered-and-shifted rule are nested): the masked unfused forward with a
    constant per-frame time kernel equals the fused oracle at that kernel,
    and the backward through it (masked weights are zero) equals its
    gradients. A mask of ones changes nothing; a fully masked query gets a
    zero output."""
    import oracle as _o
    grid, kernel, heads, D = (6, 5, 4), (5, 3, 3), 2, 3
    q, k, v, dout = (_hm(grid, heads, D, seed + j) for j in range(4))
    for kt in (1, 3):
        mask = _o.frame_window_mask(grid, kernel, [kt] * grid[0])
        P, out = orc.unfused_fwd(q, k, v, kernel, 1, 0.8, mask=mask)
        dq, dk, dv = orc.unfused_bwd(q, k, v, P, dout, kernel, 1, 0.8)
        small = (kt,) + kernel[1:]
        tm = lambda x: np.moveaxis(x, 1, -2)  # noqa: E731
        o_ref, _ = orc.na_fwd(tm(q), tm(k), tm(v), small, 1, 0.8)
        g_ref = orc.na_bwd(tm(q), tm(k), tm(v), tm(dout), small, 1, 0.8)
        assert np.max(np.abs(tm(out) - o_ref)) < 1e-12, kt
        for got, ref in zip((dq, dk, dv), g_ref):
            assert np.max(np.abs(tm(got) - ref)) < 1e-12, kt
    ones = np.ones(grid + (int(np.prod(kernel)),), np.uint8)
    P1, o1 = orc.unfused_fwd(q, k, v, kernel, 1, 0.8, mask=ones)
    P0, o0 = orc.unfused_fwd(q, k, v, kernel, 1, 0.8)
    assert np.array_equal(P1, P0) and np.array_equal(o1, o0)
    dead = ones.copy()
    dead[2, 1, 3, :] = 0
    Pd, od = orc.unfused_fwd(q, k, v, kernel, 1, 0.8, mask=dead)
    assert np.all(Pd[:, :, 2, 1, 3] == 0) and np.all(od[:, :, 2, 1, 3] == 0)


def check_outer_window_mask(orc, seed=19):
    """Windows restricted along the outermost axis: a table worked out by hand
    from the definition (2D, five rows, kernel 3 x 1, per-row sizes 3, 1, 2, 0,
    3); and a constant restricted size k' gives neighborhood attention with
    kernel k' along that axis (2D and 3D, with dilation along it), forward and
    backward through the masked unfused ops."""
    import oracle as _o
    m = _o.outer_window_mask((5, 2), (3, 1), [3, 1, 2, 0, 3])
    # row 0: window rows 0..2, own window of 3 -> 0..2;  row 1: own window {1};
    # row 2: window rows 1..3, own 2 -> rows 1, 2;  row 3: nothing;  row 4: rows 2..4
    want = [[1, 1, 1], [0, 1, 0], [1, 1, 0], [0, 0, 0], [1, 1, 1]]
    for x0 in range(5):
        for x1 in range(2):
            assert list(m[x0, x1]) == want[x0], (x0, list(m[x0, x1]))
    cases = [((7, 6), (5, 3), 1, (3, 1)), ((9, 5), (3, 3), (2, 1), (1, 2)),
             ((5, 4, 3), (3, 3, 3), 1, (1, 2))]
    for grid, kernel, dil, ks in cases:
        heads, D = 2, 3
        q, k, v, dout = (_hm(grid, heads, D, seed + j) for j in range(4))
        tm = lambda x: np.moveaxis(x, 1, -2)  # noqa: E731
        for kk in ks:
            mask = _o.outer_window_mask(grid, kernel, [kk] * grid[0], dil)
            P, out = orc.unfused_fwd(q, k, v, kernel, dil, 0.8, mask=mask)
            dq, dk, dv = orc.unfused_bwd(q, k, v, P, dout, kernel, dil, 0.8)
            small = (kk,) + tuple(kernel[1:])
            o_ref, _ = orc.na_fwd(tm(q), tm(k), tm(v), small, dil, 0.8)
            g_ref = orc.na_bwd(tm(q), tm(k), tm(v), tm(dout), small, dil, 0.8)
            assert np.max(np.abs(tm(out) - o_ref)) < 1e-12, (grid, kk)
            for got, ref in zip((dq, dk, dv), g_ref):
                assert np.max(np.abs(tm(got) - ref)) < 1e-12, (grid, kk)


def window_tokens(grid, kernel, dil, x, window_start):
    """Flat indices of the tokens of query x's window, from the per-axis
    window starts (start + dilation * j, j < kernel)."""
    axes = [[window_start(grid[a], kernel[a], dil[a], x[a]) + dil[a] * j for j in range(kernel[a])]
            for a in range(len(grid))]
    return [int(np.ravel_multi_index(c, grid)) for c in itertools.product(*axes)]


def check_index_mask(orc, seed=20):
    """Index tensors of attended tokens turned into window masks. Entries
    worked out by hand from the definition (2D 5 x 4 grid, 3 x 3 window; a
    dilated 6 x 7 grid); and, on 2D and 3D grids with dilation, a random
    subset of every query's window listed as indices (shuffled, with -1 slots
    and a repeated token) gives, through the masked unfused forward, exactly
    softmax attention over the listed tokens, computed densely over the whole
    grid without any window arithmetic."""
    import oracle as _o
    # query (0, 0): rows 0..2, cols 0..2; query (4, 3): rows 2..4, cols 1..3
    idx = np.full((5, 4, 6), -1, np.int64)
    idx[0, 0] = [0, 10, 7, -1, 20, 10]      # (0,0) -> 0, (2,2) -> 8, (1,3) outside, 20 off-grid
    idx[4, 3] = [19, 9, 12, -1, -1, -3]     # (4,3) -> 8, (2,1) -> 0, (3,0) outside, -3 invalid
    m, bad = _o.window_mask_from_indices((5, 4), (3, 3), idx)
    assert list(np.nonzero(m[0, 0])[0]) == [0, 8] and bad[0, 0] == 2
    assert list(np.nonzero(m[4, 3])[0]) == [0, 8] and bad[4, 3] == 2
    assert not m[1:4].any() and not bad[1:4].any()
    # dilation 2 along H on 6 rows: query (1, 3) sees rows 1, 3, 5 and columns 2..4
    idx = np.full((6, 7, 3), -1, np.int64)
    idx[1, 3] = [3 * 7 + 4, 2 * 7 + 3, 5 * 7 + 2]   # (3,4) -> 1*3+2, (2,3) other class, (5,2) -> 6
    m, bad = _o.window_mask_from_indices((6, 7), (3, 3), idx, (2, 1))
    assert list(np.nonzero(m[1, 3])[0]) == [5, 6] and bad[1, 3] == 1
    r = _rng(seed)
    for grid, kernel, dil in (((7, 6), (3, 5), (2, 1)), ((4, 5, 6), (3, 3, 3), (1, 1, 2))):
        nd, heads, D = len(grid), 2, 3
        toks, m_slots = int(np.prod(grid)), int(np.prod(kernel)) + 3
        idx = np.full(grid + (m_slots,), -1, np.int64)
        listed = {}
        for x in np.ndindex(*grid):
            win = window_tokens(grid, kernel, dil, x, orc.window_start)
            keep = [t for t in win if r.random() < 0.6] or [win[0]]
            slots = keep + [keep[0]]
            r.shuffle(slots)
            idx[x][:len(slots)] = slots
            listed[x] = set(keep)
        mask, bad = _o.window_mask_from_indices(grid, kernel, idx, dil)
        assert not bad.any()
        q, k, v = (_hm(grid, heads, D, seed + j) for j in range(3))
        _, out = orc.unfused_fwd(q, k, v, kernel, dil, 0.8, mask=mask)
        qf, kf, vf = (a.reshape(1, heads, toks, D) for a in (q, k, v))
        allowed = np.zeros((toks, toks), bool)
        for x, ys in listed.items():
            allowed[np.ravel_multi_index(x, grid), sorted(ys)] = True
        s = np.where(allowed, 0.8 * np.einsum("bhxc,bhyc->bhxy", qf, kf), -np.inf)
        p = np.exp(s - s.max(-1, keepdims=True))
        ref = (p / p.sum(-1, keepdims=True)) @ vf
        assert np.max(np.abs(out.reshape(ref.shape) - ref)) < 1e-12, grid


ALL_CHECKS = [
    ("windows", lambda o: check_windows(o)),
    ("dense2d", lambda o: check_dense(o, grid=(4, 5))),
    ("dense3d", lambda o: check_dense(o, grid=(2, 3, 4))),
    ("weights", check_weights),
    ("k1", check_k1),
    ("kt1", check_kt1),
    ("dilation", check_dilation),
    ("heads", check_heads),
    ("sums", check_sums),
    ("reflection", check_reflection),
    ("scale", check_scale),
    ("selection", check_selection),
    ("unfused_dense", check_unfused_dense),
    ("unfused_adjoint", check_unfused_adjoint),
    ("unfused_matches_fused", check_unfused_matches_fused),
    ("softmax", check_softmax),
    ("unfused_selection", check_unfused_selection),
    ("rpb_worked_examples", check_rpb_worked_examples),
    ("rpb_adjoint", check_rpb_adjoint),
    ("rpb_fd", check_rpb_fd),
    ("masked_windows", check_masked_windows),
    ("outer_window_mask", check_outer_window_mask),
    ("index_mask", check_index_mask),
] + [(f"fd{i}", (lambda c: (lambda o: check_fd(o, c)))(c)) for i, c in enumerate(FD_CASES)]


def failing_checks(orc, first_only=False):
    """Names of the checks the given oracle build fails (cheapest checks first;
    with first_only, stop at the first failure)."""
    bad = []
    for name, fn in ALL_CHECKS:
        try:
            fn(orc)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            bad.append(name)
            if first_only:
                break
    return bad
