#!/usr/bin/env python3
"""Benchmark of fused neighborhood attention forward + backward on one MI355X.

One step is the whole hot path on one batch of synthetic input: na_fwd, then
the gather backward (na_bwd_dq, na_bwd_dkdv -- together exactly na_bwd with
NA_BWD_GATHER), inputs resident in HBM. W untimed warm-up steps, then K timed
steps between two device synchronizations; per-kernel durations come from HIP
events recorded on the stream the kernels are launched on.

Workloads (from NATTEN issue #161's benchmark script: 8 heads of dimension 32,
fp32, q/k/v standard normal, loss = out.sum() so dout = ones): the headline is
the 2D 1024x1024 grid with a 9x9 window; the 3D 16x256x256 grid with a 3x5x5
window is measured in the same run and reported beside it.

Effective FLOPs (the metric's convention): forward 4*N*heads*K*D, backward
2.5x that, with N tokens and K = prod(kernel). Prints one JSON line on stdout;
progress goes to stderr.

Timing protocol: before each pass (forward; backward) a 1 GiB buffer is
overwritten, which evicts the inputs from the L2 caches and the 256 MB
Infinity Cache, so every pass starts cold as it would inside a model; the
flush itself is outside the timed events. Per pass the median, minimum and
mean over the timed steps are reported; the headline value uses the medians.
The same steps without the flush are reported beside it ("warm").

The 3D workload is also timed with every window restricted along T to a
constant 1 and 2 of its 3 planes (na_fwd_framed / na_bwd_framed, "framed"):
the kernels skip key planes outside a query's frame window, so the time
should follow the kept fraction of the window. It is also timed with an
arbitrary window mask that keeps 2/3 of every window at random
(na_fwd_masked / na_bwd_masked, "masked"), whose time follows the full
window.

Beside the headline step the same run times the KV-parallel backward variant
on the same inputs ("kvparallel", per kv_splits: 0 = float atomics, 1 and 4 =
bounded accumulator copies, bitwise reproducible), the headline shape with
fp16 tensors ("fp16") and the two bf16 workloads ("bf16"; the head_dim-32 one
also with the random 2/3 window mask, "masked").

The same function is also timed through the unfused ops (the script's method
= 'unfused': window scores, softmax, weighted sum, and their backward AGRAD,
VGRAD, softmax backward, QGRAD, KGRAD, on head-major copies of the same
inputs) and reported under "unfused", with each op's share of the HBM
roofline: the fused-versus-unfused comparison the issue is about.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from fwd_bwd_amd import na  # noqa: E402
from fwd_bwd_amd.inputs import HEADLINE, HEADLINE_3D, WORKLOADS, make_inputs  # noqa: E402

METRIC = "NA fwd+bwd ms & TFLOP/s (% roofline): 2D 1024² k9×9, 3D 16×256² k3×5×5"
PEAK_TFLOPS = {"fp32_mfma": 157.3, "bf16_mfma": 2516.6}
PEAK_HBM_GBS = 8000.0
DTYPE_LABEL = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}
# parity bar of the sampled check beside the CPU baseline (max abs error over
# max abs reference value, per tensor), as in the GPU parity tests
TOLERANCE = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 2e-3}
FLUSH_BYTES = 1 << 30


def mfma_peak(dtype):
    """Dense MFMA peak (TFLOP/s) of the workload's arithmetic type: fp32 for
    fp32 tensors; the 16-bit MFMA rate (bf16 and fp16 alike) for 16-bit ones."""
    return PEAK_TFLOPS["fp32_mfma"] if dtype == torch.float32 else PEAK_TFLOPS["bf16_mfma"]


def stats(xs):
    xs = [float(x) for x in xs]
    return {"median": round(float(np.median(xs)), 4), "min": round(min(xs), 4),
            "mean": round(float(np.mean(xs)), 4)}

# contraction FLOPs each kernel performs per (query or key) x window entry x channel,
# without tile waste: fwd = QK^T + PV; dq = QK^T + dO V^T + dS K;
# dk/dv = QK^T + dO V^T + P^T dO + dS^T Q
KERNEL_FLOP_UNITS = {"fwd": 4, "bwd_dq": 6, "bwd_dkdv": 8, "bwd_kvparallel": 10}

# the bf16 workloads (3D 2x8x128x128 with a 5x7x7 window; 2D 4x512x512, 13x13, dilation 2,
# head_dim 64), timed beside the headline for their roofline fractions
BF16_WORKLOADS = ("3d_b2_8x128x128_k5x7x7_h8_d32_bf16", "2d_b4_512x512_k13_d2_h4_d64_bf16")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "fwd_bwd_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# the sources the fused kernels (the bench phases) are built from
FUSED_SOURCES = ("na_api.hip", "na_common.hpp", "na_fast.hpp", "na_host.hpp", "na_index.hpp",
                 "na_kernels.hpp", "na_m16.hip", "na_mfma16.hpp")


def kernel_source_hash():
    """sha256 over the fused kernels' sources; a recorded traffic figure is
    only reported while the kernels it was measured on are unchanged."""
    h = hashlib.sha256()
    for name in sorted(FUSED_SOURCES):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary profiles/traffic_<kernel>_<workload>.md, or None
    when there is none or it was taken on other kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def flops(w):
    base = w.tokens * w.heads * w.window * w.head_dim
    return 4.0 * base, 10.0 * base


def algorithmic_bytes(w):
    e = torch.tensor([], dtype=w.dtype).element_size()
    t = w.tokens * w.heads * w.head_dim * e
    rows = w.tokens * w.heads * 4
    fwd = 4 * t + rows                  # q, k, v read; out written; lse written
    bwd = 8 * t + rows + 2 * rows       # q, k, v, out, dout read; dq, dk, dv written; lse; delta w+r
    return fwd, bwd, {"fwd": 4 * t + rows, "bwd_dq": 5 * t + 2 * rows,
                      "bwd_dkdv": 6 * t + 2 * rows, "bwd_kvparallel": bwd}


class Runner:
    def __init__(self, w, variant, seed=0, kv_splits=0, host=None):
        self.w = w
        self.variant = variant
        self.kv_splits = kv_splits
        dev = torch.device("cuda:0")
        if host is None:
            log(f"[bench] generating inputs for {w.name}")
            host = make_inputs(w, seed)
        q, k, v, dout = host
        self.host = (q, k, v, dout)
        self.q, self.k, self.v, self.dout = (t.to(dev) for t in (q, k, v, dout))
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:-1], dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
        self.delta = torch.empty_like(self.lse)
        p = na.make_problem(w.shape, w.dtype, w.kernel, w.dilation, w.the_scale)
        ws = na.bwd_workspace_bytes(p, na.VARIANTS[variant], kv_splits)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.args = (w.kernel, w.dilation, w.the_scale)

    def fwd(self):
        na.na_fwd(self.q, self.k, self.v, *self.args, out=self.out, lse=self.lse)

    def bwd_dq(self):
        na.na_bwd_dq(self.q, self.k, self.v, self.out, self.dout, self.lse, *self.args,
                     dq=self.dq, delta=self.delta)

    def bwd_dkdv(self):
        na.na_bwd_dkdv(self.q, self.k, self.v, self.dout, self.lse, self.delta, *self.args,
                       dk=self.dk, dv=self.dv)

    def bwd_kvpar(self):
        na.na_bwd(self.q, self.k, self.v, self.out, self.dout, self.lse, *self.args,
                  variant="kvparallel", workspace=self.ws, grads=(self.dq, self.dk, self.dv),
                  kv_splits=self.kv_splits)

    def outputs_host(self):
        """The last pass's results on the host (for the parity check of the
        CPU-baseline sample)."""
        torch.cuda.synchronize()
        return {"out": self.out.cpu(), "lse": self.lse.cpu(), "dq": self.dq.cpu(),
                "dk": self.dk.cpu(), "dv": self.dv.cpu()}

    def phases(self):
        if self.variant == "gather":
            return [("fwd", self.fwd), ("bwd_dq", self.bwd_dq), ("bwd_dkdv", self.bwd_dkdv)]
        return [("fwd", self.fwd), ("bwd_kvparallel", self.bwd_kvpar)]

    def time(self, steps, warmup, flush=None):
        """Per-phase kernel durations (ms lists over `steps`) and the wall time
        per step. With a flush buffer, it is overwritten before the forward
        and before the backward pass (outside the timed events)."""
        ph = self.phases()
        for _ in range(warmup):
            for _, f in ph:
                f()
        torch.cuda.synchronize()
        n = len(ph)
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            for i, (name, f) in enumerate(ph):
                if flush is not None and (name == "fwd" or i == 1):
                    flush.fill_((s + i) & 0xff)
                ev[s][i][0].record()
                f()
                ev[s][i][1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        per = {name: [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)]
               for i, (name, _) in enumerate(ph)}
        return per, wall


class FramedRunner(Runner):
    """The same step through na_fwd_framed / na_bwd_framed (gather): every
    query's window restricted along the outermost axis to frame[x0] positions
    (the requester's per-frame time kernel on 3D grids)."""

    def __init__(self, w, frame, host=None, seed=0):
        super().__init__(w, "gather", seed, host=host)
        self.frame = list(frame)
        self.fk = torch.tensor(self.frame, dtype=torch.int32, device="cuda:0")

    def fwd(self):
        na.na_fwd_framed(self.q, self.k, self.v, self.fk, *self.args, out=self.out, lse=self.lse)

    def bwd(self):
        na.na_bwd_framed(self.q, self.k, self.v, self.out, self.dout, self.lse, self.fk,
                         *self.args, workspace=self.ws, grads=(self.dq, self.dk, self.dv))

    def phases(self):
        return [("fwd", self.fwd), ("bwd_framed", self.bwd)]


class MaskedRunner(Runner):
    """The same step through na_fwd_masked / na_bwd_masked (gather): an
    arbitrary byte mask over every query's window (1 keeps the key), shared by
    batch elements and heads."""

    def __init__(self, w, mask, host=None, seed=0):
        super().__init__(w, "gather", seed, host=host)
        self.mask = mask.to("cuda:0")

    def fwd(self):
        na.na_fwd_masked(self.q, self.k, self.v, self.mask, *self.args, out=self.out, lse=self.lse)

    def bwd(self):
        na.na_bwd_masked(self.q, self.k, self.v, self.out, self.dout, self.lse, self.mask,
                         *self.args, workspace=self.ws, grads=(self.dq, self.dk, self.dv))

    def phases(self):
        return [("fwd", self.fwd), ("bwd_masked", self.bwd)]


def random_window_mask(w, keep, seed=0):
    """A seeded byte mask [(T,) H, W, K] keeping each window entry with
    probability keep."""
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(tuple(w.grid) + (w.window,), generator=g) < keep).to(torch.uint8)


def kept_fraction(w, frame):
    """Mean share of a query's full window that a restricted window keeps:
    along the outermost axis a query at x0 keeps min(frame[x0], k0) of the k0
    window positions."""
    k0 = w.kernel[0]
    return float(np.mean([min(max(f, 0), k0) for f in frame])) / k0


def framed_leg(w, per, full):
    """Times of a restricted-window step beside the unrestricted step (full)."""
    s = summarize(w, per)
    return {"fwd_ms": s["fwd_ms"], "bwd_ms": s["bwd_ms"], "ms_per_step": s["ms_per_step"],
            "step_ms_stats": s["step_ms_stats"], "kernel_ms": s["kernel_ms"],
            "time_vs_full": {"fwd": round(s["fwd_ms"] / full["fwd_ms"], 4),
                             "bwd": round(s["bwd_ms"] / full["bwd_ms"], 4),
                             "step": round(s["ms_per_step"] / full["ms_per_step"], 4)}}


# ----------------------------------------------------------------------------- unfused leg
# The same function through the unfused ops on head-major tensors (the issue's
# method = 'unfused': na_qk, softmax, na_av and, in the backward, AGRAD, VGRAD,
# the softmax backward, QGRAD and KGRAD), one kernel launch per op.

def unfused_bytes(w):
    """Algorithmic HBM bytes of each unfused op (every operand read once, every
    result written once): vectors N*heads*D*4, attention arrays N*heads*K*4."""
    t = w.tokens * w.heads * w.head_dim * 4
    a = w.tokens * w.heads * w.window * 4
    return {"qk": 2 * t + a, "softmax": 2 * a, "av": a + 2 * t, "agrad": 2 * t + a,
            "vgrad": a + 2 * t, "softmax_bwd": 3 * a, "qgrad": a + 2 * t, "kgrad": a + 2 * t}


class UnfusedRunner:
    def __init__(self, w, host):
        self.w = w
        dev = torch.device("cuda:0")
        hm = lambda t: t.movedim(-2, 1).contiguous().to(dev)  # noqa: E731
        self.q, self.k, self.v, self.dout = (hm(t) for t in host)
        self.probs = torch.empty(self.q.shape[:-1] + (w.window,), dtype=torch.float32, device=dev)
        self.ds = torch.empty_like(self.probs)
        self.out, self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(4))
        kk, dd, sc = w.kernel, w.dilation, w.the_scale
        self.ops = [
            ("qk", lambda: na.na_qk(self.q, self.k, kk, dd, sc, attn=self.probs)),
            ("softmax", lambda: na.na_softmax(self.probs, kk, dd, out=self.probs)),
            ("av", lambda: na.na_av(self.probs, self.v, kk, dd, 1.0, out=self.out)),
            ("agrad", lambda: na.na_qk(self.dout, self.v, kk, dd, 1.0, attn=self.ds)),
            ("vgrad", lambda: na.na_av_inverse(self.probs, self.dout, kk, dd, 1.0, out=self.dv)),
            ("softmax_bwd", lambda: na.na_softmax_bwd(self.probs, self.ds, kk, dd, out=self.ds)),
            ("qgrad", lambda: na.na_av(self.ds, self.k, kk, dd, sc, out=self.dq)),
            ("kgrad", lambda: na.na_av_inverse(self.ds, self.q, kk, dd, sc, out=self.dk)),
        ]

    def time(self, steps, warmup):
        for _ in range(warmup):
            for _, f in self.ops:
                f()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.ops) + 1)]
              for _ in range(steps)]
        for s in range(steps):
            ev[s][0].record()
            for i, (_, f) in enumerate(self.ops):
                f()
                ev[s][i + 1].record()
        torch.cuda.synchronize()
        # medians over the steps, as for the fused legs (one slow step must not
        # move an op's figure)
        per = {name: float(np.median([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]))
               for i, (name, _) in enumerate(self.ops)}
        step = float(np.median([ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)]))
        return step, per

    def time_chain(self, steps, warmup):
        """na_unfused_fwd + na_unfused_bwd: the same ops, with the window softmax and
        its backward taken inside the score kernels where a query's window fits."""
        w = self.w
        kk, dd, sc = w.kernel, w.dilation, w.the_scale

        def step():
            na.na_unfused_fwd(self.q, self.k, self.v, kk, dd, sc, probs=self.probs, out=self.out)
            na.na_unfused_bwd(self.q, self.k, self.v, self.probs, self.dout, kk, dd, sc,
                              dscores=self.ds, grads=(self.dq, self.dk, self.dv))
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for s in range(steps):
            step()
            ev[s + 1].record()
        torch.cuda.synchronize()
        return float(np.median([ev[s].elapsed_time(ev[s + 1]) for s in range(steps)]))


def unfused_summary(w, step, per):
    f_fwd, f_bwd = flops(w)
    by = unfused_bytes(w)
    name = max(per, key=per.get)
    gbs = by[name] / (per[name] * 1e-3) / 1e9
    return {"ms_per_step": round(step, 4),
            "fwd_ms": round(sum(per[k] for k in ("qk", "softmax", "av")), 4),
            "bwd_ms": round(sum(v for k, v in per.items() if k not in ("qk", "softmax", "av")), 4),
            "tflops_total": round((f_fwd + f_bwd) / step / 1e9, 3),
            "kernel_ms": {k: round(v, 4) for k, v in per.items()},
            "hbm_frac": {k: round(by[k] / (per[k] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) for k in per},
            "roofline": {"bound": "hbm", "kernel": name, "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": None, "bytes_per_launch": by[name],
                         "avg_launch_ms": round(per[name], 4)}}


def summarize(w, per):
    """Times, effective TFLOP/s and roofline fractions of one workload from
    per-phase duration lists; fractions against the MFMA peak of the
    workload's arithmetic type and against HBM."""
    f_fwd, f_bwd = flops(w)
    b_fwd, b_bwd, _ = algorithmic_bytes(w)
    steps = len(per["fwd"])
    bwd = [sum(per[k][s] for k in per if k != "fwd") for s in range(steps)]
    step = [per["fwd"][s] + bwd[s] for s in range(steps)]
    fwd_ms = float(np.median(per["fwd"]))
    bwd_ms = float(np.median(bwd))
    ms_step = float(np.median(step))
    peak = mfma_peak(w.dtype)
    return {
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4), "ms_per_step": round(ms_step, 4),
        "fwd_ms_stats": stats(per["fwd"]), "bwd_ms_stats": stats(bwd), "step_ms_stats": stats(step),
        "tflops_fwd": round(f_fwd / fwd_ms / 1e9, 3), "tflops_bwd": round(f_bwd / bwd_ms / 1e9, 3),
        "tflops_total": round((f_fwd + f_bwd) / ms_step / 1e9, 3),
        "mfma_peak_tflops": peak,
        "mfma_frac_fwd": round(f_fwd / fwd_ms / 1e9 / peak, 5),
        "mfma_frac_bwd": round(f_bwd / bwd_ms / 1e9 / peak, 5),
        "mfma_frac_total": round((f_fwd + f_bwd) / ms_step / 1e9 / peak, 5),
        "hbm_frac_fwd": round(b_fwd / fwd_ms / 1e6 / PEAK_HBM_GBS, 4),
        "hbm_frac_bwd": round(b_bwd / bwd_ms / 1e6 / PEAK_HBM_GBS, 4),
        "hbm_frac_total": round((b_fwd + b_bwd) / ms_step / 1e6 / PEAK_HBM_GBS, 4),
        "roofline_ms": round(max((f_fwd + f_bwd) / peak / 1e9,
                                 (b_fwd + b_bwd) / PEAK_HBM_GBS / 1e6), 4),
        "kernel_ms": {k: stats(v) for k, v in per.items()},
    }


def roofline(w, per, tag=None):
    """Roofline entry of the longest kernel (by median duration): its
    contraction FLOPs and algorithmic bytes per launch; bound by whichever of
    the MFMA peak of the workload's type and HBM its intensity puts it under."""
    med = {k: float(np.median(v)) for k, v in per.items() if k in KERNEL_FLOP_UNITS}
    name = max(med, key=med.get)
    base = w.tokens * w.heads * w.window * w.head_dim
    fl = KERNEL_FLOP_UNITS[name] * base
    by = algorithmic_bytes(w)[2][name]
    peak = mfma_peak(w.dtype)
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    t = med[name] * 1e-3
    out = {"kernel": name, "flops_per_launch": fl, "bytes_per_launch": by,
           "intensity_flop_per_byte": round(fl / by, 2), "ridge_flop_per_byte": round(ridge, 2),
           "avg_launch_ms": round(med[name], 4), "dtype": DTYPE_LABEL[w.dtype]}
    if fl / by >= ridge:
        achieved = fl / t / 1e12
        out.update({"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4)})
    else:
        achieved = by / t / 1e9
        out.update({"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)})
    out["traffic"] = recorded_traffic(name, tag or w.name)
    return out


def leg(w, per, wall=None, warm=None, tag=None):
    """Summary of one timed workload: cold (flushed) medians, the roofline of
    its longest kernel, and the warm medians beside them."""
    out = summarize(w, per)
    out["roofline"] = roofline(w, per, tag)
    if wall is not None:
        out["wall_ms_per_step"] = round(wall, 4)
    if warm is not None:
        ws = summarize(w, warm)
        out["warm"] = {k: ws[k] for k in ("fwd_ms", "bwd_ms", "ms_per_step", "tflops_total")}
    return out


def cpu_baseline(w, host, target_s, seed=1, gpu=None):
    """The oracle on a random sample of (b, token, head) units sized for about
    target_s seconds, scaled linearly to the workload. With the GPU results of
    the timed passes (gpu), the sample's oracle values also give the parity
    errors of every output tensor at those units (max abs error over max abs
    reference value)."""
    import oracle
    q, k, v, dout = (t.float().numpy().astype(np.float64) for t in host)
    units = w.tokens * w.heads
    rng = np.random.default_rng(seed)

    def run(n):
        sel = np.sort(rng.integers(0, units, n))
        t0 = time.perf_counter()
        o, lse = oracle.na_fwd(q, k, v, w.kernel, w.dilation, w.the_scale, sel=sel)
        dq, dk, dv = oracle.na_bwd(q, k, v, dout, w.kernel, w.dilation, w.the_scale, sel=sel)
        return time.perf_counter() - t0, sel, {"out": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}

    # a warm-up call (thread team start-up), then a pilot long enough to time,
    # sizes the sample to about target_s of work; one resize if it came out short
    run(256)
    pilot_n = 8192
    t_pilot = run(pilot_n)[0]
    n = int(max(pilot_n, min(units, pilot_n * target_s / max(t_pilot, 1e-6))))
    log(f"[bench] oracle pilot {pilot_n} units {t_pilot:.2f}s -> sample {n} units")
    t, sel, ref = run(n)
    if t < 0.5 * target_s and n < units:
        n = int(min(units, n * target_s / max(t, 1e-6)))
        log(f"[bench] oracle sample short ({t:.1f}s) -> {n} units")
        t, sel, ref = run(n)
    f_fwd, f_bwd = flops(w)
    full_s = t * units / n
    out = {"value": round((f_fwd + f_bwd) / full_s / 1e12, 6), "unit": "TFLOP/s",
           "cores": oracle.num_threads(), "kind": "oracle",
           "sample": (f"{n} random (b, token, head) units of {w.name}: forward and dq at them "
                      f"as queries, dk and dv at them as keys, fp64, {t:.1f} s; rate "
                      f"extrapolated linearly to the whole workload ({full_s:.0f} s)"),
           "est_full_ms": round(full_s * 1e3, 1)}
    if gpu is not None:
        errs = {}
        for name, r in ref.items():
            flat = gpu[name].float().numpy()
            g = (flat.reshape(-1)[sel] if name == "lse" else
                 flat.reshape(-1, w.head_dim)[sel]).astype(np.float64)
            errs[name] = float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-30))
        out["parity"] = {"units": int(n), "max_rel_err": {k_: round(e, 8) for k_, e in errs.items()},
                         "tolerance": TOLERANCE[w.dtype],
                         "within": bool(all(e <= TOLERANCE[w.dtype] for e in errs.values()))}
    return out


def host_info():
    """Where the numbers were taken: host CPU, GPU, ROCm and the library build."""
    model = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    from fwd_bwd_amd import build as hipbuild
    lib_sha = na.source_sha256()
    return {"cpu_count": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "cpu_model": model, "gpu": torch.cuda.get_device_name(0),
            "gpu_arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
            "rocm": rocm, "torch_hip": torch.version.hip, "torch": torch.__version__,
            "libna_source_sha256": lib_sha,
            "libna_matches_tree": lib_sha == hipbuild.source_sha256()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--variant", default="gather", choices=["gather", "kvparallel"])
    ap.add_argument("--kv-splits", type=int, default=0,
                    help="accumulator copies of the KV-parallel backward (0: atomics)")
    ap.add_argument("--no-secondary", action="store_true", help="skip the 3D workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused-path leg")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the KV-parallel backward, fp16 and bf16 legs")
    ap.add_argument("--no-flush", action="store_true",
                    help="time warm passes only (no cache flush between passes)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--source-hash", action="store_true", help="print the kernel source hash")
    ap.add_argument("--frame", type=int, default=None,
                    help="only time the workload with every window restricted to this many "
                         "positions along the outermost axis (na_fwd_framed / na_bwd_framed; "
                         "prints the times alone)")
    args = ap.parse_args()
    if args.source_hash:
        print(kernel_source_hash())
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: neighborhood attention here runs on a single "
              "MI355X; this benchmark does not run several GPUs.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    na.load()

    if args.calibrate_copy:
        # a plain copy of known size: 1 GiB read, 1 GiB written per launch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel() * 4, "launches": 3}))
        return

    flush = None if args.no_flush else torch.empty(FLUSH_BYTES, dtype=torch.uint8,
                                                   device="cuda:0")

    def timed(wl, variant, steps, warmup, kv_splits=0):
        r = Runner(wl, variant, kv_splits=kv_splits)
        log(f"[bench] timing {wl.name} ({variant}, kv_splits {kv_splits}): warmup {warmup}, "
            f"steps {steps}")
        per, wall = r.time(steps, warmup, flush)
        warm = None
        if flush is not None:
            warm, _ = r.time(steps, 0, None)
        out = leg(wl, per, wall, warm,
                  wl.name if variant == "gather" else f"{wl.name}_kv{kv_splits}")
        log(f"[bench] {wl.name} ({variant}): step {out['ms_per_step']} ms, "
            f"fwd {out['fwd_ms']} ms, bwd {out['bwd_ms']} ms, {out['tflops_total']} TFLOP/s")
        return r, out

    w = WORKLOADS[args.workload]
    if args.frame is not None:
        # restricted windows only (one kernel trace holds the framed launches alone)
        frame = [args.frame] * w.grid[0]
        rf = FramedRunner(w, frame)
        log(f"[bench] timing {w.name} with frame {args.frame}")
        per, _ = rf.time(args.steps, args.warmup, flush)
        s = summarize(w, per)
        print(json.dumps({"workload": w.name, "frame": args.frame,
                          "kept_fraction": round(kept_fraction(w, frame), 4),
                          **{k: s[k] for k in ("fwd_ms", "bwd_ms", "ms_per_step", "kernel_ms")}}),
              flush=True)
        return
    r, main_leg = timed(w, args.variant, args.steps, args.warmup, args.kv_splits)
    gpu_main = None if args.no_cpu_baseline else r.outputs_host()

    result = {
        "metric": METRIC,
        "value": main_leg["tflops_total"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_leg["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_LABEL[w.dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "grid": list(w.grid),
                   "heads": w.heads, "head_dim": w.head_dim, "kernel": list(w.kernel),
                   "dilation": list(w.dilation), "backward": args.variant,
                   **({"kv_splits": args.kv_splits} if args.variant == "kvparallel" else {}),
                   "timing": "median of cold passes (1 GiB flush before each pass)"
                   if flush is not None else "median of warm passes"},
        **{k: v for k, v in main_leg.items() if k != "ms_per_step"},
    }

    host = r.host
    del r
    torch.cuda.empty_cache()
    unfused = {}

    def run_unfused(wl, h):
        if args.no_unfused or wl.dtype != torch.float32:
            return
        u = UnfusedRunner(wl, h)
        log(f"[bench] timing the unfused ops on {wl.name}")
        step, per_u = u.time(args.steps, args.warmup)
        unfused[wl.name] = unfused_summary(wl, step, per_u)
        unfused[wl.name]["chain_ms_per_step"] = round(u.time_chain(args.steps, args.warmup), 4)
        log(f"[bench] unfused {wl.name}: {unfused[wl.name]}")
        del u
        torch.cuda.empty_cache()

    run_unfused(w, host)
    if not args.no_extra and args.workload == HEADLINE:
        # the KV-parallel backward on the same inputs, and the same shape with fp16
        # tensors (the maintainer's second profiled precision)
        extra = {}
        if args.variant == "gather":
            # kv_splits 0: float atomics into one accumulator; 1 and 4: bounded copies of the
            # accumulator, bitwise reproducible (the memory-preference cap)
            nk = min(args.steps, 2)
            kvp = {}
            for splits in (0, 1, 4):
                rk, kvp[f"kv_splits_{splits}"] = timed(w, "kvparallel", nk, min(args.warmup, 1),
                                                       splits)
                kvp[f"kv_splits_{splits}"]["steps"] = nk
                del rk
                torch.cuda.empty_cache()
            extra["kvparallel"] = kvp
        w16 = WORKLOADS.get(w.name.replace("_f32", "_f16"))
        if w16 is not None:
            r16, s16 = timed(w16, args.variant, args.steps, args.warmup)
            extra["fp16"] = {"workload": w16.name, **s16}
            del r16
            torch.cuda.empty_cache()
        result.update(extra)
    h3 = gpu_3d = None
    if not args.no_secondary and args.workload == HEADLINE:
        w3 = WORKLOADS[HEADLINE_3D]
        r3, s3 = timed(w3, args.variant, args.steps, args.warmup)
        result["secondary"] = {"workload": w3.name, **s3}
        h3 = r3.host
        gpu_3d = None if args.no_cpu_baseline else r3.outputs_host()
        del r3
        torch.cuda.empty_cache()
        if not args.no_extra and args.variant == "gather":
            # the same 3D step with windows restricted per frame (na_fwd_framed /
            # na_bwd_framed): constant time windows of 1 and 2 of the 3 planes
            framed = {}
            for f in (1, 2):
                frame = [f] * w3.grid[0]
                rf = FramedRunner(w3, frame, host=h3)
                log(f"[bench] timing {w3.name} with frame {f}")
                per, _ = rf.time(args.steps, args.warmup, flush)
                framed[f"frame_{f}"] = {"kept_fraction": round(kept_fraction(w3, frame), 4),
                                        **framed_leg(w3, per, s3)}
                del rf
                torch.cuda.empty_cache()
            result["secondary"]["framed"] = framed
            # the same step with an arbitrary window mask keeping 2/3 of every
            # window at random (na_fwd_masked / na_bwd_masked)
            rm = MaskedRunner(w3, random_window_mask(w3, 2 / 3), host=h3)
            log(f"[bench] timing {w3.name} with a random window mask")
            per, _ = rm.time(args.steps, args.warmup, flush)
            result["secondary"]["masked"] = {"kept_fraction": 0.6667, **framed_leg(w3, per, s3)}
            del rm
            torch.cuda.empty_cache()
        run_unfused(w3, h3)
    if unfused:
        result["unfused"] = unfused
    if not args.no_extra and args.workload == HEADLINE:
        # the two bf16 workloads (fp32 accumulate), each against the roofline of its
        # own type: 16-bit MFMA or HBM, whichever its arithmetic intensity binds
        bf16 = {}
        for name in BF16_WORKLOADS:
            wb = WORKLOADS[name]
            nb = min(args.steps, 5)
            rb, sb = timed(wb, args.variant, nb, min(args.warmup, 2))
            bf16[name] = {"steps": nb, **sb}
            del rb
            torch.cuda.empty_cache()
            if wb.head_dim == 32:
                # the same step with a random window mask keeping 2/3 of every
                # window: masked 16-bit problems compute in fp32 on the
                # register-resident kernels
                rm = MaskedRunner(wb, random_window_mask(wb, 2 / 3))
                log(f"[bench] timing {name} with a random window mask")
                per, _ = rm.time(nb, min(args.warmup, 2), flush)
                bf16[name]["masked"] = {"kept_fraction": 0.6667, **framed_leg(wb, per, sb)}
                del rm
                torch.cuda.empty_cache()
        result["bf16"] = bf16

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds, gpu=gpu_main)
        if h3 is not None:
            result["secondary"]["cpu_baseline"] = cpu_baseline(WORKLOADS[HEADLINE_3D], h3,
                                                               args.cpu_seconds, gpu=gpu_3d)
    else:
        result["cpu_baseline"] = None

    result["host"] = host_info()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
