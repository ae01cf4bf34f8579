"""CPU checks of bench.py's throughput model against the figures the pages
print (tests/golden/arithmetic_intensity.json): the fused forward's FLOPs over
its algorithmic bytes must reproduce the maintainer's arithmetic intensities
of the issue's two fp32 problems, and the same roofline arithmetic must give
the ridge point the page quotes for the A40."""
import json
import os

import pytest

import bench
import torch

from fwd_bwd_amd.inputs import WORKLOADS, make_inputs

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "arithmetic_intensity.json")))


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=[c["workload"] for c in GOLDEN["cases"]])
def test_fused_arithmetic_intensity_matches_page(case):
    w = WORKLOADS[case["workload"]]
    f_fwd, f_bwd = bench.flops(w)
    b_fwd, b_bwd, _ = bench.algorithmic_bytes(w)
    ai = f_fwd / b_fwd
    assert abs(ai - case["fused_flop_per_byte_approx"]) <= 0.5, ai
    # the backward metric is 2.5x the forward FLOPs
    assert f_bwd == pytest.approx(2.5 * f_fwd)


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=[c["workload"] for c in GOLDEN["cases"]])
def test_unfused_arithmetic_intensity_model(case):
    # unfused forward: q, k, v read and out written (4D values per token-head),
    # the window weights written once and read once (2K values per token-head)
    w = WORKLOADS[case["workload"]]
    f_fwd, _ = bench.flops(w)
    units = w.tokens * w.heads
    bytes_unfused = 4 * units * (4 * w.head_dim + 2 * w.window)
    assert abs(f_fwd / bytes_unfused - case["unfused_flop_per_byte_approx"]) <= 0.5


def test_a40_ridge():
    a = GOLDEN["a40"]
    ridge = a["peak_tflops"] * 1e12 / (a["hbm_gbs"] * 1e9)
    assert abs(ridge - a["ridge_flop_per_byte_approx"]) <= 0.5


def test_mi355x_ridges_used_by_bench():
    # fp32 MFMA 157.3 TFLOP/s over 8 TB/s: the headline problems sit at the ridge
    ridge = bench.PEAK_TFLOPS["fp32_mfma"] * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    assert 19 < ridge < 20.5


def test_traffic_only_reported_for_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "traffic_k_w.md").write_text("source_sha256: " + "0" * 64 + "\nhbm_bytes_per_launch: 5e9\n")
    assert bench.recorded_traffic("k", "w") is None
    (tmp_path / "traffic_k_w.md").write_text(
        "source_sha256: " + bench.kernel_source_hash() + "\nhbm_bytes_per_launch: 5e9\n")
    assert bench.recorded_traffic("k", "w") == 5e9


def test_bench_side_workloads_exist():
    """The workloads the bench times beside the headline are defined, with
    the types their legs assume."""
    import torch
    for name in bench.BF16_WORKLOADS:
        assert name in WORKLOADS and WORKLOADS[name].dtype == torch.bfloat16, name
    assert WORKLOADS[bench.HEADLINE].dtype == torch.float32
    assert WORKLOADS[bench.HEADLINE_3D].dtype == torch.float32
    assert bench.HEADLINE.replace("_f32", "_f16") in WORKLOADS


def _per(ms):
    return {k: [v, v, v] for k, v in ms.items()}


def test_roofline_picks_the_bound_of_each_workloads_type():
    """fp32 kernels with intensity above the fp32 ridge are priced against the
    fp32 MFMA peak; the 16-bit workloads sit below the 16-bit MFMA ridge
    (2516.6 TFLOP/s over 8 TB/s) and are priced against HBM."""
    import torch
    w = WORKLOADS[bench.HEADLINE]
    r = bench.roofline(w, _per({"fwd": 1.0, "bwd_dq": 2.0, "bwd_dkdv": 3.0}))
    assert r["kernel"] == "bwd_dkdv" and r["bound"] == "mfma" and r["peak"] == 157.3
    base = w.tokens * w.heads * w.window * w.head_dim
    assert r["achieved"] == pytest.approx(8 * base / 3e-3 / 1e12, rel=1e-3)
    for name in bench.BF16_WORKLOADS:
        wb = WORKLOADS[name]
        rb = bench.roofline(wb, _per({"fwd": 1.0, "bwd_dq": 2.0, "bwd_dkdv": 3.0}))
        assert rb["bound"] == "hbm" and rb["unit"] == "GB/s" and rb["peak"] == bench.PEAK_HBM_GBS
        assert rb["intensity_flop_per_byte"] < rb["ridge_flop_per_byte"]
        by = bench.algorithmic_bytes(wb)[2]["bwd_dkdv"]
        assert rb["achieved"] == pytest.approx(by / 3e-3 / 1e9, rel=1e-3)
        s = bench.summarize(wb, _per({"fwd": 1.0, "bwd_dq": 2.0, "bwd_dkdv": 3.0}))
        assert s["mfma_peak_tflops"] == bench.PEAK_TFLOPS["bf16_mfma"]
    assert bench.mfma_peak(torch.float16) == bench.PEAK_TFLOPS["bf16_mfma"]
    assert bench.DTYPE_LABEL[torch.float16] == "f16"
    assert bench.DTYPE_LABEL[torch.bfloat16] == "bf16"


def test_summarize_reports_medians_and_the_step_sum():
    w = WORKLOADS[bench.HEADLINE]
    per = {"fwd": [1.0, 5.0, 2.0], "bwd_dq": [2.0, 2.0, 9.0], "bwd_dkdv": [3.0, 3.0, 3.0]}
    s = bench.summarize(w, per)
    assert s["fwd_ms"] == 2.0 and s["fwd_ms_stats"]["min"] == 1.0
    # per step: 6, 10, 14 -> median 10; backward per step 5, 5, 12 -> median 5
    assert s["ms_per_step"] == 10.0 and s["bwd_ms"] == 5.0


def test_cpu_baseline_parity_check_reads_the_sampled_units():
    """bench.cpu_baseline compares the GPU results it is given with the
    oracle at the sampled units: results equal to the oracle's pass, a 0.1%
    error in one tensor is reported for that tensor."""
    import numpy as np
    import oracle
    w = WORKLOADS["2d_16x16_k3_h2_d16_f32"]
    host = make_inputs(w, 0)
    q, k, v, do = (t.double().numpy() for t in host)
    o, lse = oracle.na_fwd(q, k, v, w.kernel, w.dilation, w.the_scale)
    dq, dk, dv = oracle.na_bwd(q, k, v, do, w.kernel, w.dilation, w.the_scale)
    gpu = {n: torch.tensor(np.asarray(x)) for n, x in
           (("out", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    par = bench.cpu_baseline(w, host, 0.2, gpu=gpu)["parity"]
    assert par["within"] and max(par["max_rel_err"].values()) < 1e-6
    gpu["dk"] = gpu["dk"] * 1.001
    par = bench.cpu_baseline(w, host, 0.2, gpu=gpu)["parity"]
    assert not par["within"]
    assert abs(par["max_rel_err"]["dk"] - 1e-3) < 1e-5 and par["max_rel_err"]["dq"] < 1e-6


def test_framed_leg_kept_fraction_and_ratios():
    """The restricted-window leg: a constant frame of f of the 3 time planes
    keeps f/3 of every window (sizes above the window or below zero are
    clipped), and the leg's times are reported against the full step."""
    w = WORKLOADS[bench.HEADLINE_3D]
    assert bench.kept_fraction(w, [1] * w.grid[0]) == pytest.approx(1 / 3)
    assert bench.kept_fraction(w, [2] * w.grid[0]) == pytest.approx(2 / 3)
    assert bench.kept_fraction(w, [5] * 8 + [0] * 8) == pytest.approx(0.5)
    per = {"fwd": [1.0, 1.0, 1.0], "bwd_framed": [2.0, 3.0, 2.0]}
    full = {"fwd_ms": 2.0, "bwd_ms": 8.0, "ms_per_step": 10.0}
    leg = bench.framed_leg(w, per, full)
    assert leg["ms_per_step"] == 3.0
    assert leg["time_vs_full"] == {"fwd": 0.5, "bwd": 0.25, "step": 0.3}


def test_random_window_mask_of_the_masked_leg():
    """The masked leg's mask: bytes [(T,) H, W, K], seeded, about 2/3 ones."""
    import torch
    w = bench.WORKLOADS["2d_16x16_k3_h2_d16_f32"]
    m1, m2 = bench.random_window_mask(w, 2 / 3), bench.random_window_mask(w, 2 / 3)
    assert m1.dtype == torch.uint8 and tuple(m1.shape) == tuple(w.grid) + (w.window,)
    assert torch.equal(m1, m2)
    assert set(m1.unique().tolist()) <= {0, 1}
    assert abs(float(m1.float().mean()) - 2 / 3) < 0.05
