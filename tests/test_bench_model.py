"""CPU checks of bench.py's throughput model against the figures the pages
print (tests/golden/arithmetic_intensity.json): the fused forward's FLOPs over
its algorithmic bytes must reproduce the maintainer's arithmetic intensities
of the issue's two fp32 problems, and the same roofline arithmetic must give
the ridge point the page quotes for the A40."""
import json
import os

import pytest

import bench
from fwd_bwd_amd.inputs import WORKLOADS

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
