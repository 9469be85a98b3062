"""Host-side arithmetic of bench.py: the per-kernel roofline report, the bytes the fused combine
adds, and the workload names the per-workload leg times (no GPU)."""
import math
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_inputs as mi  # noqa: E402


def test_kernel_report_flop_and_byte_kinds():
    c = mi.BY_NAME["dsv3-stack"]
    N = c.T * c.k
    # two gate/up launches of 25 ms each, over one step
    rep = bench.kernel_report({"gemm_gate_up": (2, 50.0), "combine": (4, 8.0)}, c, steps=1)
    g = rep["gemm_gate_up"]
    assert g["launches"] == 2 and g["avg_ms"] == 25.0 and g["ms_per_step"] == 50.0
    flop = 4.0 * N * c.d * c.c
    assert g["tflops"] == pytest.approx(flop / 25e-3 / 1e12, abs=0.05)
    assert g["frac_mfma_peak"] == pytest.approx(g["tflops"] / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    # combine: read Y (bf16) and w/idx, read residual + shared, write fp32 out
    cb = rep["combine"]
    per = N * c.d * 2.0 + N * 8.0 + c.T * c.d * 10.0
    assert cb["gbs"] == pytest.approx(4 * per / 8e-3 / 1e9, rel=1e-4)
    assert cb["frac_hbm_peak"] == pytest.approx(cb["gbs"] / bench.PEAK_HBM_GBS, abs=1e-4)


def test_kernel_report_extra_bytes_and_empty_kinds():
    c = mi.BY_NAME["qwen3-30b-a3b"]
    base = bench.kernel_report({"combine": (3, 3.0), "topk": (0, 0.0)}, c, steps=3)
    extra = bench.kernel_report({"combine": (3, 3.0)}, c, steps=3, extra_bytes={"combine": 1e9})
    assert "topk" not in base            # kinds without launches are left out
    # 1 GB per step over 3 steps in 3 ms adds 1000 GB/s
    assert extra["combine"]["gbs"] - base["combine"]["gbs"] == pytest.approx(1000.0, abs=0.2)


def test_fused_input_bytes():
    c = mi.BY_NAME["dsv3-stack"]
    xb = c.T * c.d * 2.0
    assert bench.fused_input_bytes(c, "none") == 0.0
    # L - 2 combines also form the next input: a bf16 write, plus a read of S for partial inputs
    assert bench.fused_input_bytes(c, "partial") == (c.layers - 2) * 2 * xb
    assert bench.fused_input_bytes(c, "outdated") == (c.layers - 2) * xb
    assert bench.fused_input_bytes(c.scaled(layers=2), "partial") == 0.0
    assert bench.fused_input_bytes(c.scaled(n_shared=0), "partial") == (c.layers - 2) * xb


def test_small_workloads_are_single_layers_of_known_shape():
    seen = set()
    for name in bench.SMALL_WORKLOADS:
        c = mi.BY_NAME[name]
        assert c.layers == 1 and name not in seen
        seen.add(name)
        f = c.flops_per_token()
        assert f["total"] == 2 * c.d * c.E + 6 * c.d * c.c * c.k + 6 * c.d * c.shared_width
    # the layer FLOP per token of the DSV2-Lite and Scout workloads (router + routed + shared)
    assert mi.BY_NAME["dsv2-lite"].flops_per_token()["total"] == 262144 + 103809024 + 34603008
    assert mi.BY_NAME["llama4-scout"].flops_per_token()["total"] == 163840 + 251658240 + 251658240
    assert not math.isnan(bench.PEAK_F32_TFLOPS)


def test_stream_overlap_from_launch_intervals():
    # main stream 1: [0, 10) and [12, 20); side stream 2: [5, 14) and [30, 31)
    launches = [("gemm_gate_up", 1, 0.0, 10.0), ("router_gemm", 2, 5.0, 14.0), ("gemm_down", 1, 12.0, 20.0),
                ("combine", 2, 30.0, 31.0)]
    ov = bench.stream_overlap(launches, 1)
    # |M| = 18, |S| = 10, |M n S| = [5, 10) + [12, 14) = 7
    assert ov["main_busy_ms"] == 18.0 and ov["side_busy_ms"] == 10.0 and ov["both_busy_ms"] == 7.0
    assert ov["side_hidden_frac"] == 0.7 and ov["main_covered_frac"] == round(7 / 18, 4)
    assert ov["launches"] == 4


def test_route_report_per_layer():
    c = mi.BY_NAME["dsv3-stack"]
    kernels = {"router_gemm": {"ms_per_step": 1.8, "launches": 40}, "topk": {"ms_per_step": 0.44, "launches": 40}}
    r = bench.route_report(kernels, c)
    assert r["ms_per_layer"] == pytest.approx((1.8 + 0.44) / c.layers)
    nbytes = c.T * c.d * 2 + c.E * c.d * 2 + c.T * c.E * 4 + c.T * c.k * 8
    assert r["bytes_per_layer"] == nbytes
    assert r["gbs"] == pytest.approx(nbytes / (r["ms_per_layer"] * 1e-3) / 1e9, abs=0.1)
    assert r["frac_mfma_peak"] == pytest.approx(2.0 * c.T * c.d * c.E / (r["ms_per_layer"] * 1e-3) / 1e12
                                                / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    assert bench.route_report({"topk": {"ms_per_step": 1.0, "launches": 4}}, c) is None
    fused = bench.route_report({"router_gemm": {"ms_per_step": 2.0, "launches": 4}}, c)   # top-k in the epilogue
    assert fused["ms_per_layer"] == pytest.approx(2.0 / c.layers)


def test_host_cpu_reports_cores():
    h = bench.host_cpu()
    assert h["cores"] >= 1 and h["affinity_cpus"] >= 1
