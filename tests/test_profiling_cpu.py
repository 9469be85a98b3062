"""The rocprofv3 CSV summarizer on small fabricated files (column layout of rocprofv3's CSV output)."""
import csv

from mixture_experts_layer_sum_amd import profiling

G1 = "void fsm::k_gemm_bf16<256, 256, 2, 4, 1, 0>(fsm::GemmArgs)"
R = "void fsm::k_gemm_bf16<256, 256, 2, 4, 2, 1>(fsm::GemmArgs)"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_overlap(tmp_path, capsys):
    p = tmp_path / "t.csv"
    hdr = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    # main queue 1 busy [0,100) and [150,250); side queue 2 busy [50,120): overlap 50 of side's 70
    _write(p, hdr, [["KERNEL_DISPATCH", 1, 1, 1, 1, G1, 0, 100], ["KERNEL_DISPATCH", 1, 2, 2, 2, R, 50, 120],
                    ["KERNEL_DISPATCH", 1, 1, 1, 3, G1, 150, 250], ["KERNEL_DISPATCH", 1, 3, 3, 4, "other", 0, 999]])
    profiling.main(["trace", str(p)])
    out = capsys.readouterr().out
    assert "|M n S|/|S| = 0.7143" in out
    assert "|M n S|/|M| = 0.2500" in out


def test_counters_calibration(tmp_path, capsys):
    p = tmp_path / "c.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(p, hdr, [[1, "elementwise_copy_kernel", "FETCH_SIZE", 1048576 / 2], [2, G1, "FETCH_SIZE", 1000.0],
                    [3, G1, "FETCH_SIZE", 3000.0]])
    profiling.main(["counters", str(p), "--copy-gib", "1"])
    out = capsys.readouterr().out
    assert "scale 2.0000" in out
    assert "FETCH_SIZE=2000" in out and "(0.004 GB calibrated)" in out
    assert "grouped GEMM source digest" in out


def test_stats_filters_library_kernels(tmp_path, capsys):
    p = tmp_path / "s.csv"
    _write(p, ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"],
           [[G1, 4, 4e6, 1e6, 60.0], ["at::native::foo", 9, 1e3, 1e2, 1.0]])
    profiling.main(["stats", str(p)])
    out = capsys.readouterr().out
    assert "k_gemm_bf16" in out and "foo" not in out


def test_traffic_join_picks_copy_closest_to_size(tmp_path, capsys):
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    gib = 1048576.0
    # a 1.75 GiB conversion copy must not be taken for the 4 GiB calibration copy
    _write(f, hdr, [[1, "bf16_to_f32_copy", "FETCH_SIZE", 0.875 * gib], [2, "direct_copy", "FETCH_SIZE", 4.0 * gib],
                    [3, G1, "FETCH_SIZE", 2 * gib]])
    _write(w, hdr, [[1, "bf16_to_f32_copy", "WRITE_SIZE", 1.75 * gib], [2, "direct_copy", "WRITE_SIZE", 4.0 * gib],
                    [3, G1, "WRITE_SIZE", gib]])
    assert profiling.main(["traffic", "--fetch", str(f), "--write", str(w), "--copy-gib", "4"]) == 0
    out = capsys.readouterr().out
    assert "scale 1.0000" in out
    line = [l for l in out.splitlines() if l.startswith("traffic|") and "k_gemm_bf16" in l][0]
    fields = line.split("|")
    assert abs(float(fields[3]) - 2 * 2**30 / 1e9) < 1e-3 and abs(float(fields[4]) - 2**30 / 1e9) < 1e-3


def test_gemm_symbol_classification():
    gu8 = "void fsm::k_gemm_bf16<256, 256, 2, 4, 1, 2, 64, 2>(fsm::GemmArgs)"
    assert profiling.gemm_args(gu8) == (256, 256, 2, 4, 1, 2, 64, 2)
    assert profiling.is_routed_gate_up(gu8) and profiling.is_routed_gate_up(G1)
    assert profiling.is_routed("void fsm::k_gemm_bf16<64, 256, 1, 4, 0, 0, 32, 4>(fsm::GemmArgs)")
    shared = "void fsm::k_gemm_bf16<256, 256, 2, 4, 1, 1, 64, 2>(fsm::GemmArgs)"
    assert not profiling.is_routed_gate_up(shared) and not profiling.is_routed(shared)
    assert not profiling.is_routed(R) and profiling.gemm_args("fsm::k_combine(int)") is None
    # the weight-streaming flag of the 64-row tiles prints as a bool
    nt = "void fsm::k_gemm_bf16<64, 256, 1, 4, 1, 2, 64, 3, true>(fsm::GemmArgs)"
    assert profiling.gemm_args(nt) == (64, 256, 1, 4, 1, 2, 64, 3, 1) and profiling.is_routed_gate_up(nt)
    assert profiling.is_routed_gate_up("void fsm::k_gemm_bf16<256, 256, 2, 4, 1, 2, 64, 2, false>(fsm::GemmArgs)")


def test_overlap_of_intervals():
    # main busy [0, 10) and [20, 30); side busy [5, 25) (two pieces that touch): 10 of side's 20 hidden
    ov = profiling.overlap([(0, 10), (20, 30)], [(5, 15), (15, 25)])
    assert (ov["main"], ov["side"], ov["both"]) == (20, 20, 10)
    assert ov["side_hidden"] == 0.5 and ov["main_covered"] == 0.5
    # nested and repeated intervals are merged before measuring
    ov = profiling.overlap([(0, 4), (1, 2), (0, 4)], [(3, 8)])
    assert (ov["main"], ov["side"], ov["both"]) == (4, 5, 1)
    # one stream only: no side fraction
    assert profiling.overlap([(0, 1)], [])["side_hidden"] is None
