"""CPU: the rocprofv3 report helpers behind profiles/ (no GPU, synthetic CSVs).

The kernel report must keep workloads that share one kernel instantiation
apart (M=64 and M=256 share a grid, so duration decides), and the SQ report
must derive its figures from the counters it was given."""

from __future__ import annotations

import csv

from tp_vocab_logits_amd import profiling

FUSED1 = "void hg::(anonymous namespace)::k_fused<1, 2, 2, 8>(hg::Geometry, int)"
FUSED2 = "void hg::(anonymous namespace)::k_fused<2, 2, 2, 8>(hg::Geometry, int)"
GEMM = "void hg::(anonymous namespace)::k_lmhead_4x2<8, true, false, true>(int)"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _trace(tmp_path, dispatches):
    """dispatches: (name, grid threads, duration ns)."""
    rows, t = [], 1000
    for i, (name, grid, ns) in enumerate(dispatches):
        rows.append(["KERNEL_DISPATCH", 1, 1, 1, 1, i + 1, 7, name, i + 1, t, t + ns, 0, 0, 32, 0, 16,
                     256, 1, 1, grid, 1, 1])
        t += ns + 500
    path = tmp_path / "t_kernel_trace.csv"
    _write(path, ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
                  "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
                  "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
                  "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"], rows)
    return str(path)


def _stats(tmp_path, dispatches):
    per = {}
    for name, _, ns in dispatches:
        per.setdefault(name, []).append(ns)
    total = sum(sum(v) for v in per.values())
    rows = [[n, len(v), sum(v), sum(v) / len(v), 100.0 * sum(v) / total, min(v), max(v), 0.0]
            for n, v in per.items()]
    path = tmp_path / "t_kernel_stats.csv"
    _write(path, ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                  "StdDev"], rows)
    return str(path)


def test_kernel_report_separates_row_counts_sharing_a_kernel(tmp_path):
    d = ([(FUSED1, 20480, 3300)] * 50 + [(FUSED1, 81920, 3900)] * 20 + [(FUSED1, 512, 2500)] * 10
         + [(FUSED2, 262144, 17000)] * 30 + [(FUSED2, 262144, 61000)] * 6 + [(FUSED2, 262144, 62000)] * 2
         + [(GEMM, 262144, 650000)] * 3)
    text = profiling.kernels_report(_stats(tmp_path, d), "cmd", _trace(tmp_path, d))
    # per name the M=64 and M=256 calls are mixed ...
    assert "| `hg::k_fused<2, 2, 2, 8>` | 38 |" in text
    # ... the M=256 line takes only the eight calls above 40 us: 61.25 us
    m256 = next(ln for ln in text.splitlines() if ln.startswith("M=256"))
    assert "8 calls, 61.25 us average" in m256
    assert f"{profiling.M256_BYTES / 61.25e-6 / 1e9:.1f} GB/s" in m256
    # the decode line takes the most frequent fused launch shape only
    m1 = next(ln for ln in text.splitlines() if ln.startswith("M=1"))
    assert "grid 20480 threads" in m1 and "50 calls, 3.300 us average" in m1
    # every (kernel, grid) pair has its own row
    assert "| `hg::k_fused<1, 2, 2, 8>` | 81920 | 20 |" in text
    assert "| `hg::k_fused<2, 2, 2, 8>` | 262144 | 38 |" in text


def test_kernel_report_without_trace_has_no_workload_lines(tmp_path):
    d = [(FUSED2, 262144, 61000)] * 3
    text = profiling.kernels_report(_stats(tmp_path, d), "cmd", None)
    assert "M=256" not in text and "M=1" not in text and "hg::k_fused<2, 2, 2, 8>" in text


def _counters(tmp_path, name, values, dur_ns=500_000):
    rows, t = [], 10_000
    for disp, (counter, v) in enumerate(values):
        rows.append([1, disp + 1, "Agent 1", 1, 1, 1, 262144, 3, GEMM, 512, 0, 0, 240, 0, 30, counter, v,
                     t, t + dur_ns])
        t += dur_ns + 1000
    path = tmp_path / f"{name}_counter_collection.csv"
    _write(path, ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
                  "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size",
                  "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value",
                  "Start_Timestamp", "End_Timestamp"], rows)
    return str(path)


def test_sq_report_derivations(tmp_path):
    # 2.0 GHz over 500 us on 8 XCDs; MFMA busy half of 1024 SIMDs' cycles
    cyc = 2.0e9 * 500e-6
    a = _counters(tmp_path, "a", [("GRBM_GUI_ACTIVE", 8 * cyc)])
    b = _counters(tmp_path, "b", [("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * cyc), ("SQ_INSTS_MFMA", 0.5 * 1024 * cyc / 32)])
    c = _counters(tmp_path, "c", [("SQ_LDS_BANK_CONFLICT", 25.0), ("SQ_LDS_IDX_ACTIVE", 100.0),
                                  ("SQ_WAIT_INST_ANY", 40.0), ("SQ_WAVE_CYCLES", 100.0),
                                  ("TCC_HIT_sum", 3.0), ("TCC_MISS_sum", 1.0)])
    text = profiling.sq_report([a, b, c], "k_lmhead", ["cmd a", "cmd b", "cmd c"])
    assert "shader clock: GRBM_GUI_ACTIVE / 8 / that dispatch's duration = 2.00 GHz" in text
    assert "= 50.0 %" in text                       # MFMA busy per SIMD
    assert "busy cycles per MFMA instruction: 32.0" in text
    assert "LDS active cycles: 25.0 %" in text
    assert "SQ_WAVE_CYCLES = 40.0 %" in text
    assert "L2 hit rate: 75.0 %" in text
    for cmd in ("cmd a", "cmd b", "cmd c"):
        assert "    " + cmd in text


def test_m1_fused_times_takes_the_most_frequent_fused_shape(tmp_path):
    # the timed M=1 loop is the most frequent fused launch; other fused shapes
    # and other kernels do not enter its median
    d = ([(FUSED1, 20480, 3000 + 10 * (i % 7)) for i in range(51)] + [(FUSED1, 81920, 3900)] * 20
         + [(FUSED2, 262144, 61000)] * 30 + [(GEMM, 262144, 650000)] * 60)
    m1 = profiling.m1_fused_times(_trace(tmp_path, d))
    assert m1["grid_threads"] == 20480 and m1["calls"] == 51
    assert m1["median_us"] == 3.03 and m1["min_us"] == 3.0
    assert m1["kernel_source_sha256_16"] == profiling.kernel_source_hash()
    assert profiling.m1_fused_times(_trace(tmp_path, [(GEMM, 262144, 650000)])) is None


def test_clock_report_per_dispatch(tmp_path):
    # two dispatches: 500 us at 2.0 GHz with MFMA busy 60 %, 625 us at 1.6 GHz
    rows, t = [], 10_000
    for disp, (ns, ghz, busy) in enumerate([(500_000, 2.0, 0.6), (625_000, 1.6, 0.65)]):
        cyc = ghz * ns
        for counter, v in (("GRBM_GUI_ACTIVE", 8 * cyc), ("SQ_VALU_MFMA_BUSY_CYCLES", busy * 1024 * cyc)):
            rows.append([1, disp + 1, "Agent 1", 1, 1, 1, 262144, 3, GEMM, 512, 0, 0, 240, 0, 30, counter, v,
                         t, t + ns])
        t += ns + 1000
    path = tmp_path / "clk_counter_collection.csv"
    _write(path, ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
                  "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size",
                  "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value",
                  "Start_Timestamp", "End_Timestamp"], rows)
    text = profiling.clock_report(str(path), "k_lmhead", "the command")
    assert "| 1 | 500.0 | 2.00 | 60.0 | 1000 |" in text
    assert "| 2 | 625.0 | 1.60 | 65.0 | 1000 |" in text
    assert "fastest 500.0 us at 2.00 GHz, slowest 625.0 us at 1.60 GHz" in text
    assert "    the command" in text


def test_m1_split_times_sum_push_and_collect_at_the_decode_grid(tmp_path):
    push = "void hg::(anonymous namespace)::k_push<1, 8>(int)"
    coll = "void hg::(anonymous namespace)::k_collect<1, 1>(int)"
    d = ([(push, 20480, 2700 + 10 * (i % 3)) for i in range(30)] + [(coll, 20480, 2800)] * 30
         + [(push, 1048576, 30000)] * 40 + [(coll, 1048576, 37000)] * 40)
    sp = profiling.m1_split_times(_trace(tmp_path, d), 20480)
    assert sp["push"]["median_us"] == 2.71 and sp["collect"]["median_us"] == 2.8
    assert sp["sum_median_us"] == 5.51 and sp["push"]["calls"] == 30
    assert profiling.m1_split_times(_trace(tmp_path, [(push, 20480, 2700)]), 20480) is None
