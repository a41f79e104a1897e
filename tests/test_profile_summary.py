"""profile_summary.py (the tool that writes the profiles/ summaries) on
synthetic rocprofv3 CSV output: dispatch selection by launch order, the
per-kernel statistics, the HBM-traffic scaling against the calibration copy
and the counter ratios."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import profile_summary as ps  # noqa: E402

FWD = "void (anonymous namespace)::fa_fwd_kernel<1, 128, false, false, false, 8>(x)"
MERGE = "void (anonymous namespace)::fa_merge_kernel<1, 128>(y)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_ktrace_selects_timed_dispatches_in_launch_order(tmp_path):
    # dispatch ids out of file order; durations 1000 * id ns
    rows = []
    for i in (3, 1, 2, 5, 4, 6):
        rows.append([i, FWD, 10_000 * i, 10_000 * i + 1000 * i])
        rows.append([100 + i, MERGE, 0, 7])
    _write(str(tmp_path / "kt" / "run_kernel_trace.csv"),
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = tmp_path / "s.txt"
    ps.main(["ktrace", "--dir", str(tmp_path / "kt"), "--kernel", "fa_fwd_kernel", "--skip", "2",
             "--take", "3", "--flops", "3e6", "--also", "fa_merge_kernel", "--title", "t",
             "--command", "c", "-o", str(out)])
    text = out.read_text()
    # dispatches 3, 4, 5 (after skipping 1 and 2): 3000, 4000, 5000 ns
    assert "dispatches: 3  mean_ns: 4000  median_ns: 4000  min_ns: 3000  max_ns: 5000" in text
    assert "TFLOP/s at mean: 0.7" in text           # 3e6 FLOP / 4 us = 0.75 TFLOP/s
    assert "kernel: fa_merge_kernel<1, 128>" in text
    assert "sum of the kernels' mean durations (one step): 4007 ns" in text
    assert "--also fa_merge_kernel --skip 2 --take 3" in text


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # the 1 GiB copy reads 524288 KiB by FETCH_SIZE (factor 2) and writes 1048576 KiB
    _write(str(tmp_path / "f" / "run_counter_collection.csv"), hdr,
           [[1, COPY, "FETCH_SIZE", 524288.0], [2, FWD, "FETCH_SIZE", 999.0],
            [3, FWD, "FETCH_SIZE", 100.0], [4, FWD, "FETCH_SIZE", 300.0]])
    _write(str(tmp_path / "w" / "run_counter_collection.csv"), hdr,
           [[1, COPY, "WRITE_SIZE", 1048576.0], [2, FWD, "WRITE_SIZE", 999.0],
            [3, FWD, "WRITE_SIZE", 50.0], [4, FWD, "WRITE_SIZE", 50.0]])
    out = tmp_path / "t.txt"
    ps.main(["traffic", "--fetch-dir", str(tmp_path / "f"), "--write-dir", str(tmp_path / "w"),
             "--kernel", "fa_fwd_kernel", "--skip", "1", "--algorithmic", str(1024 * 450),
             "--title", "t", "--command", "c", "-o", str(out)])
    text = out.read_text()
    # fetch: mean 200 KiB x 2 = 400 KiB; write: 50 KiB x 1
    assert "fetch_bytes_per_launch: 4.0960e+05" in text
    assert "write_bytes_per_launch: 5.1200e+04" in text
    assert "traffic / algorithmic: 1.000" in text


def test_counters_clock_and_busy(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    t_ns = 1_000_000                                   # 1 ms per dispatch
    grbm = 8 * 2.0e9 * 1e-3                            # 8 XCDs at 2.0 GHz for 1 ms
    busy = 0.5 * grbm / 8 * 1024                       # matrix pipe half busy
    _write(str(tmp_path / "p" / "run_counter_collection.csv"), hdr,
           [[1, FWD, "GRBM_GUI_ACTIVE", grbm], [1, FWD, "SQ_VALU_MFMA_BUSY_CYCLES", busy],
            [1, FWD, "SQ_WAVES", 10.0], [1, FWD, "SQ_INSTS_MFMA", 160.0],
            [1, FWD, "SQ_INSTS_VALU", 160.0 + 590.0]])
    _write(str(tmp_path / "p" / "run_kernel_trace.csv"),
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], [[1, FWD, 0, t_ns]])
    out = tmp_path / "c.txt"
    ps.main(["counters", "--dirs", str(tmp_path / "p"), "--kernel", "fa_fwd_kernel",
             "--title", "t", "--command", "c", "-o", str(out)])
    text = out.read_text()
    assert "engine clock = GRBM_GUI_ACTIVE / 8 XCDs / time: 2.000 GHz" in text
    assert "(GRBM_GUI_ACTIVE / 8 x 1024 SIMDs): 0.500" in text
    assert "per 16 MFMA: VALU excl. MFMA 59.0" in text


def test_missing_kernel_fails(tmp_path):
    _write(str(tmp_path / "kt" / "run_kernel_trace.csv"),
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], [[1, MERGE, 0, 5]])
    with pytest.raises(SystemExit):
        ps.main(["ktrace", "--dir", str(tmp_path / "kt"), "--kernel", "fa_fwd_kernel",
                 "--title", "t", "--command", "c", "-o", str(tmp_path / "x.txt")])
