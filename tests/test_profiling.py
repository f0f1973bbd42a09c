"""The rocprofv3 summary writer (int4_group_quantized_g128_amd/profiling.py) on synthetic
counter files with known values: copy-calibrated HBM bytes, trace averages, the
matrix-core and instruction-issue figures, and the key=value file bench.py reads."""
import csv
import os
import sys

import pytest

from int4_group_quantized_g128_amd import profiling

KERNEL = "void q4::k_gemm_pf<(q4::Act)2, 1, false, false, 1>(q4::GemmArgs)"
OTHER = "void q4::k_gemm_pf<(q4::Act)2, 0, false, false, 1>(q4::GemmArgs)"


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i, k, c, v])


@pytest.fixture
def summary(tmp_path, monkeypatch):
    st = tmp_path / "stats"
    st.mkdir()
    with open(st / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs"])
        w.writerow([KERNEL, 4, 400000, 100000.0])      # 100 us
        w.writerow([OTHER, 4, 200000, 50000.0])
    copy = profiling.COPY_KERNEL
    kib = profiling.COPY_BYTES // 1024
    # the copy reads half its bytes in FETCH_SIZE KiB (scale 2) and writes them exactly (scale 1)
    _write_counters(tmp_path / "fetch", [(copy, "FETCH_SIZE", kib // 2), (KERNEL, "FETCH_SIZE", 1000),
                                         (KERNEL, "FETCH_SIZE", 3000), (OTHER, "FETCH_SIZE", 7)])
    _write_counters(tmp_path / "write", [(copy, "WRITE_SIZE", kib), (KERNEL, "WRITE_SIZE", 10),
                                         (KERNEL, "WRITE_SIZE", 30), (OTHER, "WRITE_SIZE", 7)])
    per_xcd = 1000.0
    gui = per_xcd * profiling.XCD_NUM
    _write_counters(tmp_path / "mfma", [(KERNEL, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * per_xcd * profiling.SIMD_NUM),
                                        (KERNEL, "GRBM_GUI_ACTIVE", gui),
                                        (KERNEL, "SQ_INSTS_VALU_MFMA_MOPS_I8", 4e8),
                                        (KERNEL, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0)])
    issue = {"SQ_INSTS_VALU": 1024000, "SQ_INSTS_MFMA": 256000, "SQ_INSTS_LDS": 100, "SQ_LDS_BANK_CONFLICT": 50,
             "SQ_WAVE_CYCLES": 1000, "SQ_WAIT_ANY": 300, "SQ_BUSY_CYCLES": 1, "GRBM_GUI_ACTIVE": gui}
    assert set(issue) == set(profiling.ISSUE_COUNTERS)
    _write_counters(tmp_path / "issue", [(KERNEL, c, v) for c, v in issue.items()])
    out = tmp_path / "prof" / "summary"
    argv = ["profiling", "--stats", str(st), "--fetch", str(tmp_path / "fetch"), "--write", str(tmp_path / "write"),
            "--mfma", str(tmp_path / "mfma"), "--issue", str(tmp_path / "issue"),
            "--role", r"gate_up=k_gemm_pf<\(q4::Act\)2, 1, false, false, 1>", "--live", "gate_up=0.125",
            "--workload", "synthetic", "--commands", "cmd", "--out", str(out)]
    monkeypatch.setattr(sys, "argv", argv)
    profiling.main()
    return profiling.read_kv(str(out) + ".txt"), open(str(out) + ".md").read()


def test_hbm_bytes_are_copy_calibrated(summary):
    kv, _ = summary
    assert float(kv["fetch_scale"]) == pytest.approx(2.0) and float(kv["write_scale"]) == pytest.approx(1.0)
    assert int(kv["read_bytes[gate_up]"]) == 2000 * 1024 * 2       # mean FETCH_SIZE 2000 KiB x 2
    assert int(kv["write_bytes[gate_up]"]) == 20 * 1024
    assert int(kv["traffic_bytes[gate_up]"]) == 2000 * 1024 * 2 + 20 * 1024
    assert kv["kernel[gate_up]"] == KERNEL
    assert kv["source_hash"] == profiling.source_hash()


def test_trace_live_and_matrix_core_figures(summary):
    kv, md = summary
    assert float(kv["avg_us[gate_up]"]) == pytest.approx(100.0)
    assert float(kv["live_avg_us[gate_up]"]) == pytest.approx(125.0)
    assert float(kv["mfma_busy_pct[gate_up]"]) == pytest.approx(25.0)
    ops = 4e8 * profiling.MOPS_UNIT   # over the 100 us trace average: 2.048e15 op/s, 0.4096 of the INT8 peak
    assert float(kv["mfma_ops[gate_up]"]) == pytest.approx(ops)
    assert float(kv["mfma_frac_counter[gate_up]"]) == pytest.approx(0.4096, abs=1e-4)
    assert "| gate_up | 100.00 | 125.00 | 0.8000 |" in md


def test_issue_counters(summary):
    kv, _ = summary
    assert float(kv["valu_per_mfma[gate_up]"]) == pytest.approx(4.0)
    # 1024000 VALU instructions x 4 cycles over 1000 cycles x 1024 SIMDs
    assert float(kv["valu_issue_pct[gate_up]"]) == pytest.approx(400.0, rel=1e-3)
    assert float(kv["wait_pct[gate_up]"]) == pytest.approx(30.0)
    assert float(kv["lds_conflict_per_inst[gate_up]"]) == pytest.approx(0.5)


def test_read_kv_missing_file(tmp_path):
    assert profiling.read_kv(str(tmp_path / "nothing.txt")) == {}
