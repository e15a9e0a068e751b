"""Host checks of the rocprofv3 summarizer (synthetic CSV files, no GPU)."""

import csv
import json

from matrix_optimizer_step_owner_amd import profiling

UPD = ("void mfsdp::ns_gemm_kernel<mfsdp::ElemBF16, 2>(mfsdp::MatDesc const*, "
       "HIP_vector_type<int, 2u> const*, float const*, mfsdp::NsEpi)")
COPY = "__amd_rocclr_copyBuffer"


def _pmc(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, v) in enumerate(rows):
            w.writerow([i, k, counter, v])


def test_short_names():
    assert profiling.short_name(UPD) == "update"
    assert profiling.short_name(UPD.replace("ElemBF16, 2", "ElemF32, 0")) == "gram_f32"
    assert profiling.short_name("mfsdp::adamw_kernel(float*)") == "adamw"
    assert profiling.short_name("void mfsdp::adamw_kernel<4, true>(float*)") == "adamw"
    assert profiling.short_name(UPD.replace("ElemBF16, 2", "ElemBF16, 5")) == "syrk"
    assert profiling.short_name(UPD.replace("ElemBF16, 2", "ElemBF16, 4")) == "final_tall"
    assert profiling.short_name(COPY) == ""


def test_traffic_is_calibrated_by_the_copy(tmp_path):
    mib = 64
    # the counter reads half of the copied bytes (KiB units) -> factor 0.5
    _pmc(tmp_path / "f.csv", "FETCH_SIZE", [(COPY, mib * 1024 * 0.5), (UPD, 1000.0), (UPD, 3000.0)])
    _pmc(tmp_path / "w.csv", "WRITE_SIZE", [(COPY, mib * 1024), (UPD, 500.0), (UPD, 500.0)])
    tr = profiling.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), mib << 20, "update")
    assert abs(tr["FETCH_SIZE"]["factor"] - 0.5) < 1e-12
    assert abs(tr["FETCH_SIZE"]["bytes_per_launch"] - 2000.0 * 1024 / 0.5) < 1e-6
    assert abs(tr["WRITE_SIZE"]["bytes_per_launch"] - 500.0 * 1024) < 1e-6


def test_stats_summary_and_cli(tmp_path):
    p = tmp_path / "kt_kernel_stats.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow([UPD, 4, 900000, 225000, 60.0, 220000, 230000, 1.0])
    out = tmp_path / "s.txt"
    profiling.main(["stats", str(p), "--command", "bench", "--out", str(out)])
    text = out.read_text()
    assert "update" in text and "225.00" in text and "bench" in text
    _pmc(tmp_path / "f.csv", "FETCH_SIZE", [(COPY, 1024.0), (UPD, 10.0)])
    _pmc(tmp_path / "w.csv", "WRITE_SIZE", [(COPY, 1024.0), (UPD, 5.0)])
    tj = tmp_path / "t.json"
    profiling.main(["traffic", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "--calib-mib", "1",
                    "--kernel", "update", "--workload", "w", "--command", "c", "--out", str(tj)])
    doc = json.loads(tj.read_text())
    assert doc["bytes_per_launch"] == 15.0 * 1024
    assert doc["source_sha256"] == profiling.kernel_source_hash("update")
    assert profiling.kernel_source_hash("update") == profiling.kernel_source_hash("gram")
    assert profiling.kernel_source_hash("update") != profiling.kernel_source_hash("momentum")


def test_counter_table_derived_columns(tmp_path):
    """Clock, MFMA busy, executed flops and calibrated bytes from known counts."""
    p = tmp_path / "c.csv"
    dur_ns = 200_000  # 200 us
    ghz = 2.0
    cyc = ghz * 1e9 * dur_ns * 1e-9
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for i in range(2):
            t0 = 1_000_000 * (i + 1)
            # GRBM_GUI_ACTIVE summed over the 8 XCDs; MFMA busy on half of all SIMD-cycles
            rows = [("GRBM_GUI_ACTIVE", cyc * profiling.N_XCD),
                    ("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * profiling.N_SIMD),
                    ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e15 * dur_ns * 1e-9 / 512),  # 1 PFLOP/s
                    ("FETCH_SIZE", 0.5 * 1000.0)]   # KiB, counter reads half the bytes
            for name, v in rows:
                w.writerow([i, UPD, name, v, t0, t0 + dur_ns])
        w.writerow([9, COPY, "FETCH_SIZE", 0.5 * 1024, 0, 100])
    cal = profiling.calibration([str(p)], 1 << 20)
    assert abs(cal["FETCH_SIZE"] - 0.5) < 1e-12
    rows = {r["kind"]: r for r in profiling.counter_table([str(p)], cal)}
    u = rows["update"]
    assert u["dispatches"] == 2 and abs(u["avg_us"] - 200.0) < 1e-9
    assert abs(u["sclk_ghz"] - ghz) < 1e-9
    assert abs(u["mfma_busy_pct"] - 50.0) < 1e-9
    assert abs(u["mfma_tflops"] - 1000.0) < 1e-6
    assert abs(u["fetch_size_mb"] - 1000.0 * 1024 / 1e6) < 1e-9
    # short kernels get no GRBM-derived columns
    assert "sclk_ghz" not in rows["copy"]
    out = tmp_path / "c.txt"
    profiling.main(["counters", str(p), "--calib-mib", "1", "--command", "x", "--out", str(out)])
    assert "update" in out.read_text()
