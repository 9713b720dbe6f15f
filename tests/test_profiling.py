"""rocprofv3 summaries: counter scaling by the calibration copy, and traffic
figures that disappear once the measured kernel source changes (CPU only)."""
import csv

from sparse_mixture_experts_48_amd import profiling

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, value in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_scaled_by_copy_and_tied_to_source(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    gemm = "void moe::(anonymous namespace)::gemm_tile_kernel<256, 256, 4, 2, 0>(moe::GemmParams)"
    # 1 MiB copy: fetch counts in 64-byte units here (two rows per dispatch, summed), write in KiB
    _counters(tmp_path / "f.csv", "FETCH_SIZE", [(1, copy, 8192), (1, copy, 8192), (2, gemm, 100), (3, gemm, 300)])
    _counters(tmp_path / "w.csv", "WRITE_SIZE", [(1, copy, 1024), (2, gemm, 10), (3, gemm, 30)])
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    md = profiling.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1,
                                     {"gemm1": r"gemm_tile_kernel<256, 256, 4, 2, 0>"}, str(src), "w",
                                     "rocprofv3 ...", str(tmp_path))
    out = tmp_path / "hbm.md"
    out.write_text(md)
    # fetch: 1 MiB / 16384 units = 64 B per unit -> mean 200 units = 12800 B; write: 1024 B per unit -> 20480 B
    assert profiling.traffic_bytes(str(out), "gemm1", str(tmp_path)) == 12800 + 20480
    assert profiling.traffic_bytes(str(out), "gemm2", str(tmp_path)) is None
    src.write_text("kernel v2\n")
    assert profiling.traffic_bytes(str(out), "gemm1", str(tmp_path)) is None
    assert profiling.traffic_bytes(str(tmp_path / "missing.md"), "gemm1", str(tmp_path)) is None


def test_short_kernel_names():
    assert profiling.short_name(
        "void moe::(anonymous namespace)::gemm_tile_kernel<256, 256, 4, 2, 0>(moe::(anonymous namespace)::GemmParams)"
    ) == "gemm_tile_kernel<256, 256, 4, 2, 0>"
    assert profiling.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_trace_medians(tmp_path):
    """The median column comes from the per-dispatch trace (odd and even
    counts), beside the stats file's mean."""
    import csv as _csv
    stats = tmp_path / "s.csv"
    trace = tmp_path / "t.csv"
    with open(stats, "w", newline="") as f:
        w = _csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
        w.writerow(["void k_a(int)", 3, 700, 233.3, 100, 500])
        w.writerow(["void k_b(int)", 2, 300, 150, 100, 200])
    with open(trace, "w", newline="") as f:
        w = _csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for name, dur in (("void k_a(int)", 500), ("void k_a(int)", 100), ("void k_a(int)", 100),
                          ("void k_b(int)", 100), ("void k_b(int)", 200)):
            w.writerow([name, 1000, 1000 + dur])
    med = profiling.dispatch_medians(str(trace))
    assert med == {"void k_a(int)": 100, "void k_b(int)": 150.0}
    md = profiling.summarize_trace(str(stats), "cmd", "T", str(trace))
    assert "| `k_a` | 3 | 0.2 | 0.1 | 0.1 | 0.5 | 70.0 % |" in md


def test_counter_summary(tmp_path):
    """Per-launch means over dispatches, rows of one dispatch summed, the clock
    of two passes averaged, and the derived shares from their definitions."""
    gemm = "void moe::(anonymous namespace)::gemm_tile_kernel<256, 256, 4, 2, 0>(moe::GemmParams)"
    other = "void moe::(anonymous namespace)::combine_kernel<unsigned short>(moe::CombineParams)"
    a, b = tmp_path / "a.csv", tmp_path / "b.csv"
    with open(a, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, busy in ((5, 400_000), (6, 600_000)):
            # GRBM_GUI_ACTIVE reported per XCD (summed: 8 x 1000 clocks)
            for _ in range(8):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": gemm, "Counter_Name": "GRBM_GUI_ACTIVE",
                            "Counter_Value": 1000})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": gemm, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
                        "Counter_Value": busy})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": gemm, "Counter_Name": "SQ_INSTS_LDS_LOAD_BANDWIDTH",
                        "Counter_Value": 16_000})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": gemm, "Counter_Name": "SQ_WAVE_CYCLES", "Counter_Value": 200})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": gemm, "Counter_Name": "SQ_WAIT_ANY", "Counter_Value": 50})
        w.writerow({"Dispatch_Id": 7, "Kernel_Name": other, "Counter_Name": "SQ_WAVE_CYCLES", "Counter_Value": 1})
    with open(b, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        w.writerow({"Dispatch_Id": 9, "Kernel_Name": gemm, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 24_000})
    md = profiling.summarize_counters([str(a), str(b)], {"gemm1": r"gemm_tile_kernel<256, 256, 4, 2, 0>"}, "w", "cmd")
    # clock: pass A 8000, pass B 24000 per launch -> 16000, i.e. 2000 cycles per XCD
    assert "| GRBM_GUI_ACTIVE | 1.6e+04 | 1 |" in md
    assert "| SQ_VALU_MFMA_BUSY_CYCLES | 5e+05 | 2 |" in md
    d = profiling.derived_counters({"GRBM_GUI_ACTIVE": 16_000, "SQ_VALU_MFMA_BUSY_CYCLES": 500_000,
                                    "SQ_INSTS_LDS_LOAD_BANDWIDTH": 16_000, "SQ_WAVE_CYCLES": 200, "SQ_WAIT_ANY": 50})
    assert d["clock cycles (GRBM_GUI_ACTIVE / 8)"] == 2000
    assert abs(d["MFMA busy share (per SIMD)"] - 500_000 / 1024 / 2000) < 1e-12
    assert abs(d["LDS bytes read per CU per clock"] - 16_000 * 64 / 256 / 2000) < 1e-12
    assert d["SQ_WAIT_ANY / SQ_WAVE_CYCLES"] == 0.25
    assert "combine" not in md
