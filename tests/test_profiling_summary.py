"""The rocprofv3 summariser on the host, with small counter files written
here: per-launch traffic of the named kernel, calibrated by the read probe
(FETCH_SIZE) and by the run's last copy kernel (WRITE_SIZE), and the
matrix-core busy fraction with GRBM_GUI_ACTIVE summed over the 8 XCDs."""

import csv
import json

from sparse_expert_execution_amd import profiling


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i, k, c, v])


def test_summary_traffic_and_mfma(tmp_path):
    stats = tmp_path / "stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs",
                    "Percentage"])
        w.writerow(["gemm_wide_kernel<1>(args)", 2, 2000, 1000, 900, 1100, 90.0])
    probe_kib = profiling.PROBE_BYTES / 1024 / 2       # counter reads half the bytes
    _counters(tmp_path / "fetch.csv", [
        ("gemm_wide_kernel<1>(args)", "FETCH_SIZE", 1000.0),
        ("gemm_wide_kernel<1>(args)", "FETCH_SIZE", 3000.0),
        ("read_probe_kernel<8>", "FETCH_SIZE", probe_kib)])
    _counters(tmp_path / "write.csv", [
        ("vectorized_elementwise_kernel<FillFunctor>", "WRITE_SIZE", 999999.0),
        ("gemm_wide_kernel<1>(args)", "WRITE_SIZE", 10.0),
        ("gemm_wide_kernel<1>(args)", "WRITE_SIZE", 30.0),
        ("__amd_rocclr_copyBuffer", "WRITE_SIZE", profiling.COPY_BYTES / 1024)])
    _counters(tmp_path / "mfma.csv", [
        ("gemm_wide_kernel<1>(args)", "SQ_INSTS_VALU_MFMA_MOPS_F6F4", 1e9),
        ("gemm_wide_kernel<1>(args)", "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 250.0),
        ("gemm_wide_kernel<1>(args)", "GRBM_GUI_ACTIVE", 8 * 1000.0)])
    profiling.main(["summarize", "--name", "t", "--stats", str(stats),
                    "--fetch", str(tmp_path / "fetch.csv"), "--write", str(tmp_path / "write.csv"),
                    "--kernel", "gemm_wide_kernel<1", "--alg-bytes", "1",
                    "--mfma", str(tmp_path / "mfma.csv"), "--out-dir", str(tmp_path)])
    rec = json.load(open(tmp_path / "t.traffic.json"))
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12
    assert rec["write_scale"] == 1.0                   # the last copy, not the big fill
    assert abs(rec["fetch_bytes_per_launch"] - 2000.0 * 1024 * 2.0) < 1e-6
    assert abs(rec["write_bytes_per_launch"] - 20.0 * 1024) < 1e-6
    md = open(tmp_path / "t.md").read()
    assert "| 0.512 | 25.0% |" in md                   # 1e9 x 512 FLOP; 250 / 1000 busy
