"""Host logic of the measurement: the rocprofv3 summaries bench.py writes
into profiles/ and reads back into its JSON line, checked on small synthetic
counter files (no GPU).

  * HBM traffic: each counter is scaled by what it reads for the plain copy
    of known size in the same run, and the GEMM launch is the largest grid
    of the plain [K, N] GEMM kernel;
  * the decode summary picks the product and merge dispatches by name and
    grid, and reports bytes over time;
  * the matrix-unit summary recovers the per-XCD active cycles from the
    derived MfmaUtil, and the clock from them and the duration;
  * a summary is used only while the hash of the kernels' code (comments
    left out) matches; comment edits keep it, code edits drop it.
"""
import csv
import re

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, rows):
    """rows: (dispatch, kernel name, grid, counter, value, start_ns, end_ns)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for d, name, grid, counter, value, t0, t1 in rows:
            w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Agent_Id": "Agent 1", "Queue_Id": 1,
                        "Process_Id": 1, "Thread_Id": 1, "Grid_Size": grid, "Kernel_Id": 1, "Kernel_Name": name,
                        "Workgroup_Size": 256, "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 0,
                        "Accum_VGPR_Count": 0, "SGPR_Count": 0, "Counter_Name": counter,
                        "Counter_Value": f"{value:.6f}", "Start_Timestamp": t0, "End_Timestamp": t1})


GEMM = "void cfp32::(anonymous namespace)::" + bench.GEMM_KERNEL + "(cfp32::DmaArgs)"
COPY = "__amd_rocclr_copyBuffer"
CALIB_KIB = bench.CALIB_BYTES / 1024
FETCH_SKEW = 1.0001               # the copy's FETCH reads a hair above half, as measured
FETCH_SCALE = 2 / FETCH_SKEW


def traffic_files(tmp_path):
    """FETCH counts half of the copied bytes, WRITE all of them (as measured);
    the big GEMM is launched twice, a smaller one once (ignored)."""
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    write_csv(fetch, [(1, COPY, 131072, "FETCH_SIZE", CALIB_KIB / 2 * FETCH_SKEW, 0, 100),
                      (2, GEMM, 1835008, "FETCH_SIZE", 1.0e6, 0, 1500),
                      (3, GEMM, 1835008, "FETCH_SIZE", 2.0e6, 0, 1500),
                      (4, GEMM, 262144, "FETCH_SIZE", 9.0e9, 0, 200),
                      (5, "gemv_valu_kernel<1>(GemvArgs)", 229376, "FETCH_SIZE", 57344.0, 0, 20000),
                      (6, "gemv_merge_kernel<64>(float const*)", bench.GEMV_GRID, "FETCH_SIZE", 512.0, 0, 4000)])
    write_csv(write, [(1, COPY, 131072, "WRITE_SIZE", CALIB_KIB, 0, 100),
                      (2, GEMM, 1835008, "WRITE_SIZE", 4.0e5, 0, 1500),
                      (3, GEMM, 1835008, "WRITE_SIZE", 6.0e5, 0, 1500),
                      (5, "gemv_valu_kernel<1>(GemvArgs)", 229376, "WRITE_SIZE", 896.0, 0, 20000),
                      (6, "gemv_merge_kernel<64>(float const*)", bench.GEMV_GRID, "WRITE_SIZE", 56.0, 0, 4000)])
    return fetch, write


def value(text, key):
    m = re.search(rf"^{re.escape(key)}:\s*([0-9.eE+-]+)", text, re.M)
    assert m, key
    return float(m.group(1))


def test_gemm_traffic_is_scaled_by_the_copy(tmp_path):
    fetch, write = traffic_files(tmp_path)
    out = tmp_path / "gemm.txt"
    bench.summarize_counters(str(fetch), str(write), str(out), "cmd")
    text = out.read_text()
    # mean of the two big launches, FETCH doubled (the copy read half), WRITE as is
    assert value(text, "FETCH_SIZE_gemm_bytes_per_launch") == pytest.approx(1.5e6 * 1024 * FETCH_SCALE, rel=1e-4)
    assert value(text, "WRITE_SIZE_gemm_bytes_per_launch") == pytest.approx(5.0e5 * 1024, rel=1e-4)
    total = 1.5e6 * 1024 * FETCH_SCALE + 5.0e5 * 1024
    assert value(text, "hbm_bytes_per_launch") == pytest.approx(total, rel=1e-4)
    assert f"kernel_source_hash: {bench.kernel_source_hash()}" in text


def test_decode_traffic_and_rate(tmp_path):
    fetch, write = traffic_files(tmp_path)
    out = tmp_path / "gemv.txt"
    bench.summarize_gemv_counters(str(fetch), str(write), str(out), "cmd")
    text = out.read_text()
    read = 57344.0 * 1024 * FETCH_SCALE
    written = 896.0 * 1024
    assert value(text, "product_hbm_bytes_per_dispatch") == pytest.approx(read + written, rel=1e-4)
    assert value(text, "product_read_over_algorithmic") == pytest.approx(read / (4096 * 14336 * 2 + 4096 * 4),
                                                                         abs=1e-4)
    assert value(text, "product_duration_us_under_counters") == pytest.approx(20.0)
    assert value(text, "product_hbm_GBps") == pytest.approx((read + written) / 20e-6 / 1e9, rel=1e-3)


def test_mfma_clock_from_active_cycles(tmp_path):
    """Busy cycles summed over the 1024 SIMDs, MfmaUtil = busy / (active *
    1024): the summary recovers the active cycles of one XCD and, over the
    duration, the clock."""
    path = tmp_path / "mfma.csv"
    rows = []
    for (M, K, N), grid in ((mkn, g) for g, mkn in bench.GEMM_GRIDS.items()):
        dur_ns = 1000.0                      # 1 us
        active = 1.7e3                       # 1.7 GHz over 1 us, per XCD
        util = 70.0
        busy = util / 100 * active * 1024
        flops_ops = 4.0 * M * N * K / 512
        for d in (1, 2):
            for counter, v in (("MfmaUtil", util), ("SQ_VALU_MFMA_BUSY_CYCLES", busy),
                               ("SQ_INSTS_VALU_MFMA_MOPS_F16", flops_ops), ("GRBM_GUI_ACTIVE", active * 8)):
                rows.append((f"{grid}{d}", GEMM, grid, counter, v, 0, int(dur_ns)))
    write_csv(path, rows)
    out = tmp_path / "mfma.txt"
    bench.summarize_mfma(str(path), str(out), "cmd")
    text = out.read_text()
    assert value(text, "gemm_8192x4096x14336_MfmaUtil_percent") == pytest.approx(70.0)
    assert value(text, "gemm_8192x4096x14336_clock_GHz") == pytest.approx(1.7, abs=1e-3)
    assert "ratio 1.0000" in text


def test_summaries_follow_the_kernel_code_not_its_comments(tmp_path, monkeypatch):
    """A summary is read back only while the recorded hash matches the code;
    the hash ignores comments and blank space."""
    csrc = tmp_path / "compensated_fp32_projection_amd" / "csrc"
    csrc.mkdir(parents=True)
    names = ("gemm_dma.hip", "gemm.hip", "tile_order.h", "device_common.h")
    for n in names:
        (csrc / n).write_text(f"// {n}\nint f_{n.split('.')[0]}() {{ return 1; }}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "gemm.hip").write_text("/* a new\n   comment */\n// another\nint f_gemm()   {  return 1; }\n\n")
    assert bench.kernel_source_hash() == h0
    summary = tmp_path / "summary.txt"
    summary.write_text(f"kernel_source_hash: {h0}\nhbm_bytes_per_launch: 1.5e9\n")
    monkeypatch.setattr(bench, "COUNTER_SUMMARY", str(summary))
    assert bench.measured_traffic() == pytest.approx(1.5e9)
    (csrc / "gemm.hip").write_text("int f_gemm() { return 2; }\n")
    assert bench.kernel_source_hash() != h0
    assert bench.measured_traffic() is None
