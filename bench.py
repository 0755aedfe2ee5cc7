#!/usr/bin/env python3
"""Benchmark of the compensated-FP32 projection on one MI355X.

A step is one pass of the whole path over the decode + FFN projection pair
that shares one FP16 weight W [4096, 14336]:

  1. decode:  y1 = x1 W,  x1 FP32 [1, 4096]      -> cfp32_linear (small-M path:
              K-chunked product dispatch + merge dispatch)
  2. prefill: split(x2) then the dual-product GEMM with the merged epilogue,
              x2 FP32 [8192, 4096]                -> cfp32_split + cfp32_gemm
              (exactly the two launches cfp32_linear makes for M > 8)

Inputs are seeded synthetic data (compensated_fp32_projection_amd.workloads)
already resident in HBM.  Four copies of W (470 MB, more than the 256 MB
Infinity Cache) are rotated step by step so that the decode kernel streams W
from HBM.  ``value`` is whole-step throughput in FP32-equivalent TFLOP/s
(2 M N K summed over both projections).  HIP events recorded on the launch
stream inside the timed loop give each kernel's average duration; the MFMA
roofline is taken for the GEMM, the dominant kernel.

One JSON line is printed.  Extra keys: ``breakdown`` (per kernel),
``headline`` (the 4096^3 GEMM, the M = 1 decode path in both weight
layouts and captured in a graph, batched decode at M = 16 and 64, and the
FFN projection with [N, K] weights next to the [K, N] split + GEMM, each
measured on its own), ``fp32_ab_4096`` (the whole compensated projection at 4096^3 next to
the FP32 library GEMM, torch.matmul with TF32 off, on the same operands),
``geglu_ffn_8192x4096x7168`` (the FFN projection with its GEGLU fused,
next to the plain projection of the same operands),
``separate_add_4096`` (the separate-addition accumulation mode at 4096^3,
k_per_add 0 = plain accumulation in the same kernel configuration),
``configs`` (each of the five workloads through cfp32_linear on its own:
microseconds per call, kernel launches per call counted from a captured HIP
graph, rates and roofline fractions, the normalised errors of y and of the
single-FP16 product C_hi, the CPU oracle's median of 3 runs for the small
workloads and the decode, and the FP16 library GEMM for context),
``host`` (CPU model and cores, git revision and hashes of the sources and
library from the build), ``roofline``, ``rocprof_mfma`` (the GEMM's matrix-unit utilisation and
shader clock as rocprofv3 counters measured them, from the committed summary
while the GEMM source is unchanged) and ``cpu_baseline`` (the CPU oracle
timed on a bounded sample of the same workload on this host).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compensated-FP32 GEMM TFLOP/s + % FP16 MFMA peak; GEMV GB/s % HBM"
# MI355X published peaks: dense FP16 MFMA 2.5 PFLOP/s (256 CUs x 4096 FLOP/clk
# x 2.4 GHz = 2516.6 TFLOP/s) and HBM3E 8 TB/s.
PEAK_FP16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0
K_, N_, M_DEC, M_PRE = 4096, 14336, 1, 8192
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "gemm_prefill_8192x4096x14336_counters.txt")
CALIB_BYTES = 512 * 1024 * 1024  # plain device copy of known size, for counter scaling
GEMM_KERNEL = "gemm_dma_kernel<false, false, false, false, false>"  # the plain [K, N] variant
COPY_KERNEL_HINT = "copy"


def _code_hash(names) -> str:
    """Hash of the code in these csrc files, comments and blank space left
    out, so that a measured summary stays valid across comment edits."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "compensated_fp32_projection_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    return _code_hash(("gemm_dma.hip", "gemm.hip", "tile_order.h", "device_common.h"))


def measured_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when there is none or the GEMM source has changed since."""
    try:
        text = open(COUNTER_SUMMARY).read()
    except OSError:
        return None
    src = re.search(r"^kernel_source_hash:\s*(\S+)", text, re.M)
    val = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def cpu_baseline(A1, A2, W, rows_per_thread: int):
    """Time the CPU oracle's compensated linear (split, two FP32-accumulated
    products, merge) on the decode row plus a slice of the prefill rows."""
    import numpy as np
    import oracle
    threads = oracle.num_threads()
    rows = max(1, rows_per_thread * threads)
    A = np.concatenate([A1, A2[:rows]], axis=0)
    t0 = time.perf_counter()
    oracle.linear_cf32(A, W)
    dt = time.perf_counter() - t0
    flops = 2.0 * A.shape[0] * K_ * N_
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": dt,
            "sample": f"1 decode row + {rows} of the 8192 prefill rows, K=4096, N=14336 "
                      f"(split + two FP32-accumulated products + merge, OpenMP over rows)"}


def host_info():
    """CPU model and usable cores, and the build the library came from."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    info = {"cpu_model": model, "cpu_cores_usable": len(os.sched_getaffinity(0))}
    lib_dir = os.path.join(ROOT, "compensated_fp32_projection_amd")
    try:
        with open(os.path.join(lib_dir, "build_info.json")) as f:
            info["build"] = json.load(f)
    except (OSError, ValueError):
        info["build"] = None
    h = hashlib.sha256()
    with open(os.path.join(lib_dir, "libcfp32.so"), "rb") as f:
        h.update(f.read())
    info["library_sha256"] = h.hexdigest()
    return info


def graph_launches(fn):
    """Kernel launches one call makes: the call is captured into a HIP graph
    and the graph's kernel nodes are counted (None if that fails)."""
    import ctypes
    import torch
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
        g = torch.cuda.CUDAGraph(keep_graph=True)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                fn(s.cuda_stream)
        torch.cuda.synchronize()
        raw = ctypes.c_void_p(g.raw_cuda_graph())
        n = ctypes.c_size_t(0)
        if hip.hipGraphGetNodes(raw, None, ctypes.byref(n)) != 0:
            return None
        nodes = (ctypes.c_void_p * n.value)()
        if hip.hipGraphGetNodes(raw, nodes, ctypes.byref(n)) != 0:
            return None
        kernels = 0
        for i in range(n.value):
            t = ctypes.c_int(-1)
            if hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) != 0:
                return None
            kernels += int(t.value == 0)  # hipGraphNodeTypeKernel
        del g
        return kernels
    except Exception:
        return None


def timed_median(fn, stream, reps=9, min_ms=1.0):
    """Median microseconds per call over `reps` repetitions, each a loop of n
    calls with n chosen so that a repetition takes at least min_ms (HIP
    events on the launch stream)."""
    import torch
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    n = 1
    while True:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        b.synchronize()
        if a.elapsed_time(b) >= min_ms or n >= 1 << 14:
            break
        n *= 2
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b) / n * 1e3)
    times.sort()
    return times[len(times) // 2]


def _cpu_median(A, W, runs):
    """Median seconds of the oracle's compensated linear (split, two FP32
    sums, merge) on A, W."""
    import numpy as np
    import oracle
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.linear_cf32(A, W)
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def _rel_err(y, y64, abs64):
    import numpy as np
    e = np.abs(np.asarray(y, np.float64) - y64) / np.where(abs64 > 0, abs64, 1.0)
    return float(e.max()), float(np.sqrt(np.mean(e * e)))


def measure_configs(stream, with_cpu: bool, only=None):
    """Each workload through cfp32_linear on its own: microseconds per call
    (median of timed loops of at least 1 ms), kernel launches per call,
    FP32-equivalent TFLOP/s with the FP16-MFMA fraction (both products) or
    GB/s with the HBM fraction (the M = 1 decode, W rotated over four copies
    so it streams from HBM), the normalised errors of y and of the
    single-FP16 product C_hi of the same split (the GEMM's own C_hi; the
    oracle's for the decode, whose kernels do not expose it), the CPU
    oracle's median of 3 runs (configs 1-3 and 5a; one run for config 4),
    the FP64 reference's time (for information), the SHA-256 of the input
    arrays (the same bytes the oracle and the GPU receive) and the FP16
    library GEMM (torch.matmul on FP16 x, one product, context only).
    `only`: the workload ids to measure (e.g. {"2", "5a"}), or None for all."""
    import numpy as np
    import torch

    import compensated_fp32_projection_amd as cf
    import oracle
    from compensated_fp32_projection_amd import workloads
    dev = torch.device("cuda", 0)
    sh = stream.cuda_stream
    pair = workloads.decode_ffn_pair()
    cases = [("1_single_linear", workloads.single_linear().A[0], workloads.single_linear().W),
             ("2_qkv_projection", workloads.qkv_projection().A[0], workloads.qkv_projection().W),
             ("3_unaligned", workloads.unaligned().A[0], workloads.unaligned().W),
             ("4_square", workloads.square().A[0], workloads.square().W),
             ("5a_decode", pair.A[0], pair.W),
             ("5b_ffn_prefill", pair.A[1], pair.W)]
    del pair
    if only is not None:
        cases = [c for c in cases if c[0].split("_")[0] in only]
    out = {}
    threads = oracle.num_threads()
    for name, A, W in cases:
        M, K = A.shape
        N = W.shape[1]
        x = torch.from_numpy(A).to(dev)
        Ws = [torch.from_numpy(W.view(np.int16)).to(dev)]
        if M == 1:  # the decode streams W from HBM: rotate copies past the 256 MB cache
            Ws += [Ws[0].clone() for _ in range(3)]
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        need = cf.cfp32_linear_workspace_bytes(M, N, K)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def call(i, s=sh):
            st = cf.cfp32_linear(x.data_ptr(), K, Ws[i % len(Ws)].data_ptr(), N, y.data_ptr(), N, M, N, K,
                                 ws.data_ptr(), need, s)
            if st != cf.OK:
                raise RuntimeError(f"{name}: {cf.cfp32_status_string(st)}")

        us = timed_median(call, stream)
        entry = {"shape": f"{M}x{K}x{N}", "entry_point": "cfp32_linear",
                 "sha256_A": hashlib.sha256(np.ascontiguousarray(A).tobytes()).hexdigest()[:16],
                 "sha256_W": hashlib.sha256(np.ascontiguousarray(W).tobytes()).hexdigest()[:16],
                 "us": round(us, 2),
                 "launches": graph_launches(lambda s: call(0, s)),
                 "tflops_fp32eq": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 2),
                 "frac_fp16_peak": round(4.0 * M * N * K / (us * 1e-6) / 1e12 / PEAK_FP16_TFLOPS, 4)}
        if M == 1:
            bytes_ = K * N * 2 + M * K * 4 + M * N * 4
            entry["GBps"] = round(bytes_ / (us * 1e-6) / 1e9, 1)
            entry["frac_hbm"] = round(bytes_ / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        if M * N * K <= 4096 ** 3:  # FP64 reference of everything but the 8192-row prefill
            call(0)
            yh = y.cpu().numpy()
            t0 = time.perf_counter()
            y64, abs64 = oracle.y64(A, W)
            entry["cpu_fp64_reference_us"] = round((time.perf_counter() - t0) * 1e6, 1)
            entry["e_max_y"], entry["e_rms_y"] = (float(f"{v:.3g}") for v in _rel_err(yh, y64, abs64))
            if M > 1:
                hi, lo = cf.split(x)
                _, ch, _ = cf.gemm(hi, lo, Ws[0], want_y=False, want_parts=True)
                c_hi = ch.cpu().numpy()
                del hi, lo, ch
            else:
                _, c_hi, _ = oracle.linear_cf32(A, W)
            entry["e_max_c_hi"], entry["e_rms_c_hi"] = (float(f"{v:.3g}") for v in _rel_err(c_hi, y64, abs64))
            del y64, abs64
        if with_cpu and M * N * K <= 4096 ** 3:
            runs = 3 if M * N * K <= 1000 * 1000 * 1000 else 1
            t = _cpu_median(A, W, runs)
            entry["cpu_oracle_median3_us" if runs == 3 else "cpu_oracle_once_us"] = round(t * 1e6, 1)
            entry["cpu_oracle_tflops_fp32eq"] = round(2.0 * M * N * K / t / 1e12, 5)
            entry["cpu_oracle_threads_busy"] = min(M, threads)
            if M == 1:
                entry["cpu_oracle_GBps"] = round((K * N * 2 + K * 4 + N * 4) / t / 1e9, 2)
        xh = x.half()
        wh = Ws[0].view(torch.float16)
        entry["fp16_library_matmul_us"] = round(timed_median(lambda i: torch.matmul(xh, wh), stream, reps=5), 2)
        out[name] = entry
        del x, Ws, y, ws, xh, wh
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def _read_counter_csv(path):
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Dispatch_Id"], r["Kernel_Name"], int(r.get("Grid_Size", 0) or 0))
            per.setdefault(key, {})
            per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return per


def summarize_counters(fetch_csv, write_csv, out_path, command):
    """Write the HBM-traffic summary of the GEMM from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for the plain copy of CALIB_BYTES in the same run."""
    lines = [f"# rocprofv3 counter summary: dual-product GEMM 8192x4096x14336 (decode/FFN prefill step)",
             f"# command: {command}",
             f"kernel_source_hash: {kernel_source_hash()}"]
    result = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = _read_counter_csv(path)
        # the prefill GEMM is the GEMM launch with the largest grid in the run
        sizes = [gs for (d, k, gs) in per if GEMM_KERNEL in k]
        gemm = [v[name] for (d, k, gs), v in per.items() if GEMM_KERNEL in k and name in v
                and sizes and gs == max(sizes)]
        copy = [v[name] for (d, k, gs), v in per.items() if COPY_KERNEL_HINT in k.lower() and name in v
                and v[name] * 1024 > CALIB_BYTES * 0.5]
        if not gemm or not copy:
            raise SystemExit(f"{path}: no {name} rows for the GEMM or the calibration copy")
        g = sum(gemm) / len(gemm)
        c = max(copy)
        # A device copy reads and writes CALIB_BYTES each.
        factor = CALIB_BYTES / (c * 1024.0)
        result[name] = g * 1024.0 * factor
        lines += [f"{name}_gemm_KiB_per_dispatch: {g:.1f}  (dispatches: {len(gemm)})",
                  f"{name}_copy_KiB: {c:.1f}  (copy of {CALIB_BYTES} bytes)",
                  f"{name}_scale_factor: {factor:.4f}",
                  f"{name}_gemm_bytes_per_launch: {result[name]:.4e}"]
    total = result["FETCH_SIZE"] + result["WRITE_SIZE"]
    alg = 8192 * 4096 * 2 * 2 + 4096 * 14336 * 2 + 8192 * 14336 * 4
    lines += [f"hbm_bytes_per_launch: {total:.4e}",
              f"algorithmic_bytes_per_launch: {alg:.4e}  (A_hi + A_lo + W + y)",
              f"traffic_over_algorithmic: {total / alg:.3f}"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


GEMV_SUMMARY = os.path.join(ROOT, "profiles", "decode_gemv_1x4096x14336_counters.txt")
GEMV_PRODUCT_KERNEL = "gemv_valu_kernel<1>"  # the M = 1 product dispatch
GEMV_MERGE_KERNEL = "gemv_merge_kernel<64>"  # the M = 1 merge dispatch
GEMV_GRID = 14336                            # its threads (one output each)


def gemv_source_hash() -> str:
    return _code_hash(("gemv.hip", "device_common.h"))


def summarize_gemv_counters(fetch_csv, write_csv, out_path, command):
    """Write the HBM-traffic summary of the M = 1 decode path (product and
    merge dispatches) from the same two rocprofv3 --pmc runs as the GEMM's,
    each counter scaled by what it reads for the plain copy of CALIB_BYTES;
    the rate uses the dispatch timestamps of those runs."""
    import csv
    lines = ["# rocprofv3 counter summary: decode projection 1x4096x14336 (small-M product + merge dispatches)",
             f"# command: {command}",
             f"kernel_source_hash: {gemv_source_hash()}"]
    result = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        prod, merge, copy = [], [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != name:
                    continue
                v = float(r["Counter_Value"])
                dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                k = r["Kernel_Name"]
                if GEMV_PRODUCT_KERNEL in k:
                    prod.append((v, dur))
                elif GEMV_MERGE_KERNEL in k and int(r.get("Grid_Size", 0) or 0) == GEMV_GRID:
                    merge.append((v, dur))
                elif COPY_KERNEL_HINT in k.lower() and v * 1024 > CALIB_BYTES * 0.5:
                    copy.append(v)
        if not prod or not merge or not copy:
            raise SystemExit(f"{path}: no {name} rows for the decode dispatches or the calibration copy")
        factor = CALIB_BYTES / (max(copy) * 1024.0)
        for tag, rows in (("product", prod), ("merge", merge)):
            kib = sum(v for v, _ in rows) / len(rows)
            us = sum(d for _, d in rows) / len(rows) / 1e3
            result[(tag, name)] = (kib * 1024.0 * factor, us)
            lines.append(f"{tag}_{name}_KiB_per_dispatch: {kib:.1f}  (dispatches: {len(rows)}, scale {factor:.4f})")
    alg = 4096 * 14336 * 2 + 4096 * 4
    pb = result[("product", "FETCH_SIZE")][0] + result[("product", "WRITE_SIZE")][0]
    pus = result[("product", "FETCH_SIZE")][1]
    lines += [f"product_hbm_bytes_per_dispatch: {pb:.4e}",
              f"product_read_over_algorithmic: {result[('product', 'FETCH_SIZE')][0] / alg:.4f}  (W + x = {alg} bytes)",
              f"product_duration_us_under_counters: {pus:.2f}",
              f"product_hbm_GBps: {pb / (pus * 1e-6) / 1e9:.1f}  "
              f"({100 * pb / (pus * 1e-6) / 1e9 / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f} GB/s)",
              f"merge_hbm_bytes_per_dispatch: "
              f"{result[('merge', 'FETCH_SIZE')][0] + result[('merge', 'WRITE_SIZE')][0]:.4e}",
              f"merge_duration_us_under_counters: {result[('merge', 'FETCH_SIZE')][1]:.2f}"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_gemv():
    """HBM figures of the M = 1 product dispatch from the committed rocprofv3
    summary, or None when there is none or the small-M source has changed."""
    try:
        text = open(GEMV_SUMMARY).read()
    except OSError:
        return None
    src = re.search(r"^kernel_source_hash:\s*(\S+)", text, re.M)
    if not src or src.group(1) != gemv_source_hash():
        return None
    out = {}
    for key, pat in (("hbm_bytes_per_dispatch", r"^product_hbm_bytes_per_dispatch:\s*([0-9.eE+]+)"),
                     ("read_over_algorithmic", r"^product_read_over_algorithmic:\s*([0-9.]+)"),
                     ("hbm_GBps", r"^product_hbm_GBps:\s*([0-9.]+)")):
        m = re.search(pat, text, re.M)
        if not m:
            return None
        out[key] = float(m.group(1))
    out["source"] = "profiles/decode_gemv_1x4096x14336_counters.txt (rocprofv3 FETCH_SIZE, WRITE_SIZE)"
    return out


MFMA_SUMMARY = os.path.join(ROOT, "profiles", "gemm_mfma_utilisation_counters.txt")
# grid sizes (threads) of the plain GEMM launches in a bench run -> (M, K, N)
GEMM_GRIDS = {1835008: (8192, 4096, 14336), 262144: (4096, 4096, 4096)}


def summarize_mfma(csv_path, out_path, command):
    """Write the matrix-unit summary of the GEMM launches from one rocprofv3
    --pmc run of MfmaUtil (rocprofv3's derived metric: the summed
    SQ_VALU_MFMA_BUSY_CYCLES over the largest per-XCD GRBM_GUI_ACTIVE times
    the SIMD count), SQ_INSTS_VALU_MFMA_MOPS_F16 (FP16 MFMA operations / 512)
    and GRBM_GUI_ACTIVE, with each dispatch's start and end timestamps.  The
    clock follows from the active cycles of one XCD over the duration."""
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if GEMM_KERNEL not in r["Kernel_Name"]:
                continue
            grid = int(r.get("Grid_Size", 0) or 0)
            if grid not in GEMM_GRIDS:
                continue
            d = per.setdefault((grid, r["Dispatch_Id"]), {"dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = ["# rocprofv3 counter summary: dual-product GEMM matrix-unit utilisation and clock, MI355X",
             f"# command: {command}",
             f"kernel_source_hash: {kernel_source_hash()}"]
    simds = 256 * 4
    for grid, (M, K, N) in GEMM_GRIDS.items():
        ds = [v for (g, _), v in per.items() if g == grid and "MfmaUtil" in v and "SQ_VALU_MFMA_BUSY_CYCLES" in v]
        if not ds:
            raise SystemExit(f"{csv_path}: no MfmaUtil rows for the {M}x{K}x{N} GEMM")
        n = len(ds)
        util = sum(v["MfmaUtil"] for v in ds) / n
        busy = sum(v["SQ_VALU_MFMA_BUSY_CYCLES"] for v in ds) / n
        dur_us = sum(v["dur_ns"] for v in ds) / n / 1e3
        # the largest per-XCD active-cycle count, recovered from the derived metric
        active = busy / (util / 100.0 * simds)
        clock = active / (dur_us * 1e3)
        flops = sum(v["SQ_INSTS_VALU_MFMA_MOPS_F16"] for v in ds) / n * 512
        alg = 4.0 * M * N * K
        rate = alg / (dur_us * 1e-6) / 1e12
        at_clock = 256 * 4096 * clock * 1e9 / 1e12
        tag = f"gemm_{M}x{K}x{N}"
        lines += [f"{tag}_dispatches: {n}",
                  f"{tag}_MfmaUtil_percent: {util:.2f}",
                  f"{tag}_mfma_busy_cycles_per_simd: {busy / simds:.4e}",
                  f"{tag}_active_cycles_per_xcd: {active:.4e}",
                  f"{tag}_duration_us_under_counters: {dur_us:.1f}",
                  f"{tag}_clock_GHz: {clock:.3f}",
                  f"{tag}_fp16_mfma_flops_counted: {flops:.4e}  (algorithmic 4MNK: {alg:.4e}, ratio {flops / alg:.4f})",
                  f"{tag}_TFLOPs: {rate:.1f}  ({100 * rate / PEAK_FP16_TFLOPS:.1f}% of the 2.4 GHz peak, "
                  f"{100 * rate / at_clock:.1f}% of the peak at {clock:.3f} GHz)"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_mfma():
    """MfmaUtil and clock of the 8192 x 4096 x 14336 GEMM from the committed
    rocprofv3 summary, or None when there is none or the GEMM source has
    changed since."""
    try:
        text = open(MFMA_SUMMARY).read()
    except OSError:
        return None
    src = re.search(r"^kernel_source_hash:\s*(\S+)", text, re.M)
    if not src or src.group(1) != kernel_source_hash():
        return None
    out = {}
    for key, pat in (("mfma_util", r"^gemm_8192x4096x14336_MfmaUtil_percent:\s*([0-9.]+)"),
                     ("clock_ghz", r"^gemm_8192x4096x14336_clock_GHz:\s*([0-9.]+)")):
        m = re.search(pat, text, re.M)
        if not m:
            return None
        out[key] = float(m.group(1))
    out["mfma_util"] = round(out["mfma_util"] / 100.0, 4)
    out["source"] = "profiles/gemm_mfma_utilisation_counters.txt (rocprofv3 MfmaUtil, GRBM_GUI_ACTIVE)"
    return out


def summarize_trace(trace_csv, out_path, command):
    """Write per-kernel, per-grid-size durations from a rocprofv3
    --kernel-trace run (its *_kernel_trace.csv): one line per distinct
    (kernel, grid size), so launches of one kernel at different shapes are
    not averaged together."""
    import csv
    groups = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            grid = "x".join(r.get(k, "") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z")) \
                if "Grid_Size_X" in r else r.get("Grid_Size", "")
            key = (r["Kernel_Name"], grid)
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault(key, []).append(dur)
    lines = [f"# rocprofv3 kernel-trace summary: decode/FFN step, MI355X",
             f"# command: {command}",
             f"kernel_source_hash: {kernel_source_hash()}",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  {'grid':>16}  kernel"]
    for (name, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) <= 90 else name[:87] + "..."
        lines.append(f"{len(d):6d} {sum(d)/len(d):10.2f} {min(d):10.2f} {max(d):10.2f}  {grid:>16}  {short}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows-per-thread", type=int, default=40)
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload table")
    ap.add_argument("--configs", default="all",
                    help="workloads of the per-workload table: comma-separated ids out of 1,2,3,4,5a,5b, or all")
    ap.add_argument("--calibration-copy", action="store_true",
                    help=f"also run one plain device copy of {CALIB_BYTES} bytes (counter scaling reference)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT"),
                    help="summarise two rocprofv3 --pmc runs (no GPU needed)")
    ap.add_argument("--summarize-gemv-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT"),
                    help="summarise the decode dispatches of the two rocprofv3 --pmc runs (no GPU needed)")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("MFMA_CSV", "OUT"),
                    help="summarise a rocprofv3 --pmc run of MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_F16 and "
                         "GRBM_GUI_ACTIVE (no GPU needed)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "OUT"),
                    help="summarise a rocprofv3 --kernel-trace run, its *_kernel_trace.csv (no GPU needed)")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summary")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.profile_command)
        return
    if args.summarize_gemv_counters:
        summarize_gemv_counters(*args.summarize_gemv_counters, args.profile_command)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.profile_command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.profile_command)
        return
    if args.configs != "all":
        unknown = set(args.configs.split(",")) - {"1", "2", "3", "4", "5a", "5b"}
        if unknown:
            ap.error(f"--configs: unknown workload ids {sorted(unknown)} (known: 1,2,3,4,5a,5b)")
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (no sharding or collectives); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import compensated_fp32_projection_amd as cf
    from compensated_fp32_projection_amd import workloads

    cf.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    wl = workloads.decode_ffn_pair()
    A1, A2, W = wl.A[0], wl.A[1], wl.W
    Ws = [torch.from_numpy(W.view(np.int16)).to(dev)]
    for _ in range(3):
        Ws.append(Ws[0].clone())
    x1 = torch.from_numpy(A1).to(dev)
    x2 = torch.from_numpy(A2).to(dev)
    y1 = torch.empty((M_DEC, N_), dtype=torch.float32, device=dev)
    y2 = torch.empty((M_PRE, N_), dtype=torch.float32, device=dev)
    dec_ws_bytes = cf.cfp32_linear_workspace_bytes(M_DEC, N_, K_)
    dec_ws = torch.empty(max(dec_ws_bytes, 1), dtype=torch.uint8, device=dev)
    hi = torch.empty((M_PRE, K_), dtype=torch.int16, device=dev)
    lo = torch.empty((M_PRE, K_), dtype=torch.int16, device=dev)

    def check(st, what):
        if st != cf.OK:
            raise RuntimeError(f"{what}: {cf.cfp32_status_string(st)}")

    def step(s, ev=None):
        w = Ws[s % len(Ws)].data_ptr()
        if ev: ev[0].record(stream)
        check(cf.cfp32_linear(x1.data_ptr(), K_, w, N_, y1.data_ptr(), N_, M_DEC, N_, K_,
                              dec_ws.data_ptr(), dec_ws_bytes, sh), "decode")
        if ev: ev[1].record(stream)
        check(cf.cfp32_split(x2.data_ptr(), K_, hi.data_ptr(), lo.data_ptr(), K_, M_PRE, K_, sh), "split")
        if ev: ev[2].record(stream)
        check(cf.cfp32_gemm(hi.data_ptr(), lo.data_ptr(), K_, w, N_, y2.data_ptr(), None, None, N_,
                            M_PRE, N_, K_, sh), "gemm")
        if ev: ev[3].record(stream)

    for s in range(args.warmup):
        step(s)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s, events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) / args.steps * 1e3

    def avg_us(i, j):
        return sum(e[i].elapsed_time(e[j]) for e in events) / len(events) * 1e3

    dec_us, split_us, gemm_us = avg_us(0, 1), avg_us(1, 2), avg_us(2, 3)
    flops_step = 2.0 * (M_DEC + M_PRE) * K_ * N_
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    dec_bytes = K_ * N_ * 2 + M_DEC * K_ * 4 + M_DEC * N_ * 4
    split_bytes = M_PRE * K_ * (4 + 2 + 2)
    gemm_mfma_flops = 4.0 * M_PRE * N_ * K_          # both FP16 products
    gemm_tf16 = gemm_mfma_flops / (gemm_us * 1e-6) / 1e12
    traffic = measured_traffic()

    # -- the two headline kernels on their own -------------------------------
    def timed(fn, n, warm=3):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / n * 1e3

    # The same decode projection recorded in a HIP graph (four calls, one per W
    # copy) and replayed: what a captured decode loop pays per call.
    gstream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        with torch.cuda.graph(graph, stream=gstream):
            for j in range(4):
                check(cf.cfp32_linear(x1.data_ptr(), K_, Ws[j].data_ptr(), N_, y1.data_ptr(), N_, M_DEC, N_, K_,
                                      dec_ws.data_ptr(), dec_ws_bytes, gstream.cuda_stream), "decode graph")
    torch.cuda.synchronize()
    gemv_graph_us = timed(lambda i: graph.replay(), 50) / 4
    del graph
    # The decode projection with the weights as torch.nn.Linear stores them
    # ([N, K]): one dispatch, each output column streaming its own W row.
    Wts = [Ws[0].view(K_, N_).t().contiguous()]
    for _ in range(3):
        Wts.append(Wts[0].clone())
    gemv_nk_us = timed(lambda i: check(cf.cfp32_linear_ex(x1.data_ptr(), K_, Wts[i % 4].data_ptr(), K_, cf.W_NK,
                                                          None, y1.data_ptr(), N_, M_DEC, N_, K_, None, 0, sh),
                                       "decode nk"), 100)
    # The FFN projection with those weights: the split, then the [N, K] GEMM
    # (64-deep W stages), against split_us + gemm_us of the [K, N] step.
    nk_ws_bytes = cf.cfp32_linear_ex_workspace_bytes(M_PRE, N_, K_, cf.W_NK)
    nk_ws = torch.empty(max(nk_ws_bytes, 1), dtype=torch.uint8, device=dev)
    linear_nk_us = timed(lambda i: check(cf.cfp32_linear_ex(x2.data_ptr(), K_, Wts[i % 4].data_ptr(), K_, cf.W_NK,
                                                            None, y2.data_ptr(), N_, M_PRE, N_, K_,
                                                            nk_ws.data_ptr(), nk_ws_bytes, sh), "prefill nk"), 20)
    del Wts, nk_ws
    gemv_us = timed(lambda i: check(cf.cfp32_linear(x1.data_ptr(), K_, Ws[i % 4].data_ptr(), N_, y1.data_ptr(), N_,
                                                    M_DEC, N_, K_, dec_ws.data_ptr(), dec_ws_bytes, sh), "decode"), 100)
    # Batched decode (the rows of the prefill input, same W copies): 16 rows
    # take the small-M dispatches, 64 the split-K GEMM.
    batched = {}
    for mb in (16, 64):
        xb = x2[:mb]
        yb = torch.empty((mb, N_), dtype=torch.float32, device=dev)
        need_b = cf.cfp32_linear_workspace_bytes(mb, N_, K_)
        wsb = torch.empty(max(need_b, 1), dtype=torch.uint8, device=dev)
        us = timed(lambda i, xb=xb, yb=yb, wsb=wsb, mb=mb, need_b=need_b: check(
            cf.cfp32_linear(xb.data_ptr(), K_, Ws[i % 4].data_ptr(), N_, yb.data_ptr(), N_, mb, N_, K_,
                            wsb.data_ptr(), need_b, sh), "batched decode"), 50)
        bytes_b = K_ * N_ * 2 + mb * K_ * 4 + mb * N_ * 4
        batched[f"linear_{mb}x4096x14336_us"] = round(us, 2)
        batched[f"linear_{mb}x4096x14336_frac_hbm"] = round(bytes_b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        del xb, yb, wsb
    sq = workloads.square()
    xs = torch.from_numpy(sq.A[0]).to(dev)
    ws = torch.from_numpy(sq.W.view(np.int16)).to(dev)
    hs = torch.empty((4096, 4096), dtype=torch.int16, device=dev)
    ls = torch.empty((4096, 4096), dtype=torch.int16, device=dev)
    ys = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
    check(cf.cfp32_split(xs.data_ptr(), 4096, hs.data_ptr(), ls.data_ptr(), 4096, 4096, 4096, sh), "split")
    sq_us = timed(lambda i: check(cf.cfp32_gemm(hs.data_ptr(), ls.data_ptr(), 4096, ws.data_ptr(), 4096,
                                                ys.data_ptr(), None, None, 4096, 4096, 4096, 4096, sh), "gemm"), 50)
    # A/B against true FP32: the whole compensated projection (split + GEMM)
    # next to the FP32 library GEMM (torch.matmul, FP32 inputs and
    # accumulation, TF32 off) on the same 4096^3 operands.
    lin_ws_bytes = cf.cfp32_linear_workspace_bytes(4096, 4096, 4096)
    lin_ws = torch.empty(lin_ws_bytes, dtype=torch.uint8, device=dev)
    lin_us = timed(lambda i: check(cf.cfp32_linear(xs.data_ptr(), 4096, ws.data_ptr(), 4096, ys.data_ptr(), 4096,
                                                   4096, 4096, 4096, lin_ws.data_ptr(), lin_ws_bytes, sh),
                                   "linear"), 50)
    torch.backends.cuda.matmul.allow_tf32 = False
    wf32 = ws.view(torch.float16).float()
    yf32 = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
    fp32_us = timed(lambda i: torch.matmul(xs, wf32, out=yf32), 20)
    # and this library's own true-FP32 kernel (FP32 matrix unit) on the same operands
    own_fp32_us = timed(lambda i: check(cf.cfp32_linear_f32(xs.data_ptr(), 4096, ws.data_ptr(), 4096, yf32.data_ptr(),
                                                            4096, 4096, 4096, 4096, sh), "linear_f32"), 10)
    del lin_ws, wf32, yf32
    # The FFN projection with its GEGLU fused (x2 [8192, 4096], W [4096, 14336]
    # as gate | up, F = 7168) next to the plain projection of the same operands.
    geglu_ws_bytes = cf.cfp32_linear_geglu_workspace_bytes(M_PRE, N_ // 2, K_)
    geglu_ws = torch.empty(geglu_ws_bytes, dtype=torch.uint8, device=dev)
    geglu_out = torch.empty((M_PRE, N_ // 2), dtype=torch.float32, device=dev)
    geglu_us = timed(lambda i: check(cf.cfp32_linear_geglu(x2.data_ptr(), K_, Ws[i % 4].data_ptr(), N_, None,
                                                           geglu_out.data_ptr(), N_ // 2, M_PRE, N_ // 2, K_,
                                                           geglu_ws.data_ptr(), geglu_ws_bytes, sh),
                                     "geglu"), 10)
    plain_us = timed(lambda i: check(cf.cfp32_linear(x2.data_ptr(), K_, Ws[i % 4].data_ptr(), N_, y2.data_ptr(), N_,
                                                     M_PRE, N_, K_, geglu_ws.data_ptr(), geglu_ws_bytes, sh),
                                     "linear"), 10)
    del geglu_ws, geglu_out
    # The separate-addition accumulation mode at 4096^3 (same split planes),
    # with plain accumulation in the same kernel configuration as its baseline.
    sep_us = {}
    for kpa in (0, 16, 64, 256):
        sep_us[kpa] = timed(lambda i, kpa=kpa: check(cf.cfp32_gemm_separate_add(
            hs.data_ptr(), ls.data_ptr(), 4096, ws.data_ptr(), 4096, ys.data_ptr(), None, None, 4096,
            4096, 4096, 4096, kpa, sh), "separate add"), 10)
    torch.cuda.synchronize()

    only = None if args.configs == "all" else set(args.configs.split(","))
    configs = None if args.no_configs else measure_configs(stream, with_cpu=not args.no_cpu_baseline, only=only)

    if args.calibration_copy:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA x2 + f32 accumulate (compensated f32)",
        "data": "synthetic",
        "config": {"workload": "decode GEMV 1x4096x14336 + FFN GEMM 8192x4096x14336, shared FP16 W",
                   "M_decode": M_DEC, "M_prefill": M_PRE, "K": K_, "N": N_, "seed": 4,
                   "w_copies_rotated": len(Ws)},
        "roofline": {"bound": "mfma", "kernel": "dual-product GEMM 8192x4096x14336",
                     "achieved": round(gemm_tf16, 1), "peak": round(PEAK_FP16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(gemm_tf16 / PEAK_FP16_TFLOPS, 4),
                     "traffic": traffic},
        "rocprof_mfma": measured_mfma(),
        "rocprof_decode_gemv": measured_gemv(),
        "breakdown": {
            "decode_gemv_us": round(dec_us, 2),
            "decode_gemv_GBps": round(dec_bytes / (dec_us * 1e-6) / 1e9, 1),
            "split_us": round(split_us, 2),
            "split_GBps": round(split_bytes / (split_us * 1e-6) / 1e9, 1),
            "gemm_us": round(gemm_us, 2),
            "gemm_tflops_fp32eq": round(gemm_mfma_flops / 2 / (gemm_us * 1e-6) / 1e12, 1),
            "gemm_frac_fp16_peak": round(gemm_tf16 / PEAK_FP16_TFLOPS, 4),
        },
        "headline": {
            "gemm_4096x4096x4096_us": round(sq_us, 2),
            "gemm_4096_tflops_fp32eq": round(2 * 4096 ** 3 / (sq_us * 1e-6) / 1e12, 1),
            "gemm_4096_frac_fp16_peak": round(4 * 4096 ** 3 / (sq_us * 1e-6) / 1e12 / PEAK_FP16_TFLOPS, 4),
            "gemv_1x4096x14336_us": round(gemv_us, 2),
            "gemv_GBps": round(dec_bytes / (gemv_us * 1e-6) / 1e9, 1),
            "gemv_frac_hbm": round(dec_bytes / (gemv_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "gemv_graph_1x4096x14336_us": round(gemv_graph_us, 2),
            "gemv_graph_frac_hbm": round(dec_bytes / (gemv_graph_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "gemv_nk_1x4096x14336_us": round(gemv_nk_us, 2),
            "gemv_nk_frac_hbm": round(dec_bytes / (gemv_nk_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "linear_nk_8192x4096x14336_us": round(linear_nk_us, 2),
            "linear_kn_8192x4096x14336_us": round(split_us + gemm_us, 2),
            **batched,
        },
        "fp32_ab_4096": {
            "cfp32_linear_us": round(lin_us, 2),
            "cfp32_linear_tflops_fp32eq": round(2 * 4096 ** 3 / (lin_us * 1e-6) / 1e12, 1),
            "fp32_own_kernel_us": round(own_fp32_us, 2),
            "fp32_own_kernel_tflops": round(2 * 4096 ** 3 / (own_fp32_us * 1e-6) / 1e12, 1),
            "fp32_own_kernel_frac_fp32_mfma_peak": round(2 * 4096 ** 3 / (own_fp32_us * 1e-6) / 1e12 / 157.3, 4),
            "fp32_library_matmul_us": round(fp32_us, 2),
            "fp32_library_tflops": round(2 * 4096 ** 3 / (fp32_us * 1e-6) / 1e12, 1),
            "speedup_vs_own_fp32": round(own_fp32_us / lin_us, 2),
            "speedup": round(fp32_us / lin_us, 2),
        },
        "geglu_ffn_8192x4096x7168": {
            "linear_geglu_us": round(geglu_us, 2),
            "linear_plain_us": round(plain_us, 2),
            "geglu_tflops_fp32eq": round(2 * M_PRE * N_ * K_ / (geglu_us * 1e-6) / 1e12, 1),
        },
        "separate_add_4096": {
            "gemm_us": round(sq_us, 2),
            **{f"k_per_add_{k}_us": round(v, 2) for k, v in sep_us.items()},
        },
        "configs": configs,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count, "torch": torch.__version__,
                   "hip": getattr(torch.version, "hip", None)},
        "host": host_info(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(A1, A2, W, args.cpu_rows_per_thread)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
