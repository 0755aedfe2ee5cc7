"""Build libcfp32.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m compensated_fp32_projection_amd.build [--verbose] [--resource-usage]

The library is built in-tree, next to this file, so that it travels with the
source tree.  Flags that the numerics rely on:

* ``-ffp-contract=off``: the merge's scale and add stay two rounded
  operations (fused multiply-adds are written explicitly where they are meant);
* ``-fno-gpu-flush-denormals-to-zero``: FP32 subnormals are kept;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed FP32 VALU
  instructions are generated;
* never ``-ffast-math``.
"""
from __future__ import annotations

import argparse
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcfp32.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile every HIP source into libcfp32.so; returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *sources(), "-o", tmp]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and (verbose or resource_usage):
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.verbose, resource_usage=a.resource_usage))
