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
import datetime
import glob
import hashlib
import json
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcfp32.so")
# Written next to the library on every build: the git revision (and whether
# the tree had uncommitted changes), a hash of the sources and of the
# library, so a measurement can name the build it ran even where the source
# tree travels without its git history.
BUILD_INFO = os.path.join(HERE, "build_info.json")
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


def _git(*args) -> str | None:
    try:
        r = subprocess.run(["git", *args], cwd=HERE, capture_output=True, text=True, timeout=20)
        return r.stdout.strip() if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def source_hash() -> str:
    """sha256 over the library's sources and its public header."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*"))) + [os.path.join(HERE, "..", "include", "cfp32.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def file_hash(path: str) -> str:
    h = hashlib.sha256()
    with open(path, "rb") as fh:
        for chunk in iter(lambda: fh.read(1 << 20), b""):
            h.update(chunk)
    return h.hexdigest()


def write_build_info() -> dict:
    status = _git("status", "--porcelain", "--untracked-files=no")
    info = {
        "git_revision": _git("rev-parse", "HEAD"),
        "git_dirty": None if status is None else bool(status),
        "source_sha256": source_hash(),
        "library_sha256": file_hash(LIB),
        "built_utc": datetime.datetime.now(datetime.timezone.utc).strftime("%Y-%m-%dT%H:%M:%SZ"),
        "arch": ARCH,
    }
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f, indent=1)
    return info


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
    write_build_info()
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.verbose, resource_usage=a.resource_usage))
