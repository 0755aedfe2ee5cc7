"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code,
run on the CPU.

  * the CPU oracle (oracle/cfp32_oracle.c, with OpenMP) and a driver that
    calls every oracle function on operands allocated to their exact extent
    (tests/sanitize/oracle_driver.c);
  * the host side of the C ABI -- argument validation and path planning
    (api.hip, plans.hip; kernels are not built) -- with launcher stubs that
    abort if reached, and a driver running every invalid-argument, size-query
    and empty-problem case of include/cfp32.h (tests/sanitize/abi_driver.c),
    plus, where no GPU is visible, the refusal of valid calls.

Each driver must exit 0 with no sanitizer report.  GPU code is not
sanitized (those tools are not available for gfx950 here); the kernels'
memory safety is covered by the bounds reasoning in their sources and the
GPU parity tests.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "compensated_fp32_projection_amd", "csrc")
LLVM = "/opt/rocm/llvm/bin"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "4"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _clean(stderr: str):
    assert "AddressSanitizer" not in stderr and "runtime error" not in stderr, stderr


@pytest.fixture(scope="module")
def build_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


def test_oracle_under_sanitizers(build_dir):
    if not shutil.which("gcc"):
        pytest.skip("gcc is not available")
    exe = os.path.join(build_dir, "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          os.path.join(ROOT, "oracle", "cfp32_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe], env={**os.environ, **SAN_ENV})
    _clean(r.stderr)
    assert "0 failure(s)" in r.stderr


def test_abi_host_code_under_sanitizers(build_dir):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists(os.path.join(LLVM, "clang")):
        pytest.skip("the ROCm compilers are not available")
    san_host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in ("api.hip", "plans.hip"):
        obj = os.path.join(build_dir, src + ".o")
        _run([hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC", "-ffp-contract=off", *san_host,
              "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    stubs = os.path.join(build_dir, "stubs.o")
    _run([os.path.join(LLVM, "clang++"), "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-c",
          os.path.join(SAN, "launcher_stubs.cpp"), "-o", stubs])
    drv = os.path.join(build_dir, "abi_driver.o")
    _run([os.path.join(LLVM, "clang"), "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = os.path.join(build_dir, "abi_driver")
    _run([os.path.join(LLVM, "clang++"), "-fsanitize=address,undefined", drv, *objs, stubs, "-L/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    args = [exe]
    try:
        import torch
        if not torch.cuda.is_available():
            args.append("no-device")
    except ImportError:
        args.append("no-device")
    r = _run(args, env={**os.environ, **SAN_ENV})
    _clean(r.stderr)
    assert "0 failure(s)" in r.stderr


def test_the_sanitizers_report_a_planted_error(build_dir, tmp_path):
    """Control: the same flags do report a heap read one element past an
    allocation, so a clean run above means something."""
    if not shutil.which("gcc"):
        pytest.skip("gcc is not available")
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\nint main(void) { volatile int *a = malloc(4 * sizeof(int)); "
                   "int v = a[4]; free((void *)a); return v == 12345; }\n")
    exe = str(tmp_path / "oob")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60, env={**os.environ, **SAN_ENV})
    # UBSan's object-size check or ASan's heap-buffer-overflow, whichever halts first
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error" in r.stderr), r.stderr
