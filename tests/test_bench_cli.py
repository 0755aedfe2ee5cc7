"""bench.py's command line, checked on the CPU: refusals that happen before
any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_unknown_workload_ids_are_refused():
    r = run_bench("--configs", "2,9")
    assert r.returncode == 2
    assert "unknown workload ids ['9']" in r.stderr


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
