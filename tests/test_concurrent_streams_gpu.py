"""Calls in flight together: the library keeps no state between calls beyond
a per-device architecture check (an atomic) and a per-thread last HIP error,
so projections launched on different streams, each with its own workspace,
from one host thread or from several, must give the bits each gives alone.

Each case mixes the paths: the small-M decode dispatch and its partial-sum
merge ([K, N] weights), the one-dispatch [N, K] decode kernel, split K over
the GEMM tiles, the split-inside GEMM and the GEGLU epilogue.  Every output of
the concurrent runs is compared bit for bit with a serial run on the default
stream.
"""
import threading

import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
from compensated_fp32_projection_amd import workloads
from gpu_helpers import note, to_dev, to_host

pytestmark = pytest.mark.gpu

# (kind, M, K, N): "kn" / "nk" linear, "geglu" with N = 2F.
CASES = [("kn", 1, 4096, 3584), ("nk", 3, 2048, 1536), ("kn", 40, 1024, 2048), ("kn", 1024, 512, 4096),
         ("geglu", 2, 1024, 1024), ("nk", 64, 512, 1000), ("geglu", 300, 256, 512)]


class Job:
    def __init__(self, idx, kind, M, K, N, own_workspace=True):
        A, W = workloads.random_case(1000 + idx, M, K, N, a_scale=8.0)
        self.kind = kind
        self.x = to_dev(A)
        w = W if kind != "nk" else np.ascontiguousarray(W.T)
        self.w = to_dev(w).view(torch.float16)
        cols = N // 2 if kind == "geglu" else N
        self.out = torch.full((M, cols), 3.0, dtype=torch.float32, device="cuda")
        self.ws = cf.Workspace() if own_workspace else None

    def run(self, stream=None):
        if self.kind == "geglu":
            cf.linear_geglu(self.x, self.w, out=self.out, workspace=self.ws, stream=stream)
        else:
            cf.linear(self.x, self.w, out=self.out, workspace=self.ws, stream=stream, w_layout=self.kind)


def serial_results(jobs):
    res = []
    for j in jobs:
        j.run()
        res.append(to_host(j.out).copy())
    return res


def check(jobs, want, what):
    for j, w in zip(jobs, want):
        got = to_host(j.out)
        assert np.array_equal(got.view(np.uint32), w.view(np.uint32)), f"{what}: {j.kind} {tuple(j.x.shape)}"


def test_many_streams_one_thread():
    """Every job on its own stream, launched round-robin several times, with
    no synchronisation between launches."""
    jobs = [Job(i, *c) for i, c in enumerate(CASES)]
    note("concurrent streams: serial pass")
    want = serial_results(jobs)
    for j in jobs:
        j.out.fill_(3.0)
    streams = [torch.cuda.Stream() for _ in jobs]
    torch.cuda.synchronize()
    note(f"concurrent streams: {len(jobs)} streams x 3 rounds")
    for _ in range(3):
        for j, s in zip(jobs, streams):
            with torch.cuda.stream(s):
                j.run(stream=s)
    torch.cuda.synchronize()
    check(jobs, want, "streams")


def test_two_host_threads():
    """Two host threads, each with its own streams, calling the C-ABI at the
    same time (the foreign calls release the interpreter lock)."""
    jobs = [Job(i, *c) for i, c in enumerate(CASES + CASES[:1])]
    note("concurrent threads: serial pass")
    want = serial_results(jobs)
    for j in jobs:
        j.out.fill_(3.0)
    torch.cuda.synchronize()
    halves = [jobs[0::2], jobs[1::2]]
    errors = []
    barrier = threading.Barrier(2)

    def worker(mine):
        try:
            s = torch.cuda.Stream()
            barrier.wait()
            with torch.cuda.stream(s):
                for _ in range(4):
                    for j in mine:
                        j.run(stream=s)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    note("concurrent threads: 2 threads x 4 rounds")
    threads = [threading.Thread(target=worker, args=(h,)) for h in halves]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    check(jobs, want, "threads")


def test_many_streams_default_workspace():
    """The tensor helpers' own workspace (no ``workspace=`` given): one per
    device and stream, so jobs on different streams in flight together never
    share scratch memory, and each gives the bits of its serial run."""
    jobs = [Job(i, *c, own_workspace=False) for i, c in enumerate(CASES)]
    note("concurrent streams, default workspace: serial pass")
    want = serial_results(jobs)
    for j in jobs:
        j.out.fill_(3.0)
    streams = [torch.cuda.Stream() for _ in jobs]
    torch.cuda.synchronize()
    note(f"concurrent streams, default workspace: {len(jobs)} streams x 3 rounds")
    for _ in range(3):
        for j, s in zip(jobs, streams):
            with torch.cuda.stream(s):
                j.run(stream=s)
    torch.cuda.synchronize()
    check(jobs, want, "streams, default workspace")
