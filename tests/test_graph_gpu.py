"""The library under HIP graph capture: projections (both weight layouts) and
fused GEGLU calls recorded into a graph (the way decode loops usually run)
and replayed must give what the same calls give eagerly, replay after
replay, with new inputs written between replays.

The library records no memset and keeps no state between calls: the small-M
path's workspace holds partial sums that every call rewrites before reading,
and the M > 8 path's hi/lo planes likewise.  Each replay here is checked bit
for bit against an eager call on the same inputs, with eager work and
synchronisations between the replays -- also with the eager calls on the
graph's own workspace, so that eager calls and replays alternate on one
workspace.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
from compensated_fp32_projection_amd import workloads
from gpu_helpers import note, to_dev, to_host

pytestmark = pytest.mark.gpu


# [K, N] weights: the small-M product + merge dispatches, the generic small-M
# kernel, the small-grid kernel, the generic GEMM's 32 x 128 tile with the
# split in registers.  [N, K] weights: the one-dispatch small-M kernel (one
# and three groups of 8 rows), the small-grid kernel and the 32 x 128 tile.
@pytest.mark.parametrize("shared_ws", [False, True])
@pytest.mark.parametrize("M,K,N,layout", [(1, 4096, 14336, "kn"), (4, 1000, 520, "kn"), (2, 24, 40, "kn"),
                                          (12, 2048, 3000, "kn"), (300, 512, 768, "kn"), (512, 776, 2304, "kn"),
                                          (1, 4096, 14336, "nk"), (20, 1024, 3000, "nk"), (300, 512, 768, "nk"),
                                          (600, 200, 2000, "nk")])
def test_linear_replays_match_eager(M, K, N, layout, shared_ws):
    A, W = workloads.random_case(M + K + N, M, K, N, a_scale=4.0)
    dw = to_dev(W if layout == "kn" else np.ascontiguousarray(W.T)).view(torch.float16)
    x = to_dev(A)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = cf.Workspace()
    note(f"graph capture linear {M}x{K}x{N} {layout}")
    cf.linear(x, dw, out=y, workspace=ws, w_layout=layout)  # allocates the workspace outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            cf.linear(x, dw, out=y, workspace=ws, stream=stream, w_layout=layout)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M * 7 + N)
    for r in range(4):
        new = (rng.standard_normal(A.shape) * (r + 1)).astype(np.float32)
        x.copy_(torch.from_numpy(new).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_host(y).copy()
        ref = to_host(cf.linear(x, dw, workspace=ws if shared_ws else cf.Workspace(), w_layout=layout))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"replay {r}"


# The fused GEGLU: small-M product + GEGLU merge (M = 1), split K with the
# GEGLU merge (M = 40), the GEMM's GEGLU epilogue (M = 2100).
@pytest.mark.parametrize("M,K,F", [(1, 4096, 1536), (40, 512, 300), (2100, 512, 1000)])
def test_geglu_replays_match_eager(M, K, F):
    A, W = workloads.random_case(M + K + 3 * F, M, K, 2 * F, a_scale=4.0)
    dw = to_dev(W).view(torch.float16)
    x = to_dev(A)
    out = torch.empty((M, F), dtype=torch.float32, device="cuda")
    ws = cf.Workspace()
    note(f"graph capture geglu {M}x{K}x{F}")
    cf.linear_geglu(x, dw, out=out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            cf.linear_geglu(x, dw, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M * 5 + F)
    for r in range(4):
        new = (rng.standard_normal(A.shape) * (r + 1)).astype(np.float32)
        x.copy_(torch.from_numpy(new).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_host(out).copy()
        ref = to_host(cf.linear_geglu(x, dw, workspace=cf.Workspace()))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"replay {r}"
