"""The library under HIP graph capture: calls recorded into a graph (the
way decode loops usually run) and replayed must give what the same calls give
eagerly, replay after replay, with new inputs written between replays.

The library records no memset and keeps no state between calls: the small-M
path's workspace holds partial sums that every call rewrites before reading,
and the M > 8 path's hi/lo planes likewise.  Each replay here is checked bit
for bit against an eager call on the same inputs, with eager work and
synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
from compensated_fp32_projection_amd import workloads
from gpu_helpers import note, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N", [(1, 4096, 14336), (4, 1000, 520), (2, 24, 40), (300, 512, 768)])
def test_linear_replays_match_eager(M, K, N):
    A, W = workloads.random_case(M + K + N, M, K, N, a_scale=4.0)
    dw = to_dev(W).view(torch.float16)
    x = to_dev(A)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = cf.Workspace()
    note(f"graph capture linear {M}x{K}x{N}")
    cf.linear(x, dw, out=y, workspace=ws)  # allocates the workspace outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            cf.linear(x, dw, out=y, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M * 7 + N)
    for r in range(4):
        new = (rng.standard_normal(A.shape) * (r + 1)).astype(np.float32)
        x.copy_(torch.from_numpy(new).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_host(y).copy()
        ref = to_host(cf.linear(x, dw, workspace=cf.Workspace()))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"replay {r}"
