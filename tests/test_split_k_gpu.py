"""GPU tests of the batched-decode paths of cfp32_linear / cfp32_linear_ex
(fewer than 128 output tiles of 128 x 256; from 17 to 64 rows except where
32 x 128 output tiles number 192 to 256 and K <= 4096; above 64 rows only where K
gives at least 128 blocks of four 64-deep units, 192 where the small-grid
kernel could run the grid):
  * split K (the GEMM path; K % 8 == 0): K is cut into chunks of 64-deep
    units, each chunk's C_hi, C_lo go to FP32 partial sums, and a merge
    dispatch adds them in chunk order and merges once.  The plan depends on
    M, N, K only, so the LDS-DMA kernel (aligned weights, M > 16) and the
    generic kernel (unaligned weights) give identical bits in both layouts;
  * [K, N] weights with M <= 16 that allow 16-byte loads: the small-M
    product and merge dispatches with two groups of 8 rows of x ([N, K]
    weights take split K there too).
Each: y is finite and within 1e-5 * sum|a w| of the FP64 reference, its
error at least 16x below that of the single-FP16 product, repeated calls give
identical bits, and the bias is one more FP32 addition after the merge.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import assert_better_than_single, assert_within_tolerance, note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu


def run(A, W, layout=cf.W_KN, w_offset=0, bias=None):
    M, K = A.shape
    N = W.shape[1]
    Wl = W if layout == cf.W_KN else np.ascontiguousarray(W.T)
    rows, cols = Wl.shape
    ldw = cols + w_offset
    wb = np.zeros(rows * ldw + w_offset, np.uint16)
    wb[w_offset:].reshape(rows, ldw)[:, :cols] = Wl.view(np.uint16)
    dx, dw = to_dev(A), to_dev(wb)
    db = to_dev(bias) if bias is not None else None
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, layout)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")  # contents must not matter
    st = cf.cfp32_linear_ex(dx.data_ptr(), K, dw.data_ptr() + 2 * w_offset, ldw, layout,
                            db.data_ptr() if db is not None else None, y.data_ptr(), N, M, N, K,
                            ws.data_ptr() if need else None, need, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    return to_host(y)


def planes_bytes(M, K):
    ld = (K + 7) // 8 * 8
    return 2 * ((M * ld * 2 + 255) // 256 * 256)


def check(y, A, W, what):
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, what)
    _, ch, _ = oracle.linear_cf32(A[:16], W)
    assert_better_than_single(y[:16], ch, y64[:16], abs64[:16], what)


# (M, K, N): the smallest M of the GEMM path, ragged N and K; many chunks;
# the batched-decode FFN down projection at 64 rows; a ragged last unit of K;
# a chunk count that is not a power of two.
SHAPES = [(9, 1000, 777), (16, 4096, 2048), (64, 14336, 4096), (40, 4104, 520), (24, 2000, 777)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_split_k_against_reference_and_across_kernels(M, K, N):
    """Unaligned weights (generic kernel) in both layouts, and aligned ones
    from 17 ([K, N]) or 33 ([N, K]) rows up (LDS-DMA kernel with the hi and
    lo rows stacked into one tile), cut K at the same places: the same bits,
    within tolerance.  Below that aligned weights take the small-M
    dispatches (checked against the reference).  [K, N] weights with N not a
    multiple of 8 are copied into aligned rows first, so up to 16 rows they
    too take the small-M dispatches."""
    need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, cf.W_NK)
    assert need > planes_bytes(M, K) + 256, "shape does not take the split-K path"
    A, W = workloads.random_case(M * 7 + K + N, M, K, N, a_scale=20.0)
    note(f"split-K {M}x{K}x{N}")
    y = run(A, W, layout=cf.W_NK, w_offset=1)  # generic kernel, split K
    check(y, A, W, f"split-K {M}x{K}x{N}")
    y_kn = run(A, W, w_offset=1)
    runs = []
    if M > 16 or N % 8 == 0:  # the [K, N] run cuts K the same way
        runs.append(y_kn)
    else:
        check(y_kn, A, W, f"small-M (padded W) {M}x{K}x{N}")
        assert np.array_equal(y_kn.view(np.uint32), run(A, W).view(np.uint32))
    if M > 16:
        runs.append(run(A, W))
    if M > 32:
        runs.append(run(A, W, layout=cf.W_NK))
    else:  # aligned [N, K] weights up to 32 rows take the small-M [N, K] dispatch
        check(run(A, W, layout=cf.W_NK), A, W, f"small-M [N, K] {M}x{K}x{N}")
    for y2 in runs:
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    y3 = run(A, W, w_offset=1)
    assert np.array_equal(y_kn.view(np.uint32), y3.view(np.uint32)), "not deterministic"


# (M, K, N): ragged M inside the second group of 8 rows, ragged N and K, the
# batched-decode FFN shape, one chunk (many tiles).
WIDE = [(9, 1000, 776), (16, 4096, 14336), (13, 333, 1000), (12, 64, 140000), (16, 4100, 2048)]


@pytest.mark.parametrize("layout", [cf.W_KN, cf.W_NK])
@pytest.mark.parametrize("M,K,N", WIDE)
def test_small_m_groups_against_reference(M, K, N, layout):
    A, W = workloads.random_case(M * 11 + K + 3 * N, M, K, N, a_scale=20.0)
    note(f"small-M groups {M}x{K}x{N} layout {layout}")
    y = run(A, W, layout=layout)
    if N > 20000:  # the FP64 reference on a column sample
        cols = np.random.default_rng(N).choice(N, 2048, replace=False)
        check(y[:, cols], A, np.ascontiguousarray(W[:, cols]), f"small-M groups {M}x{K}x{N}")
    else:
        check(y, A, W, f"small-M groups {M}x{K}x{N}")
    y2 = run(A, W, layout=layout)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"


@pytest.mark.parametrize("M,K,N,layout", [(32, 2048, 1000, cf.W_NK), (24, 2048, 1000, cf.W_KN),
                                          (16, 2048, 1000, cf.W_KN), (12, 2048, 1000, cf.W_NK)])
def test_bias_is_one_addition(M, K, N, layout):
    A, W = workloads.random_case(99 + M, M, K, N, a_scale=20.0)
    bias = (np.random.default_rng(5).standard_normal(N) * 3).astype(np.float32)
    note(f"bias {M}x{K}x{N}")
    y0 = run(A, W, layout=layout)
    y1 = run(A, W, layout=layout, bias=bias)
    assert np.array_equal(y1.view(np.uint32), (y0 + bias[None, :]).astype(np.float32).view(np.uint32))


# (M, K, N) above 64 rows: the batched FFN shape (four chunks), ragged M, N
# and a ragged last unit of K, three chunks with 192 blocks, ragged M with
# many chunks, ragged M with three chunks and 144 blocks.
WIDE_SPLIT = [(96, 4096, 14336), (200, 4000, 10000), (256, 4096, 8192), (130, 8192, 2056), (300, 4096, 4096)]


@pytest.mark.parametrize("M,K,N", WIDE_SPLIT)
def test_split_k_above_64_rows(M, K, N):
    """The same cut of K from every kernel (LDS-DMA with aligned weights in
    both layouts, the generic kernel with unaligned ones): identical bits,
    within tolerance of FP64, below the single-FP16 error, repeatable."""
    need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, cf.W_NK)
    assert need > planes_bytes(M, K) + 256, "shape does not take the split-K path"
    A, W = workloads.random_case(M * 5 + K + 3 * N, M, K, N, a_scale=20.0)
    note(f"split-K above 64 rows {M}x{K}x{N}")
    y = run(A, W)
    check(y, A, W, f"split-K {M}x{K}x{N}")
    for other in (run(A, W, layout=cf.W_NK), run(A, W, w_offset=1), run(A, W, layout=cf.W_NK, w_offset=1)):
        assert np.array_equal(y.view(np.uint32), other.view(np.uint32)), "kernels cut K differently"
    assert np.array_equal(y.view(np.uint32), run(A, W).view(np.uint32)), "not deterministic"
    bias = (np.random.default_rng(M).standard_normal(N) * 3).astype(np.float32)
    yb = run(A, W, bias=bias)
    assert np.array_equal(yb.view(np.uint32), (y + bias[None, :]).astype(np.float32).view(np.uint32))
