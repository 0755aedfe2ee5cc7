"""The small-grid projection kernel (gemm_ksplit.hip): K split across the four
waves of each 32 x 64 output tile, x split in registers, one launch.

cfp32_linear takes it for projections that do not split K across blocks and
whose 32 x 64 tiles fit the GPU at once (at most 512 blocks), where the
generic kernel's 32 x 128 tiles would number fewer than 128.  Its summation
order differs from the K-sequential kernels', so its bits are its own; the
checks are those of every path (compensated-FP32 paragraph of the laya.cpp
Vulkan guide): every element within 1e-5 * sum |a w| of the FP64 reference,
error at least 16x below the single-FP16-conversion product, repeatable
bits, the same bits for [K, N] and [N, K] weights, and a bias that is one
more FP32 addition."""
import numpy as np
import pytest
import torch

import bench
import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import assert_better_than_single, assert_within_tolerance, note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu


def run(A, W, layout=cf.W_KN, bias=None, stream=None):
    M, K = A.shape
    N = W.shape[1]
    Wl = W if layout == cf.W_KN else np.ascontiguousarray(W.T)
    ldw = Wl.shape[1]
    dx, dw = to_dev(A), to_dev(Wl.view(np.uint16))
    db = to_dev(bias) if bias is not None else None
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, layout)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")

    def call(s):
        st = cf.cfp32_linear_ex(dx.data_ptr(), K, dw.data_ptr(), ldw, layout,
                                db.data_ptr() if db is not None else None, y.data_ptr(), N, M, N, K,
                                ws.data_ptr() if need else None, need, s)
        assert st == cf.OK, cf.cfp32_status_string(st)

    call(stream_handle())
    out = to_host(y)
    launches = bench.graph_launches(call)
    return out, launches


def takes_ksplit(M, N, K):
    """At most 512 tiles of 32 x 64 and fewer than 128 of 32 x 128 (from
    there the generic kernel's 32 x 128 tile), K % 8 == 0, and no split of K
    across blocks (that needs M <= 64 and at least four 64-deep units per
    chunk)."""
    tiles = ((M + 31) // 32) * ((N + 63) // 64)
    small = ((M + 31) // 32) * ((N + 127) // 128)
    return tiles <= 512 and small < 128 and K % 8 == 0 and (M > 64 or K < 512)


# (M, K, N): 96 rows of a 4096 x 4096 weight; a square panel; a cube; the
# unaligned workload's rows and K with N rounded to 8; ragged M, N and a K
# that is not a whole number of 32-deep stages (264 = 33 x 8); K below one
# stage; 40 rows with K too short to split across blocks; one output
# column; a single column of tiles with K = 4096.
SHAPES = [(96, 4096, 4096), (128, 2048, 2048), (512, 512, 512), (333, 1000, 784), (65, 264, 130),
          (100, 8, 72), (40, 40, 64), (130, 4096, 1), (512, 4096, 64)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_ksplit_against_reference(M, K, N):
    assert takes_ksplit(M, N, K)
    A, W = workloads.random_case(M * 13 + K + 7 * N, M, K, N, a_scale=40.0)
    note(f"ksplit {M}x{K}x{N}")
    y, launches = run(A, W)
    # one launch; [K, N] weights with N % 8 != 0 are first copied into rows of
    # N rounded up to 8 (one more launch)
    want = 1 + (N % 8 != 0)
    assert launches in (None, want), f"{launches} launches, not {want}: not the small-grid kernel"
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, f"ksplit {M}x{K}x{N}")
    rows = min(M, 32)
    _, ch, _ = oracle.linear_cf32(A[:rows], W)
    assert_better_than_single(y[:rows], ch, y64[:rows], abs64[:rows], f"ksplit {M}x{K}x{N}")
    y2, _ = run(A, W)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    if M > 32:  # [N, K] weights reach the same kernel (up to 32 rows they take the small-M [N, K] one)
        y_nk, launches_nk = run(A, W, layout=cf.W_NK)
        assert launches_nk in (None, 1)
        assert np.array_equal(y.view(np.uint32), y_nk.view(np.uint32)), "[N, K] and [K, N] differ"


# (M, K, N): up to 16 rows the kernel replaces the small-M dispatches on
# tiny grids with K <= 1024: the single-linear workload's shape, a wider W,
# two groups of rows, a K that is not a whole number of stages, odd N.
TINY = [(16, 256, 384), (12, 256, 2048), (9, 512, 512), (16, 1024, 1024), (13, 264, 200), (10, 96, 77)]


@pytest.mark.parametrize("M,K,N", TINY)
def test_small_rows_on_tiny_grids(M, K, N):
    A, W = workloads.random_case(M * 17 + K + N, M, K, N, a_scale=40.0)
    note(f"tiny grid {M}x{K}x{N}")
    y, _ = run(A, W)
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, f"tiny {M}x{K}x{N}")
    _, ch, _ = oracle.linear_cf32(A, W)
    assert_better_than_single(y, ch, y64, abs64, f"tiny {M}x{K}x{N}")
    y2, _ = run(A, W)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    bias = np.random.default_rng(M).standard_normal(N).astype(np.float32)
    yb, _ = run(A, W, bias=bias)
    assert np.array_equal(yb.view(np.uint32), (y + bias[None, :]).astype(np.float32).view(np.uint32))


def test_ksplit_unaligned_workload_with_padded_copy():
    """The unaligned workload (333 x 1000 x 777): W is first copied into rows
    of 784 elements, then the small-grid kernel runs (two launches)."""
    wl = workloads.unaligned()
    A, W = wl.A[0], wl.W
    note("ksplit unaligned workload")
    y, launches = run(A, W)
    assert launches in (None, 2)
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, "unaligned")
    _, ch, _ = oracle.linear_cf32(A, W)
    assert_better_than_single(y, ch, y64, abs64, "unaligned")


@pytest.mark.parametrize("layout", [cf.W_KN, cf.W_NK])
def test_ksplit_bias_is_one_addition(layout):
    M, K, N = 70, 520, 200
    A, W = workloads.random_case(99, M, K, N, a_scale=10.0)
    bias = np.random.default_rng(7).standard_normal(N).astype(np.float32)
    note(f"ksplit bias layout {layout}")
    y, _ = run(A, W, layout=layout)
    yb, _ = run(A, W, layout=layout, bias=bias)
    assert np.array_equal(yb.view(np.uint32), (y + bias[None, :]).astype(np.float32).view(np.uint32))


def test_ksplit_wider_grids_keep_the_tiled_kernels():
    """Above 512 tiles of 32 x 64 (the QKV workload: 576) the projection keeps
    the tiled GEMM (here its 32 x 128 tile, with the split in registers: one
    launch), whose bits equal cfp32_split + cfp32_gemm."""
    wl = workloads.qkv_projection()
    A, W = wl.A[0], wl.W
    M, K = A.shape
    N = W.shape[1]
    assert not takes_ksplit(M, N, K) or ((M + 31) // 32) * ((N + 63) // 64) > 512
    note("qkv workload: tiled GEMM")
    y, launches = run(A, W)
    assert launches in (None, 1)
    dx, dw = to_dev(A), to_dev(W)
    hi = torch.empty((M, K), dtype=torch.int16, device="cuda")
    lo = torch.empty((M, K), dtype=torch.int16, device="cuda")
    y2 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    assert cf.cfp32_split(dx.data_ptr(), K, hi.data_ptr(), lo.data_ptr(), K, M, K, stream_handle()) == cf.OK
    assert cf.cfp32_gemm(hi.data_ptr(), lo.data_ptr(), K, dw.data_ptr(), N, y2.data_ptr(), None, None, N,
                         M, N, K, stream_handle()) == cf.OK
    assert np.array_equal(y.view(np.uint32), to_host(y2).view(np.uint32))


# (M, K, F): F % 8 == 0 (the kernel reads W in place); F % 8 == 4 (2F % 8
# == 0: cfp32_linear_ex runs the kernel on W in place, the GEGLU entry on a
# copy with the up columns moved to F rounded up to 8); F odd (2F % 8 != 0:
# both run on copies of W); 12 rows on a tiny grid.
GEGLU = [(70, 520, 96), (40, 256, 300), (100, 1000, 77), (12, 256, 300)]


@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("M,K,F", GEGLU)
def test_ksplit_geglu_matches_the_projection(M, K, F, with_bias):
    """cfp32_linear_geglu on small grids: gelu(gate) * up of exactly the gate
    and up sums cfp32_linear_ex forms for the [K, 2F] projection, within the
    GELU evaluation tolerance, and the projection within tolerance of FP64."""
    from test_geglu_gpu import check_geglu, full_projection, run_geglu
    assert takes_ksplit(M, 2 * F, K)
    A, W = workloads.random_case(M + 3 * K + F, M, K, 2 * F, a_scale=8.0)
    bias = (np.random.default_rng(F).standard_normal(2 * F) * 0.5).astype(np.float32) if with_bias else None
    note(f"ksplit geglu {M}x{K}x{F} bias={with_bias}")
    out = run_geglu(A, W, bias)
    y_full = full_projection(A, W, bias)
    check_geglu(out, y_full, F, f"ksplit geglu {M}x{K}x{F}")
    out2 = run_geglu(A, W, bias)
    assert np.array_equal(out.view(np.uint32), out2.view(np.uint32)), "not deterministic"
    y64, abs64 = oracle.y64(A, W)
    if bias is not None:
        y64 = y64 + bias.astype(np.float64)
        abs64 = abs64 + np.abs(y64) * 1e-2
    assert_within_tolerance(y_full, y64, abs64, f"ksplit projection {M}x{K}x{2 * F}")
