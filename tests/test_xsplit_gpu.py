"""The projection in one launch on the generic kernel's 32 x 128-tile grids
(gemm.hip, FP32-input form): x is split in registers as each stage is
loaded, with the split dispatch's conversion (split/merge paragraph of the
laya.cpp Vulkan guide), so the planes, and every bit of y, are those of
cfp32_split followed by cfp32_gemm.  Checked here: one launch, the same
bits as the two-launch form through the public calls, every element within
tolerance of the FP64 reference with the error at least 16x below the
single-FP16-conversion product, a ragged last stage, short K (one stage
ahead instead of two), [N, K] weights, a bias as one more FP32 addition,
and x whose rows are not 16-byte aligned (split + GEMM instead)."""
import numpy as np
import pytest
import torch

import bench
import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import assert_better_than_single, assert_within_tolerance, note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu


def small_tile_grid(M, N):
    """Grids the generic kernel runs in its 32 x 128 tile (fewer than 128
    tiles of 128 x 256; at most 768 of 32 x 128 or fewer than 256 of
    64 x 128), with more than 512 small-grid tiles of 32 x 64 (fewer take the
    small-grid kernel)."""
    large = ((M + 127) // 128) * ((N + 255) // 256)
    medium = ((M + 63) // 64) * ((N + 127) // 128)
    small = ((M + 31) // 32) * ((N + 127) // 128)
    ks = ((M + 31) // 32) * ((N + 63) // 64)
    return large < 128 and (medium < 256 or small <= 768) and ks > 512


def linear(A, W, layout=cf.W_KN, bias=None, ldx=None):
    M, K = A.shape
    N = W.shape[1]
    Wl = W if layout == cf.W_KN else np.ascontiguousarray(W.T)
    ldw = Wl.shape[1]
    ldx = ldx or K
    xp = np.zeros((M, ldx), np.float32)
    xp[:, :K] = A
    dx, dw = to_dev(xp), to_dev(Wl.view(np.uint16))
    db = to_dev(bias) if bias is not None else None
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, layout)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")

    def call(s):
        st = cf.cfp32_linear_ex(dx.data_ptr(), ldx, dw.data_ptr(), ldw, layout,
                                db.data_ptr() if db is not None else None, y.data_ptr(), N, M, N, K,
                                ws.data_ptr() if need else None, need, s)
        assert st == cf.OK, cf.cfp32_status_string(st)

    call(stream_handle())
    out = to_host(y)
    return out, bench.graph_launches(call)


def two_launch(A, W):
    """cfp32_split into planes, then cfp32_gemm (public calls)."""
    M, K = A.shape
    N = W.shape[1]
    dx, dw = to_dev(A), to_dev(W.view(np.uint16))
    hi = torch.empty((M, K), dtype=torch.int16, device="cuda")
    lo = torch.empty((M, K), dtype=torch.int16, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    assert cf.cfp32_split(dx.data_ptr(), K, hi.data_ptr(), lo.data_ptr(), K, M, K, stream_handle()) == cf.OK
    assert cf.cfp32_gemm(hi.data_ptr(), lo.data_ptr(), K, dw.data_ptr(), N, y.data_ptr(), None, None, N,
                         M, N, K, stream_handle()) == cf.OK
    return to_host(y)


# (M, K, N): the QKV workload's shape; K = 776 (twelve 64-deep stages and a
# ragged 8) with ragged M and N (N % 8 != 0: after the padded copy); K = 200
# (three full stages and a ragged one: one stage ahead); a larger K; a wide,
# short one; a grid of 256 tiles of 64 x 128 that takes the 32 x 128 tile.
SHAPES = [(512, 768, 2304), (520, 776, 2300), (600, 200, 2000), (384, 2048, 3072), (320, 72, 4000),
          (1024, 1024, 2048)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_xsplit_one_launch_same_bits(M, K, N):
    assert small_tile_grid(M, N)
    A, W = workloads.random_case(M + 5 * K + N, M, K, N, a_scale=40.0)
    note(f"xsplit {M}x{K}x{N}")
    y, launches = linear(A, W)
    # one launch; [K, N] weights with N % 8 != 0 are first copied into rows of
    # N rounded up to 8 (one more launch)
    want = 1 + (N % 8 != 0)
    assert launches in (None, want), f"{launches} launches, not {want}"
    y2 = two_launch(A, W)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not the bits of split + GEMM"
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, f"xsplit {M}x{K}x{N}")
    _, ch, _ = oracle.linear_cf32(A, W)
    assert_better_than_single(y, ch, y64, abs64, f"xsplit {M}x{K}x{N}")
    y3, _ = linear(A, W)
    assert np.array_equal(y.view(np.uint32), y3.view(np.uint32)), "not deterministic"


def test_xsplit_qkv_workload_and_layouts():
    """The QKV workload: [K, N] and [N, K] weights give the same bits in one
    launch each; a bias is one more FP32 addition."""
    wl = workloads.qkv_projection()
    A, W = wl.A[0], wl.W
    N = W.shape[1]
    note("xsplit qkv workload")
    y, launches = linear(A, W)
    assert launches in (None, 1)
    y_nk, launches_nk = linear(A, W, layout=cf.W_NK)
    assert launches_nk in (None, 1)
    assert np.array_equal(y.view(np.uint32), y_nk.view(np.uint32)), "[N, K] and [K, N] differ"
    bias = np.random.default_rng(3).standard_normal(N).astype(np.float32)
    yb, _ = linear(A, W, bias=bias)
    assert np.array_equal(yb.view(np.uint32), (y + bias[None, :]).astype(np.float32).view(np.uint32))
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, "qkv")


@pytest.mark.parametrize("M", [33, 64])
def test_batched_decode_rows_one_launch(M):
    """Batched decode from 33 to 64 rows against [4096, 14336] weights: 224
    tiles of 32 x 128 (192 to 256, K <= 4096), so K is not split and the projection is
    one launch in either layout, with the bits of split + GEMM and of the
    other layout, within tolerance of FP64 and below the single-FP16 error."""
    K, N = 4096, 14336
    assert 192 <= ((M + 31) // 32) * ((N + 127) // 128) <= 256
    A, W = workloads.random_case(M * 13 + 1, M, K, N, a_scale=20.0)
    note(f"batched decode one launch {M}x{K}x{N}")
    y, launches = linear(A, W)
    assert launches in (None, 1), f"{launches} launches"
    y_nk, launches_nk = linear(A, W, layout=cf.W_NK)
    assert launches_nk in (None, 1), f"[N, K]: {launches_nk} launches"
    assert np.array_equal(y.view(np.uint32), y_nk.view(np.uint32)), "[N, K] and [K, N] differ"
    assert np.array_equal(y.view(np.uint32), two_launch(A, W).view(np.uint32)), "not the bits of split + GEMM"
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, f"batched decode {M}x{K}x{N}")
    _, ch, _ = oracle.linear_cf32(A[:8], W)
    assert_better_than_single(y[:8], ch, y64[:8], abs64[:8], f"batched decode {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N,ldx", [(512, 100, 2304, 100), (520, 1003, 2304, 1004), (600, 7, 2000, 8)])
def test_xsplit_k_not_multiple_of_8(M, K, N, ldx):
    """K % 8 != 0 (or K < 64: only a ragged stage), rows padded to a multiple
    of 4 floats so that they stay 16-byte aligned: one launch, the bits of
    split + GEMM."""
    assert small_tile_grid(M, N)
    A, W = workloads.random_case(M * 3 + K + N, M, K, N, a_scale=20.0)
    note(f"xsplit ragged K {M}x{K}x{N} ldx={ldx}")
    y, launches = linear(A, W, ldx=ldx)
    assert launches in (None, 1), f"{launches} launches"
    y2 = two_launch(A, W)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not the bits of split + GEMM"
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, f"xsplit {M}x{K}x{N}")


def test_xsplit_unaligned_rows_fall_back():
    """Rows of x 4-byte but not 16-byte aligned (ldx % 4 != 0): split +
    GEMM (two launches), the same bits."""
    M, K, N = 512, 768, 2304
    A, W = workloads.random_case(77, M, K, N, a_scale=4.0)
    note("xsplit unaligned ldx")
    y, launches = linear(A, W, ldx=K + 1)
    assert launches in (None, 2)
    y2, _ = linear(A, W)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
