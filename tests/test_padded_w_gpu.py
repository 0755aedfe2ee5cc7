"""[K, N] weights whose rows do not allow 16-byte loads (N not a multiple of
8, any leading dimension or pointer offset): cfp32_linear first copies W into
the workspace with rows of N rounded up to 8 and then runs the path a
16-byte-aligned W of that width takes.  The copy holds the same values, so
the result must be bit-identical to a call on an aligned W, and within the
tolerance of the FP64 reference (graph paragraph of the laya.cpp Vulkan
guide: every projection of the model goes through the same call, whatever
its shape)."""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import assert_better_than_single, assert_within_tolerance, note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu


def run(A, W, ldw, w_offset):
    """cfp32_linear with W [K, N] stored at element offset w_offset of its
    buffer with leading dimension ldw; the workspace starts as 0xFF bytes."""
    M, K = A.shape
    N = W.shape[1]
    wb = np.full(K * ldw + w_offset + 8, 0x7E00, np.uint16)  # NaN bits outside W: must not be read into y
    wb[w_offset:w_offset + K * ldw].reshape(K, ldw)[:, :N] = W.view(np.uint16)
    dx, dw = to_dev(A), to_dev(wb)
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_workspace_bytes(M, N, K)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    st = cf.cfp32_linear(dx.data_ptr(), K, dw.data_ptr() + 2 * w_offset, ldw, y.data_ptr(), N, M, N, K,
                         ws.data_ptr() if need else None, need, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    return to_host(y)


# (M, K, N): the unaligned workload (333 x 1000 x 777, generic GEMM kernel
# on a small grid); split K with stacked hi/lo tiles (24 rows); the small-M
# dispatches (12 rows); the LDS-DMA GEMM (16 x 12 = 192 tiles of 128 x 256);
# a single column.
SHAPES = [(333, 1000, 777), (24, 2000, 777), (12, 1000, 777), (2048, 128, 3001), (40, 64, 1)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_padded_copy_matches_aligned_weights(M, K, N):
    assert N % 8
    A, W = workloads.random_case(M + 3 * K + 7 * N, M, K, N, a_scale=50.0)
    n8 = (N + 7) // 8 * 8
    note(f"padded W {M}x{K}x{N}: aligned reference")
    ref = run(A, W, ldw=n8, w_offset=0)
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(ref, y64, abs64, f"aligned {M}x{K}x{N}")
    _, ch, _ = oracle.linear_cf32(A[:16], W)
    assert_better_than_single(ref[:16], ch, y64[:16], abs64[:16], f"aligned {M}x{K}x{N}")
    for ldw, off in [(N, 0), (N, 1), (N + 2, 3), (n8, 5)]:
        note(f"padded W {M}x{K}x{N}: ldw {ldw}, offset {off}")
        y = run(A, W, ldw=ldw, w_offset=off)
        assert np.array_equal(y.view(np.uint32), ref.view(np.uint32)), f"ldw {ldw} offset {off}: bits differ"


def test_padded_copy_with_bias_and_nk_unaffected():
    """The copy is only made for [K, N] weights; [N, K] weights with K not a
    multiple of 8 keep their own path (within tolerance), and a bias is still
    one FP32 addition after the merge of the padded-copy path."""
    M, K, N = 100, 300, 333
    A, W = workloads.random_case(4242, M, K, N, a_scale=10.0)
    bias = np.random.default_rng(5).standard_normal(N).astype(np.float32)
    y64, abs64 = oracle.y64(A, W)
    dx, db = to_dev(A), to_dev(bias)
    wb = np.zeros(K * N + 1, np.uint16)
    wb[1:].reshape(K, N)[:] = W.view(np.uint16)
    dw = to_dev(wb)
    need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, cf.W_KN)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    note("padded W with bias")
    st = cf.cfp32_linear_ex(dx.data_ptr(), K, dw.data_ptr() + 2, N, cf.W_KN, db.data_ptr(), out.data_ptr(), N,
                            M, N, K, ws.data_ptr(), need, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    y_bias = to_host(out)
    st = cf.cfp32_linear_ex(dx.data_ptr(), K, dw.data_ptr() + 2, N, cf.W_KN, None, out.data_ptr(), N,
                            M, N, K, ws.data_ptr(), need, stream_handle())
    assert st == cf.OK
    y = to_host(out)
    assert np.array_equal(y_bias.view(np.uint32), (y + bias[None, :]).astype(np.float32).view(np.uint32))
    assert_within_tolerance(y, y64, abs64, "padded W, no bias")
    # [N, K] with K = 300 (ldw % 8 != 0): no copy, the generic kernel
    wt = np.ascontiguousarray(W.T)
    dwt = to_dev(wt)
    need_nk = cf.cfp32_linear_ex_workspace_bytes(M, N, K, cf.W_NK)
    assert need_nk < need  # no room for a W copy
    ws2 = torch.full((need_nk,), 0xFF, dtype=torch.uint8, device="cuda")
    note("[N, K] weights, K = 300")
    st = cf.cfp32_linear_ex(dx.data_ptr(), K, dwt.data_ptr(), K, cf.W_NK, None, out.data_ptr(), N,
                            M, N, K, ws2.data_ptr(), need_nk, stream_handle())
    assert st == cf.OK
    assert_within_tolerance(to_host(out), y64, abs64, "[N, K] K = 300")
