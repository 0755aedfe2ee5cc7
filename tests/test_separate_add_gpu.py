"""GPU tests of cfp32_gemm_separate_add, the separate-addition accumulation
mode of the laya.cpp Vulkan guide's AMD path (compensated-FP32 paragraph:
tile results are added to the running sums with separate FP32 additions).

For every mode (0 = plain accumulation in the same kernel configuration,
16 / 64 / 256 = depth of K per separate addition):
  * y within 1e-5 * sum|a w| of the FP64 reference, and measurably below the
    single-FP16 product C_hi;
  * y equals the FP32 merge of the C_hi, C_lo the same call writes;
  * repeated calls give identical bits;
  * the drift case (one large leading term, many small ones, K = 8192) stays
    within twice the error of sequential FP32 accumulation.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import (assert_better_than_single, assert_within_tolerance, note, rel_errors, stream_handle,
                         to_dev, to_host)

pytestmark = pytest.mark.gpu

MODES = [0, 16, 64, 256]


def run_separate_add(A, W, k_per_add, a_offset=0, w_offset=0):
    """Split A on the GPU, then the separate-addition GEMM writing y, C_hi and
    C_lo.  *_offset shift the operands by whole elements inside a larger
    buffer (unaligned pointers and leading dimensions)."""
    M, K = A.shape
    N = W.shape[1]
    hi_t, lo_t = cf.split(to_dev(A))
    lda = K + a_offset
    buf_a = torch.zeros((2, M * lda + a_offset), dtype=torch.int16, device="cuda")
    if K:
        buf_a[0, a_offset:a_offset + M * lda].view(M, lda)[:, :K] = hi_t.view(torch.int16)
        buf_a[1, a_offset:a_offset + M * lda].view(M, lda)[:, :K] = lo_t.view(torch.int16)
    ldw = N + w_offset
    buf_w = np.zeros(K * ldw + w_offset, np.uint16)
    buf_w[w_offset:].reshape(K, ldw)[:, :N] = W.view(np.uint16)
    dw = to_dev(buf_w)
    y = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    ch = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    cl = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    st = cf.cfp32_gemm_separate_add(buf_a.data_ptr() + 2 * a_offset,
                                    buf_a.data_ptr() + buf_a.stride(0) * 2 + 2 * a_offset, lda,
                                    dw.data_ptr() + 2 * w_offset, ldw, y.data_ptr(), ch.data_ptr(), cl.data_ptr(),
                                    N, M, N, K, k_per_add, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    return to_host(y), to_host(ch), to_host(cl)


@pytest.mark.parametrize("k_per_add", MODES)
@pytest.mark.parametrize("name", ["single_linear", "qkv_projection", "unaligned"])
def test_separate_add_workloads(name, k_per_add):
    wl = workloads.ALL[name]()
    A, W = wl.A[0], wl.W
    note(f"separate add {name} k_per_add={k_per_add}")
    y, ch, cl = run_separate_add(A, W, k_per_add)
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, f"{name} k_per_add={k_per_add}")
    assert_better_than_single(y, ch, y64, abs64, name)
    assert np.array_equal(oracle.merge(ch, cl).view(np.uint32), y.view(np.uint32))
    y2, _, _ = run_separate_add(A, W, k_per_add)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"


@pytest.mark.parametrize("k_per_add", MODES)
def test_separate_add_edges(k_per_add):
    """Ragged M, N, K (K not a multiple of 16, 64 or 256), unaligned operands."""
    for M, K, N, a_off, w_off in [(1, 15, 1, 0, 0), (65, 300, 129, 1, 3), (130, 1000, 257, 0, 0), (7, 64, 33, 2, 1)]:
        A, W = workloads.random_case(M * 7 + K + N, M, K, N, a_scale=50.0)
        note(f"separate add edge M={M} K={K} N={N} k_per_add={k_per_add}")
        y, ch, cl = run_separate_add(A, W, k_per_add, a_offset=a_off, w_offset=w_off)
        y64, abs64 = oracle.y64(A, W)
        assert_within_tolerance(y, y64, abs64, f"edge {M}x{K}x{N}")
        assert np.array_equal(oracle.merge(ch, cl).view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("k_per_add", MODES)
def test_separate_add_k_zero(k_per_add):
    note(f"separate add K=0 k_per_add={k_per_add}")
    y = torch.full((5, 9), 2.0, dtype=torch.float32, device="cuda")
    st = cf.cfp32_gemm_separate_add(None, None, 0, None, 9, y.data_ptr(), None, None, 9, 5, 9, 0, k_per_add,
                                    stream_handle())
    assert st == cf.OK
    assert (to_host(y) == 0).all()


@pytest.mark.parametrize("k_per_add", MODES)
def test_separate_add_drift(k_per_add):
    """The guide's drift case: one large leading term and many small ones."""
    M, N, K = 32, 32, 8192
    rng = np.random.default_rng(2)
    A = (rng.uniform(0.5, 1.0, (M, K)) * 2.0 ** -10).astype(np.float32)
    A[:, 0] = 1024.0
    W = np.full((K, N), 0.5, np.float16)
    W[:, ::2] = np.float16(0.25)
    note(f"separate add drift k_per_add={k_per_add}")
    y, _, _ = run_separate_add(A, W, k_per_add)
    y64, abs64 = oracle.y64(A, W)
    gmax, _ = rel_errors(y, y64, abs64)
    ycpu, _, _ = oracle.linear_cf32(A, W)
    cmax, _ = rel_errors(ycpu, y64, abs64)
    note(f"drift k_per_add={k_per_add}: gpu max rel err {gmax:.3g}, sequential fp32 {cmax:.3g}")
    assert gmax <= 2 * cmax + 1e-7
