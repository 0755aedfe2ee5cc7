"""The true-FP32 projection (cfp32_linear_f32) against the oracle.

The laya.cpp Vulkan guide's true FP32 matrix kernels keep FP32 operands
from being converted to FP16 (true-FP32 paragraph).  Here x stays FP32, W is
widened exactly, and the matrix unit forms FP32 products and sums.  The
oracle's plain FP32 product (fused multiply-adds, k ascending) and the FP64
reference bound it:
  * every output within 1e-5 * sum|a w| of FP64 (the benchmark spec's tolerance,
    which FP32 accumulation meets on these inputs) and finite;
  * within 2e-5 * sum|a w| of the oracle's FP32 product (two FP32
    accumulations in different orders, each within the bound above);
  * without the FP16 conversion of x: on the workloads whose activations
    lose bits in one FP16 rounding, its error is far below the single-FP16
    product's (the oracle's C_hi);
  * repeatable bits; any M, N, K including ragged tiles, K = 0 and operands
    that are not 16-byte aligned.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import (RATIO, assert_within_tolerance, check_all_rows, note, rel_errors, stream_handle, to_dev,
                         to_host)

pytestmark = pytest.mark.gpu


def run_f32(A, W, x_pad=0, w_offset=0, y_pad=0):
    M, K = A.shape
    N = W.shape[1]
    xb = np.zeros((M, K + x_pad), np.float32)
    xb[:, :K] = A
    ldw = N + w_offset
    wb = np.zeros(K * ldw + w_offset, np.uint16)
    wb[w_offset:].reshape(K, ldw)[:, :N] = W.view(np.uint16)
    dx, dw = to_dev(xb), to_dev(wb)
    y = torch.full((M, N + y_pad), 5.0, dtype=torch.float32, device="cuda")
    st = cf.cfp32_linear_f32(dx.data_ptr(), K + x_pad, dw.data_ptr() + 2 * w_offset, ldw, y.data_ptr(), N + y_pad,
                             M, N, K, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    out = to_host(y)
    if y_pad:
        assert (out[:, N:] == 5.0).all(), "padding columns were written"
    return np.ascontiguousarray(out[:, :N])


@pytest.mark.parametrize("name", ["single_linear", "qkv_projection", "unaligned", "square"])
def test_linear_f32_workloads(name):
    wl = workloads.ALL[name]()
    A, W = wl.A[0], wl.W
    note(f"linear_f32 workload {name}")
    y = run_f32(A, W)
    ymax, yrms, _, _ = check_all_rows(A, W, y, None, f"f32 {name}")
    if A.shape[0] <= 512:
        yf = oracle.linear_f32(A, W)
        y64, abs64 = oracle.y64(A, W)
        assert (np.abs(y.astype(np.float64) - yf) <= 2e-5 * abs64).all(), f"{name}: off the oracle's FP32 product"
        _, ch, _ = oracle.linear_cf32(A, W)
        smax, srms = rel_errors(ch, y64, abs64)
        assert ymax * RATIO <= smax and yrms * RATIO <= srms, f"{name}: not below the single-FP16 product"
    y2 = run_f32(A, W)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 14336, 4096), (17, 3, 5), (127, 129, 15), (128, 128, 16),
                                   (129, 257, 17), (300, 777, 1000), (64, 4096, 4096), (1000, 64, 33)])
def test_linear_f32_edge_shapes(M, N, K):
    A, W = workloads.random_case(M + 3 * N + 7 * K, M, K, N, a_scale=10.0)
    note(f"linear_f32 edge {M}x{N}x{K}")
    y = run_f32(A, W, y_pad=3)
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, f"f32 edge {M}x{N}x{K}")


@pytest.mark.parametrize("x_pad,w_offset", [(1, 0), (0, 1), (3, 5)])
def test_linear_f32_unaligned_operands_same_bits(x_pad, w_offset):
    A, W = workloads.random_case(31, 200, 333, 150)
    note(f"linear_f32 unaligned x_pad={x_pad} w_offset={w_offset}")
    y = run_f32(A, W, x_pad=x_pad, w_offset=w_offset)
    y0 = run_f32(A, W)
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))


def test_linear_f32_k_zero():
    note("linear_f32 K=0")
    y = torch.full((40, 50), 9.0, dtype=torch.float32, device="cuda")
    st = cf.cfp32_linear_f32(None, 0, None, 50, y.data_ptr(), 50, 40, 50, 0, stream_handle())
    assert st == cf.OK
    out = to_host(y)
    assert (out == 0).all() and not np.signbit(out).any()


def test_linear_f32_tensor_helper():
    A, W = workloads.random_case(4, 70, 90, 110)
    note("linear_f32 helper")
    y = to_host(cf.linear_f32(to_dev(A), to_dev(W).view(torch.float16)))
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, "f32 helper")
