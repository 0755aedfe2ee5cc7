"""GPU tests of cfp32_linear_ex: the projection with a bias and with the
weights in either layout ([K, N], or [N, K] as torch.nn.Linear stores them).

  * bias: y(bias) equals fl32(y(no bias) + bias) bit for bit on every path
    (small-M chunked, small-M single chunk, small-M [N, K], the split-inside
    GEMM, split + GEMM, the generic GEMM, K = 0), since the bias is one FP32
    addition after the merge;
  * [N, K] weights, M > 32: the same tiles, operands and k order as [K, N],
    so bit-identical to the [K, N] call on the transposed weights;
  * [N, K] weights, M <= 32: a different kernel (each block streams 64 whole
    W rows through LDS in 1 KiB pieces of K, the waves' sums added in wave
    order), checked against the FP64 reference and for determinism;
  * [K, N] without a bias is exactly cfp32_linear.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import assert_better_than_single, assert_within_tolerance, check_all_rows, note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_ex(A, W, layout, bias=None, w_offset=0, w_ld_pad=0, x_pad=0):
    """cfp32_linear_ex on A FP32 [M, K] and W FP16 [K, N] given in `layout`
    (transposed to [N, K] for W_NK), optionally shifted / padded in memory."""
    M, K = A.shape
    N = W.shape[1]
    xb = np.zeros((M, K + x_pad), np.float32)
    xb[:, :K] = A
    Wl = W if layout == cf.W_KN else np.ascontiguousarray(W.T)
    rows, cols = Wl.shape
    ldw = cols + w_offset + w_ld_pad
    wb = np.zeros(rows * ldw + w_offset, np.uint16)
    wb[w_offset:].reshape(rows, ldw)[:, :cols] = Wl.view(np.uint16)
    dx, dw = to_dev(xb), to_dev(wb)
    db = to_dev(bias) if bias is not None else None
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, layout)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    st = cf.cfp32_linear_ex(dx.data_ptr(), K + x_pad, dw.data_ptr() + 2 * w_offset, ldw, layout,
                            db.data_ptr() if db is not None else None, y.data_ptr(), N, M, N, K,
                            ws.data_ptr() if need else None, need, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    return to_host(y)


# (M, K, N): small-M chunked, small-M one chunk, M = 8, generic GEMM (small
# grid), split inside the GEMM (N <= 4096, >= 128 tiles), split + DMA GEMM.
SHAPES = [(1, 4096, 1536), (3, 20, 700), (8, 1000, 520), (40, 256, 300), (8192, 512, 512), (2048, 1024, 4608)]


@pytest.mark.parametrize("layout", [cf.W_KN, cf.W_NK])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_bias_is_one_fp32_addition(M, K, N, layout):
    A, W = workloads.random_case(M + 3 * K + N, M, K, N, a_scale=20.0)
    bias = (np.random.default_rng(N).standard_normal(N) * 3.0).astype(np.float32)
    note(f"linear_ex bias {M}x{K}x{N} layout={layout}")
    y0 = run_ex(A, W, layout)
    y1 = run_ex(A, W, layout, bias)
    assert np.array_equal(y1.view(np.uint32), (y0 + bias[None, :]).astype(np.float32).view(np.uint32))
    rows = np.arange(M)
    y64, abs64 = oracle.y64(A[rows], W)
    assert_within_tolerance(y0[rows], y64, abs64, f"{M}x{K}x{N} layout={layout}")


def test_bias_with_k_zero():
    for M in (2, 20):
        bias = np.array([1.5, -0.0, 3.25, -2.0, 0.0], np.float32)
        note(f"linear_ex K=0 bias M={M}")
        y = torch.full((M, 5), 9.0, dtype=torch.float32, device="cuda")
        db = to_dev(bias)
        st = cf.cfp32_linear_ex(None, 0, None, 5, cf.W_KN, db.data_ptr(), y.data_ptr(), 5, M, 5, 0, None, 0,
                                stream_handle())
        assert st == cf.OK
        expect = (np.zeros(5, np.float32) + bias).astype(np.float32)  # +0 + b
        assert np.array_equal(to_host(y).view(np.uint32), np.broadcast_to(expect, (M, 5)).view(np.uint32))


@pytest.mark.parametrize("M,K,N", [(40, 256, 300), (8192, 512, 512), (2048, 1024, 4608), (300, 1000, 777),
                                   (4100, 64, 8200)])
def test_nk_matches_kn_bitwise_above_32_rows(M, K, N):
    """M > 32: [N, K] weights reach the same tiles with the same k order."""
    A, W = workloads.random_case(M * 5 + K + N, M, K, N, a_scale=10.0)
    note(f"linear_ex nk vs kn {M}x{K}x{N}")
    y_kn = run_ex(A, W, cf.W_KN)
    y_nk = run_ex(A, W, cf.W_NK)
    assert np.array_equal(y_kn.view(np.uint32), y_nk.view(np.uint32))


def test_nk_ffn_prefill_full_size_matches_kn():
    """The FFN projection 8192 x 4096 x 14336 with the weights in both
    layouts (the [N, K] GEMM with 64-deep W stages, as bench.py times it):
    the same bits everywhere, and every element within tolerance of the FP64
    reference."""
    wl = workloads.decode_ffn_pair()
    A, W = wl.A[1], wl.W
    M, K = A.shape
    N = W.shape[1]
    note("linear_ex nk vs kn 8192x4096x14336")
    dx = to_dev(A)
    dw_kn = to_dev(W.view(np.uint16))
    dw_nk = dw_kn.view(K, N).t().contiguous()
    outs = []
    for layout, dw, ldw in ((cf.W_KN, dw_kn, N), (cf.W_NK, dw_nk, K)):
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, layout)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        st = cf.cfp32_linear_ex(dx.data_ptr(), K, dw.data_ptr(), ldw, layout, None, y.data_ptr(), N, M, N, K,
                                ws.data_ptr(), need, stream_handle())
        assert st == cf.OK, cf.cfp32_status_string(st)
        torch.cuda.synchronize()
        outs.append(y)
        del ws
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32)), "[N, K] and [K, N] differ"
    check_all_rows(A, W, to_host(outs[1]), None, "nk ffn prefill")


@pytest.mark.parametrize("M", list(range(1, 18)) + [23, 24, 25, 31, 32])
def test_nk_small_m(M):
    """M <= 32 with [N, K] weights.  The LDS-DMA kernel (48, 56 or 64 W rows
    per block, 1 KiB pieces of K; one, two or four groups of 8 rows of x):
    the full decode shape (56-row blocks), K below one piece (down to one
    granule), exactly one piece, a ragged last piece, an odd number of pieces
    with a padded row stride, 16 pieces, N with a partial last block (down to
    one row), and partial last blocks of 56, 48 and 64 rows.  K % 8 != 0 and unaligned weights
    take the generic kernel (M <= 8) or the GEMM path."""
    cases = [(4096, 14336, 0, 0), (1000, 777, 0, 0), (256, 100, 0, 0), (512, 65, 0, 0), (1536, 130, 0, 8),
             (8192, 200, 0, 0), (8, 1, 0, 0), (16, 3, 0, 0), (1001, 64, 0, 0), (64, 33, 1, 0), (8, 1, 0, 3),
             (96, 520, 0, 5), (1024, 13000, 0, 0), (520, 10300, 0, 0), (264, 15999, 0, 0)]
    for K, N, w_off, w_pad in cases:
        A, W = workloads.random_case(M * 100 + K + N, M, K, N, a_scale=30.0)
        note(f"linear_ex nk small M={M} K={K} N={N} w_off={w_off} w_pad={w_pad}")
        y = run_ex(A, W, cf.W_NK, w_offset=w_off, w_ld_pad=w_pad)
        y64, abs64 = oracle.y64(A, W)
        assert_within_tolerance(y, y64, abs64, f"nk M={M} K={K} N={N}")
        # "measurably below a single FP16 conversion": this kernel does not
        # expose its C_hi, so the oracle's FP32 C_hi of the same inputs is
        # the single-conversion product
        _, ch, _ = oracle.linear_cf32(A, W)
        assert_better_than_single(y, ch, y64, abs64, f"nk M={M} K={K} N={N}")
        y2 = run_ex(A, W, cf.W_NK, w_offset=w_off, w_ld_pad=w_pad)
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"


def test_ex_without_bias_is_linear():
    A, W = workloads.random_case(5, 333, 1000, 777)
    note("linear_ex == linear")
    y_ex = run_ex(A, W, cf.W_KN)
    y = cf.linear(to_dev(A), to_dev(W).view(torch.float16))
    assert np.array_equal(y_ex.view(np.uint32), to_host(y).view(np.uint32))


def test_tensor_helper_nn_linear_layout():
    """cf.linear(x, weight, bias=b, w_layout='nk') with an nn.Linear-shaped weight."""
    A, W = workloads.random_case(6, 4, 512, 384)
    bias = np.linspace(-1, 1, 384, dtype=np.float32)
    note("linear helper nk + bias")
    weight = to_dev(np.ascontiguousarray(W.T)).view(torch.float16)  # [N, K]
    y = to_host(cf.linear(to_dev(A), weight, bias=to_dev(bias), w_layout="nk"))
    y64, abs64 = oracle.y64(A, W)
    y0 = run_ex(A, W, cf.W_NK)
    assert np.array_equal(y.view(np.uint32), (y0 + bias[None, :]).astype(np.float32).view(np.uint32))
    assert_within_tolerance(y0, y64, abs64, "helper nk")
