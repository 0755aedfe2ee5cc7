"""GPU tests at the largest operand extents: every operand placed so that the
byte offset of its last row passes 2^32.

The fast kernels address their operands through raw buffer loads with 32-bit
offsets; operands that reach further must go to the kernels that form 64-bit
addresses (the generic GEMM tiles, the generic small-M kernels), and the
split and merge kernels must form 64-bit row offsets.  Each operand here is
a few rows at a large leading dimension inside a zero-filled allocation of a
few GiB, so the computation stays small:
  * split planes bit-exact against the oracle's split, merge bit-exact
    against the oracle's merge;
  * projections within 1e-5 * sum|a w| of the FP64 reference, every element;
  * GEGLU within the FP32 GELU rounding of the oracle's GEGLU of the
    projection the same operands give.
The split also runs with more rows than one grid dimension holds (65535).
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import assert_within_tolerance, note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu

PAST_32 = 1 << 32


def ld_past_32(rows: int, itemsize: int, at_least: int) -> int:
    """A leading dimension (multiple of 8, >= at_least) at which row rows-1
    starts past 2^32 bytes."""
    ld = PAST_32 // (itemsize * (rows - 1)) + 8
    ld = max(ld, at_least)
    return (ld + 7) // 8 * 8


def placed(a: np.ndarray, ld: int) -> torch.Tensor:
    """A zero-filled device buffer [rows, ld] holding a in its first columns."""
    dt = torch.float32 if a.dtype == np.float32 else torch.int16
    buf = torch.zeros((a.shape[0], ld), dtype=dt, device="cuda")
    buf[:, :a.shape[1]].copy_(to_dev(a))
    return buf


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sampled(M: int) -> np.ndarray:
    """Every row: the cases here are small enough for a full FP64 check."""
    return np.arange(M)


@pytest.mark.parametrize("cols", [1000, 999])
def test_split_and_merge_rows_past_32bit_offsets(cols):
    rows = 5
    x = workloads.random_case(cols, rows, cols, 1)[0] * np.float32(300.0)
    ldx, ldh = ld_past_32(rows, 4, cols), ld_past_32(rows, 2, cols)
    note(f"split rows={rows} cols={cols} ldx={ldx} ldh={ldh}")
    dx = placed(x, ldx)
    hi = torch.zeros((rows, ldh), dtype=torch.int16, device="cuda")
    lo = torch.zeros((rows, ldh), dtype=torch.int16, device="cuda")
    st = cf.cfp32_split(dx.data_ptr(), ldx, hi.data_ptr(), lo.data_ptr(), ldh, rows, cols, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    want_hi, want_lo = oracle.split(x)
    assert np.array_equal(to_host(hi[:, :cols].contiguous()).view(np.uint16), want_hi)
    assert np.array_equal(to_host(lo[:, :cols].contiguous()).view(np.uint16), want_lo)
    del dx, hi, lo
    free()

    rng = np.random.default_rng(cols + 1)
    ch = (rng.standard_normal((rows, cols)) * 100).astype(np.float32)
    cl = (rng.standard_normal((rows, cols)) * 100).astype(np.float32)
    ldc = ld_past_32(rows, 4, cols)
    note(f"merge rows={rows} cols={cols} ldc={ldc}")
    dch, dcl = placed(ch, ldc), placed(cl, ldc)
    y = torch.full((rows, cols), 7.0, dtype=torch.float32, device="cuda")
    st = cf.cfp32_merge(dch.data_ptr(), dcl.data_ptr(), ldc, y.data_ptr(), cols, rows, cols, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    assert np.array_equal(to_host(y).view(np.uint32), oracle.merge(ch, cl).view(np.uint32))
    del dch, dcl, y
    free()


@pytest.mark.parametrize("cols", [16, 13])
def test_split_more_rows_than_one_grid_dimension(cols):
    rows = 70001
    x = workloads.random_case(rows + cols, rows, cols, 1)[0]
    note(f"split rows={rows} cols={cols}")
    hi = torch.empty((rows, cols), dtype=torch.int16, device="cuda")
    lo = torch.empty((rows, cols), dtype=torch.int16, device="cuda")
    dx = to_dev(x)
    st = cf.cfp32_split(dx.data_ptr(), cols, hi.data_ptr(), lo.data_ptr(), cols, rows, cols, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    want_hi, want_lo = oracle.split(x)
    assert np.array_equal(to_host(hi).view(np.uint16), want_hi)
    assert np.array_equal(to_host(lo).view(np.uint16), want_lo)


@pytest.mark.parametrize("far", ["planes", "weights"])
def test_gemm_operands_past_32bit_offsets(far):
    """1024 x 6144 outputs: 192 tiles of 128 x 256, so the LDS-DMA kernel is
    tried first and must decline the far operand."""
    M, K, N = 1024, 520, 6144
    A, W = workloads.random_case(M + (far == "weights"), M, K, N, a_scale=4.0)
    hi, lo = oracle.split(A)
    lda = ld_past_32(M, 2, K) if far == "planes" else K
    ldw = ld_past_32(K, 2, N) if far == "weights" else N
    note(f"gemm {M}x{N}x{K} far={far} lda={lda} ldw={ldw}")
    dhi, dlo, dw = placed(hi, lda), placed(lo, lda), placed(W.view(np.uint16), ldw)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    st = cf.cfp32_gemm(dhi.data_ptr(), dlo.data_ptr(), lda, dw.data_ptr(), ldw, y.data_ptr(), None, None, N,
                       M, N, K, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    rows = sampled(M)
    got = to_host(y)[rows]
    del dhi, dlo, dw, y
    free()
    y64, abs64 = oracle.y64(A[rows], W)
    assert_within_tolerance(got, y64, abs64, f"gemm far {far}")


def run_linear_ex(A, W, layout, ldx, ldw, bias=None):
    """cfp32_linear_ex with x at leading dimension ldx and W (given [K, N];
    transposed for W_NK) at leading dimension ldw."""
    M, K = A.shape
    N = W.shape[1]
    Wl = W if layout == cf.W_KN else np.ascontiguousarray(W.T)
    dx, dw = placed(A, ldx), placed(Wl.view(np.uint16), ldw)
    db = to_dev(bias) if bias is not None else None
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, layout)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    st = cf.cfp32_linear_ex(dx.data_ptr(), ldx, dw.data_ptr(), ldw, layout,
                            db.data_ptr() if db is not None else None, y.data_ptr(), N, M, N, K,
                            ws.data_ptr() if need else None, need, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    out = to_host(y)
    del dx, dw, db, y, ws
    free()
    return out


# M = 1 and 5 take the small-M paths, 12 the two-group small-M dispatch (which
# declines) and then split K, 40 split K over the GEMM tiles.
@pytest.mark.parametrize("layout", [cf.W_KN, cf.W_NK])
@pytest.mark.parametrize("M", [1, 5, 12, 40])
def test_linear_weights_past_32bit_offsets(M, layout):
    K, N = 1104, 600
    A, W = workloads.random_case(M * 11 + layout, M, K, N, a_scale=8.0)
    bias = (np.random.default_rng(M).standard_normal(N) * 0.5).astype(np.float32)
    rows_w = K if layout == cf.W_KN else N
    ldw = ld_past_32(rows_w, 2, N if layout == cf.W_KN else K)
    note(f"linear_ex weights far M={M} layout={layout} ldw={ldw}")
    y = run_linear_ex(A, W, layout, K, ldw, bias)
    y64, abs64 = oracle.y64(A, W)
    # The bias adds one more FP32 rounding (at most 2^-24 |y|).
    y64 = y64 + bias.astype(np.float64)
    abs64 = abs64 + np.abs(y64) * 1e-2
    assert_within_tolerance(y, y64, abs64, f"weights far M={M} layout={layout}")


# M = 5: the small-M path declines buffer loads of x; 300: split + generic
# GEMM; 4096 x 2048: the split-inside GEMM is tried first and declines, then
# split + LDS-DMA GEMM on the compact planes.
@pytest.mark.parametrize("M,K,N", [(5, 1000, 520), (12, 1000, 520), (300, 1000, 512), (4096, 1000, 2048)])
def test_linear_activations_past_32bit_offsets(M, K, N):
    A, W = workloads.random_case(M + K + N, M, K, N, a_scale=8.0)
    ldx = ld_past_32(M, 4, K)
    note(f"linear activations far {M}x{K}x{N} ldx={ldx}")
    y = run_linear_ex(A, W, cf.W_KN, ldx, N)
    rows = sampled(M)
    y64, abs64 = oracle.y64(A[rows], W)
    assert_within_tolerance(y[rows], y64, abs64, f"activations far {M}x{K}x{N}")


@pytest.mark.parametrize("M", [1, 40])
def test_geglu_weights_past_32bit_offsets(M):
    K, F = 1104, 300
    A, W = workloads.random_case(M * 5 + 3, M, K, 2 * F, a_scale=8.0)
    ldw = ld_past_32(K, 2, 2 * F)
    note(f"geglu weights far M={M} ldw={ldw}")
    dx, dw = to_dev(A), placed(W.view(np.uint16), ldw)
    out = torch.full((M, F), 5.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_geglu_workspace_bytes(M, F, K)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    st = cf.cfp32_linear_geglu(dx.data_ptr(), K, dw.data_ptr(), ldw, None, out.data_ptr(), F, M, F, K,
                               ws.data_ptr() if need else None, need, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    got = to_host(out)
    del dx, dw, out, ws
    free()
    y_full = run_linear_ex(A, W, cf.W_KN, K, ldw)
    gate, up = y_full[:, :F], y_full[:, F:]
    ref = oracle.geglu64(gate, up)
    bound = 2e-6 * np.abs(gate.astype(np.float64) * up.astype(np.float64)) + 1e-37
    assert np.isfinite(got).all()
    assert (np.abs(got.astype(np.float64) - ref) <= bound).all(), f"geglu far M={M}"
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y_full, y64, abs64, f"geglu projection far M={M}")
