"""GPU tests of cfp32_linear_geglu: the feed-forward projection with its GEGLU
fused (laya.cpp Vulkan guide, graph paragraph): out = gelu(gate) * up with
gate = x W[:, :F] (+ b[:F]) and up = x W[:, F:] (+ b[F:]).

gate and up are the projection's merged outputs: every path multiplies the
same split operands in the same k order as cfp32_linear_ex over the full
[K, 2F] weight.  So the reference is the oracle's GEGLU (exact GELU, double)
applied to those FP32 columns, and the kernel may differ from it only by its
FP32 GELU rounding: |out - ref| <= 2e-6 * |gate * up| (erff and four FP32
roundings, about 32 ulp, with the scale of gelu(gate) * up bounded by
|gate * up|).  The full-width projection itself is checked against the FP64
reference on every row, which ties the chain to the pinned oracle.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import assert_within_tolerance, check_all_rows, note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu

GELU_TOL = 2e-6


def run_geglu(A, W, bias=None, w_offset=0):
    M, K = A.shape
    F = W.shape[1] // 2
    ldw = 2 * F + w_offset
    wb = np.zeros(K * ldw + w_offset, np.uint16)
    wb[w_offset:].reshape(K, ldw)[:, :2 * F] = W.view(np.uint16)
    dx, dw = to_dev(A), to_dev(wb)
    db = to_dev(bias) if bias is not None else None
    out = torch.full((M, F), 5.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_geglu_workspace_bytes(M, F, K)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    st = cf.cfp32_linear_geglu(dx.data_ptr(), K, dw.data_ptr() + 2 * w_offset, ldw,
                               db.data_ptr() if db is not None else None, out.data_ptr(), F, M, F, K,
                               ws.data_ptr() if need else None, need, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    return to_host(out)


def full_projection(A, W, bias=None, w_offset=0):
    """cfp32_linear_ex over the whole [K, 2F] weight (gate | up columns), with
    W placed in memory as run_geglu places it (so that the same kernels, and
    summation orders, serve both)."""
    M, K = A.shape
    N = W.shape[1]
    ldw = N + w_offset
    wb = np.zeros(K * ldw + w_offset, np.uint16)
    wb[w_offset:].reshape(K, ldw)[:, :N] = W.view(np.uint16)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_ex_workspace_bytes(M, N, K, cf.W_KN)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    dx, dw = to_dev(A), to_dev(wb)
    db = to_dev(bias) if bias is not None else None
    st = cf.cfp32_linear_ex(dx.data_ptr(), K, dw.data_ptr() + 2 * w_offset, ldw, cf.W_KN,
                            db.data_ptr() if db is not None else None, y.data_ptr(), N, M, N, K,
                            ws.data_ptr() if need else None, need, stream_handle())
    assert st == cf.OK
    return to_host(y)


def check_geglu(out, y_full, F, what):
    gate, up = y_full[:, :F], y_full[:, F:]
    ref = oracle.geglu64(gate, up)
    err = np.abs(out.astype(np.float64) - ref)
    bound = GELU_TOL * np.abs(gate.astype(np.float64) * up.astype(np.float64)) + 1e-37
    assert np.isfinite(out).all(), what
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs off; worst {err[bad].max():.3g}"


# (M, K, F): small-M chunked; small-M with one stage (partials still used);
# M = 8; two groups of 8 rows in the small-M dispatch; M > 8 small grid with
# K too short to split (two-pass fallback); split K over all 2F columns with
# the GEGLU merge; the fused GEMM epilogue (>= 256 tiles of 128 x 128,
# ragged F and M).
SHAPES = [(1, 4096, 1536), (3, 24, 40), (8, 1000, 520), (13, 2048, 1000), (40, 256, 300), (48, 2048, 2000),
          (2100, 512, 2000)]


@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("M,K,F", SHAPES)
def test_geglu_paths(M, K, F, with_bias):
    A, W = workloads.random_case(M + K + 7 * F, M, K, 2 * F, a_scale=8.0)
    bias = (np.random.default_rng(F).standard_normal(2 * F) * 0.5).astype(np.float32) if with_bias else None
    note(f"geglu {M}x{K}x{F} bias={with_bias}")
    out = run_geglu(A, W, bias)
    y_full = full_projection(A, W, bias)
    check_geglu(out, y_full, F, f"{M}x{K}x{F}")
    out2 = run_geglu(A, W, bias)
    assert np.array_equal(out.view(np.uint32), out2.view(np.uint32)), "not deterministic"
    rows = np.arange(M)
    y64, abs64 = oracle.y64(A[rows], W)
    if bias is not None:
        # The bias addition rounds once more, by at most 2^-24 |y|; widen the
        # bound by 1e-5 * 0.01 |y| = 1e-7 |y| for it.
        y64 = y64 + bias.astype(np.float64)
        abs64 = abs64 + np.abs(y64) * 1e-2
    assert_within_tolerance(y_full[rows], y64, abs64, f"projection {M}x{K}x{F}")


@pytest.mark.parametrize("M", [2, 12, 40])
def test_geglu_unaligned_weight_fallback(M):
    K, F = 200, 96
    A, W = workloads.random_case(M * 3, M, K, 2 * F, a_scale=8.0)
    note(f"geglu unaligned M={M}")
    out = run_geglu(A, W, w_offset=1)
    check_geglu(out, full_projection(A, W, w_offset=1), F, f"unaligned M={M}")


def test_geglu_ffn_prefill_full_size():
    """The FFN shape: x [8192, 4096], W [4096, 14336] as gate | up (F = 7168),
    the fused GEMM epilogue: every output against the oracle's GEGLU of the
    projection's gate and up columns, and every projection output against
    the FP64 reference."""
    wl = workloads.decode_ffn_pair()
    A, W = wl.A[1], wl.W
    F = W.shape[1] // 2
    note("geglu ffn prefill 8192x4096x7168")
    out = run_geglu(A, W)
    y_full = full_projection(A, W)
    check_geglu(out, y_full, F, "ffn prefill")
    check_all_rows(A, W, y_full, None, "ffn prefill projection")


def test_geglu_k_zero():
    bias = np.array([0.5, -1.0, 2.0, 3.0, -0.25, 4.0], np.float32)  # gate 3 | up 3
    for M in (2, 20):
        note(f"geglu K=0 M={M}")
        out = torch.full((M, 3), 9.0, dtype=torch.float32, device="cuda")
        db = to_dev(bias)
        st = cf.cfp32_linear_geglu(None, 0, None, 6, db.data_ptr(), out.data_ptr(), 3, M, 3, 0, None, 0,
                                   stream_handle())
        assert st == cf.OK
        ref = oracle.geglu64(bias[:3], bias[3:])
        got = to_host(out)
        assert np.allclose(got, np.broadcast_to(ref, (M, 3)), rtol=GELU_TOL, atol=1e-7)


def test_geglu_tensor_helper():
    A, W = workloads.random_case(11, 5, 128, 64)
    note("geglu helper")
    out = to_host(cf.linear_geglu(to_dev(A), to_dev(W).view(torch.float16)))
    check_geglu(out, full_projection(A, W), 32, "helper")
