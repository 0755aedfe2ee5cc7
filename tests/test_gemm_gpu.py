"""GPU dual-product GEMM and the whole projection against the oracle.

For every workload and for random shapes that cut every tile edge:
  * y is finite and within 1e-5 * sum|a w| of the FP64 reference;
  * y equals the oracle's FP32 merge of the C_hi, C_lo the same call writes
    (the merge happens once, after both reductions);
  * each product on its own is within FP32-accumulation tolerance of its
    exact value (which also catches swapped or mis-scaled parts);
  * y's error is at least 16x below that of the single-FP16 product C_hi;
  * a repeated call gives identical bits.
At the full 8192 x 4096 x 14336 size every element is checked against the
FP64 reference too (a block of rows at a time), with the 16x ratio against
the same launch's C_hi over the whole output.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import (TOL, assert_better_than_single, assert_within_tolerance, check_all_rows, note,
                         rel_errors, stream_handle, to_dev, to_host)

pytestmark = pytest.mark.gpu


def run_gemm(A, W, want_y=True, want_parts=True, split_on_gpu=True, w_offset=0, a_offset=0, out_pad=0):
    """Split A (GPU kernel, or the oracle's split when split_on_gpu=False) and run
    cfp32_gemm.  *_offset shift the operands inside a larger buffer by whole
    elements (to reach unaligned pointers and leading dimensions)."""
    M, K = A.shape
    N = W.shape[1]
    if split_on_gpu:
        hi_t, lo_t = cf.split(to_dev(A))
        hi = to_host(hi_t).view(np.uint16)
        lo = to_host(lo_t).view(np.uint16)
    else:
        hi, lo = oracle.split(A)
    lda = K + a_offset
    buf_a = np.zeros((2, M * lda + a_offset), np.uint16)
    for p, plane in enumerate((hi, lo)):
        view = buf_a[p, a_offset:a_offset + M * lda].reshape(M, lda)
        view[:, :K] = plane
    ldw = N + w_offset
    buf_w = np.zeros(K * ldw + w_offset, np.uint16)
    buf_w[w_offset:].reshape(K, ldw)[:, :N] = W.view(np.uint16)
    da = to_dev(buf_a)
    dw = to_dev(buf_w)
    ldc = N + out_pad
    y = torch.full((M, ldc), 3.0, dtype=torch.float32, device="cuda") if want_y else None
    ch = torch.full((M, ldc), 3.0, dtype=torch.float32, device="cuda") if want_parts else None
    cl = torch.full((M, ldc), 3.0, dtype=torch.float32, device="cuda") if want_parts else None
    pa_hi = da.data_ptr() + 2 * a_offset
    pa_lo = da.data_ptr() + da.stride(0) * 2 + 2 * a_offset
    st = cf.cfp32_gemm(pa_hi, pa_lo, lda, dw.data_ptr() + 2 * w_offset, ldw,
                       y.data_ptr() if y is not None else None,
                       ch.data_ptr() if ch is not None else None,
                       cl.data_ptr() if cl is not None else None, ldc, M, N, K, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    out = []
    for t in (y, ch, cl):
        if t is None:
            out.append(None)
            continue
        h = to_host(t)
        if out_pad:
            assert (h[:, N:] == 3.0).all(), "padding columns were written"
        out.append(np.ascontiguousarray(h[:, :N]))
    return out, (hi, lo)


def check_full(A, W, y, ch, cl, planes, what, ratio=True):
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, what)
    if ch is not None:
        merged = oracle.merge(ch, cl)
        assert np.array_equal(merged.view(np.uint32), y.view(np.uint32)), f"{what}: y != merge(c_hi, c_lo)"
        hi, lo = planes
        w64 = W.astype(np.float64)
        for part, plane, name in ((ch, hi, "c_hi"), (cl, lo, "c_lo")):
            p64 = plane.view(np.float16).astype(np.float64)
            exact, mag = p64 @ w64, np.abs(p64) @ np.abs(w64)
            assert (np.abs(part.astype(np.float64) - exact) <= TOL * mag).all(), f"{what}: {name} off"
        if ratio:
            return assert_better_than_single(y, ch, y64, abs64, what)
    return rel_errors(y, y64, abs64)


@pytest.mark.parametrize("name", ["single_linear", "qkv_projection", "unaligned", "square"])
def test_gemm_workloads(name):
    wl = workloads.ALL[name]()
    A, W = wl.A[0], wl.W
    note(f"gemm workload {name}")
    (y, ch, cl), planes = run_gemm(A, W)
    check_full(A, W, y, ch, cl, planes, name)
    note(f"gemm workload {name} repeat")
    (y2, ch2, cl2), _ = run_gemm(A, W)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    assert np.array_equal(ch.view(np.uint32), ch2.view(np.uint32))


def _edge_shapes():
    rng = np.random.default_rng(2024)
    shapes = [(1, 1, 1), (9, 1, 1), (33, 65, 129), (127, 255, 63), (128, 256, 64), (129, 257, 65),
              (300, 17, 300), (31, 1000, 33), (256, 512, 1024), (257, 300, 511)]
    for _ in range(10):
        shapes.append(tuple(int(v) for v in rng.integers(1, 301, 3)))
    return shapes


@pytest.mark.parametrize("M,N,K", _edge_shapes())
def test_gemm_edge_shapes(M, N, K):
    A, W = workloads.random_case(M * 7 + N * 3 + K, M, K, N)
    note(f"gemm edge M={M} N={N} K={K}")
    (y, ch, cl), planes = run_gemm(A, W, out_pad=3)
    check_full(A, W, y, ch, cl, planes, f"edge {M}x{N}x{K}", ratio=False)


@pytest.mark.parametrize("a_off,w_off", [(1, 0), (0, 1), (3, 5)])
def test_gemm_unaligned_operands(a_off, w_off):
    """Pointers and leading dimensions that are not 16-byte multiples take the
    element-load paths; results are identical to the aligned call."""
    A, W = workloads.random_case(77, 200, 333, 150)
    note(f"gemm unaligned a_off={a_off} w_off={w_off}")
    (y, ch, cl), planes = run_gemm(A, W, a_offset=a_off, w_offset=w_off)
    (y0, _, _), _ = run_gemm(A, W)
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))
    check_full(A, W, y, ch, cl, planes, "unaligned", ratio=False)


def test_gemm_output_selection():
    """Only y, or only (c_hi, c_lo): the same bits as when both are written."""
    A, W = workloads.random_case(5, 100, 64, 70)
    note("gemm output selection")
    (y, ch, cl), _ = run_gemm(A, W)
    (y1, n1, n2), _ = run_gemm(A, W, want_parts=False)
    (n3, ch2, cl2), _ = run_gemm(A, W, want_y=False)
    assert n1 is None and n2 is None and n3 is None
    assert np.array_equal(y1.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(ch2.view(np.uint32), ch.view(np.uint32))
    assert np.array_equal(cl2.view(np.uint32), cl.view(np.uint32))


def test_gemm_k_zero_writes_zeros():
    note("gemm K=0")
    y = torch.full((40, 50), 9.0, dtype=torch.float32, device="cuda")
    st = cf.cfp32_gemm(None, None, 0, None, 0, y.data_ptr(), None, None, 50, 40, 50, 0, stream_handle())
    assert st == cf.OK
    out = to_host(y)
    assert (out == 0).all() and not np.signbit(out).any()


def test_mfma_keeps_fp16_subnormals():
    """FP16-subnormal activations and weights: every product and partial sum
    is exact in FP32 (sums of integers times 2^-24 or 2^-14), so C_hi is fixed.
    A path that flushed FP16 subnormals would lose these terms."""
    rng = np.random.default_rng(1)
    M, N, K = 64, 64, 256
    ia = rng.integers(-1023, 1024, (M, K))          # subnormal hi: ia * 2^-24
    iw = rng.integers(-8, 9, (K, N))
    A = (ia * 2.0 ** -24).astype(np.float32)
    W = iw.astype(np.float16)
    note("mfma subnormal activations")
    (y, ch, cl), (hi, lo) = run_gemm(A, W)
    assert np.array_equal(hi.view(np.float16).astype(np.float64), ia * 2.0 ** -24)
    assert (lo == 0).all()
    assert np.array_equal(ch.astype(np.float64), (ia @ iw) * 2.0 ** -24)
    # subnormal weights against integer activations
    ja = rng.integers(-8, 9, (M, K))
    jw = rng.integers(-1023, 1024, (K, N))
    A2 = ja.astype(np.float32)
    W2 = (jw * 2.0 ** -24).astype(np.float16)
    note("mfma subnormal weights")
    (y2, ch2, cl2), _ = run_gemm(A2, W2)
    assert np.array_equal(ch2.astype(np.float64), (ja @ jw) * 2.0 ** -24)
    assert (cl2 == 0).all()


def test_mfma_accumulation_drift_is_bounded():
    """A long dot product with one large leading term and many small ones (the
    drift case the guide's AMD paragraph describes): the GPU's FP32
    accumulation may not drift further from FP64 than plain sequential FP32
    accumulation of the same products (the oracle's CPU model) does."""
    M, N, K = 32, 32, 8192
    rng = np.random.default_rng(2)
    A = (rng.uniform(0.5, 1.0, (M, K)) * 2.0 ** -10).astype(np.float32)
    A[:, 0] = 1024.0
    W = np.full((K, N), 0.5, np.float16)
    W[:, ::2] = np.float16(0.25)
    note("mfma drift")
    (y, ch, cl), planes = run_gemm(A, W)
    y64, abs64 = oracle.y64(A, W)
    gmax, _ = rel_errors(y, y64, abs64)
    ycpu, _, _ = oracle.linear_cf32(A, W)
    cmax, _ = rel_errors(ycpu, y64, abs64)
    print(f"drift: gpu max rel err {gmax:.3g}, sequential fp32 {cmax:.3g}")
    assert gmax <= 2 * cmax + 1e-7
    assert np.array_equal(oracle.merge(ch, cl).view(np.uint32), y.view(np.uint32))


def test_gemm_decode_ffn_prefill_full_size():
    """8192 x 4096 x 14336, the FFN projection the benchmark times (split +
    the LDS-DMA GEMM): every one of the 117M outputs within 1e-5 * sum|a w|
    of FP64, the error 16x below the same launch's single-FP16 C_hi over the
    whole output, the merge identity everywhere, and determinism."""
    wl = workloads.decode_ffn_pair()
    A, W = wl.A[1], wl.W
    note("gemm decode_ffn prefill full size")
    hi_t, lo_t = cf.split(to_dev(A))
    dw = to_dev(W)
    y, ch, cl = cf.gemm(hi_t, lo_t, dw, want_y=True, want_parts=True)
    yh = to_host(y)
    chh = to_host(ch)
    merged = oracle.merge(chh, to_host(cl))
    assert np.array_equal(merged.view(np.uint32), yh.view(np.uint32))
    del ch, cl, merged
    ymax, yrms, smax, srms = check_all_rows(A, W, yh, chh, "prefill 8192x4096x14336")
    print(f"prefill full size: y max {ymax:.3g} rms {yrms:.3g}; C_hi max {smax:.3g} rms {srms:.3g}")
    del chh
    y2, _, _ = cf.gemm(hi_t, lo_t, dw, want_y=True, want_parts=False)
    assert torch.equal(y, y2)


# -- the whole projection through cfp32_linear ----------------------------------

def run_linear(A, W, x_pad=0, y_pad=0, w_offset=0, w_ld_pad=0):
    M, K = A.shape
    N = W.shape[1]
    xb = np.zeros((M, K + x_pad), np.float32)
    xb[:, :K] = A
    ldw = N + w_offset + w_ld_pad
    wb = np.zeros(K * ldw + w_offset, np.uint16)
    wb[w_offset:].reshape(K, ldw)[:, :N] = W.view(np.uint16)
    dx, dw = to_dev(xb), to_dev(wb)
    y = torch.full((M, N + y_pad), 5.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_workspace_bytes(M, N, K)
    # The workspace's contents on entry must not matter: fill it with NaN bytes.
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")
    st = cf.cfp32_linear(dx.data_ptr(), K + x_pad, dw.data_ptr() + 2 * w_offset, ldw, y.data_ptr(), N + y_pad,
                         M, N, K, ws.data_ptr() if need else None, need, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    out = to_host(y)
    if y_pad:
        assert (out[:, N:] == 5.0).all()
    return np.ascontiguousarray(out[:, :N])


@pytest.mark.parametrize("name", ["single_linear", "qkv_projection", "unaligned", "square"])
def test_linear_workloads(name):
    wl = workloads.ALL[name]()
    A, W = wl.A[0], wl.W
    note(f"linear workload {name}")
    y = run_linear(A, W)
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, name)
    _, ch, _ = oracle.linear_cf32(A, W) if A.shape[0] <= 512 else (None, None, None)
    if ch is not None:
        assert_better_than_single(y, ch, y64, abs64, name)


def test_linear_decode_gemv_full():
    """M = 1 against the 4096 x 14336 weight: the small-M path."""
    wl = workloads.decode_ffn_pair(prefill_rows=1)
    A, W = wl.A[0], wl.W
    note("linear decode M=1")
    y = run_linear(A, W)
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y, y64, abs64, "decode")
    yc, ch, _ = oracle.linear_cf32(A, W)
    assert_better_than_single(y, ch, y64, abs64, "decode")
    y2 = run_linear(A, W)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("M", range(1, 10))
def test_linear_small_m_edges(M):
    """M = 1..8 take the small-M path, M = 9 the split + GEMM path; ragged N
    and K, padded leading dimensions, and weights that do (ldw % 8 == 0,
    16-byte aligned: chunked products + merge dispatch) and do not allow
    16-byte loads (batched 16 + 4-byte loads and funnel shifts when
    ldw >= 16: in chunks with a merge dispatch at one row of x or narrow
    W, else one strip kernel; the last row and narrower rows in dwords or
    elements)."""
    cases = [  # N, K, pointer offset of W in elements, extra ldw padding
        (777, 1000, 0, 7),    # aligned, ragged last tile and last chunk
        (777, 1000, 0, 0),    # ldw % 8 != 0
        (100, 37, 1, 0),      # unaligned pointer
        (64, 4096, 0, 0),     # aligned, many chunks
        (1, 5, 0, 7),         # aligned, one column, fewer rows than waves
        (1, 5, 3, 0),         # unaligned
        (2048, 3000, 8, 0),   # aligned pointer offset, several tiles
        (512, 1, 0, 0),       # one row of W
        (140000, 100, 0, 0),  # more than 256 column tiles: one chunk, merged in place
        (13, 1, 1, 4),        # unaligned, ldw >= 16, one row of W (only the last-row loads)
        (13, 2, 1, 4),        # unaligned, two rows: one batched row, then the last
        (600, 200, 3, 0),     # W at a 6-byte offset, ldw odd, K past three 64-row rounds
        (9000, 300, 1, 0),    # unaligned, wide: chunked at one row of x, one launch above
    ]
    for N, K, w_off, w_ld_pad in cases:
        A, W = workloads.random_case(M * 1000 + N + K, M, K, N, a_scale=100.0)
        note(f"linear small M={M} N={N} K={K} w_off={w_off} w_ld_pad={w_ld_pad}")
        y = run_linear(A, W, x_pad=3, y_pad=2, w_offset=w_off, w_ld_pad=w_ld_pad)
        y64, abs64 = oracle.y64(A, W)
        assert_within_tolerance(y, y64, abs64, f"M={M} N={N} K={K}")
        y2 = run_linear(A, W, x_pad=3, y_pad=2, w_offset=w_off, w_ld_pad=w_ld_pad)
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"


def test_linear_k_zero():
    for M in (1, 20):
        note(f"linear K=0 M={M}")
        y = torch.full((M, 33), 4.0, dtype=torch.float32, device="cuda")
        st = cf.cfp32_linear(None, 0, None, 33, y.data_ptr(), 33, M, 33, 0, None, 0, stream_handle())
        assert st == cf.OK
        assert (to_host(y) == 0).all()


@pytest.mark.parametrize("M", [64, 1])
def test_linear_rejects_small_workspace_and_enqueues_nothing(M):
    A, W = workloads.random_case(1, M, 64, 64)
    dx, dw = to_dev(A), to_dev(W)
    y = torch.full((M, 64), 6.0, dtype=torch.float32, device="cuda")
    need = cf.cfp32_linear_workspace_bytes(M, 64, 64)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    note(f"linear small workspace M={M}")
    st = cf.cfp32_linear(dx.data_ptr(), 64, dw.data_ptr(), 64, y.data_ptr(), 64, M, 64, 64,
                         ws.data_ptr(), need - 1, stream_handle())
    assert st == cf.ERR_INVALID_VALUE
    assert (to_host(y) == 6.0).all()


def test_linear_tensor_helper():
    A, W = workloads.random_case(8, 300, 256, 200)
    note("linear tensor helper")
    y = cf.linear(to_dev(A), to_dev(W).view(torch.float16))
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(to_host(y), y64, abs64, "helper")


@pytest.mark.parametrize("M,K,N", [(8200, 1000, 504), (4096, 4096, 1024), (16384, 256, 296), (8200, 1001, 504),
                                   (8200, 1000, 500), (4096, 4096, 4096)])
def test_linear_fused_split_matches_two_launches(M, K, N):
    """Shapes for which cfp32_linear splits x inside the GEMM (N <= 1024, at
    least 128 output tiles, K % 4 == 0, ldw % 8 == 0): identical bits to
    cfp32_split + cfp32_gemm, and within tolerance of the FP64 reference.
    K = 1001 (partial 16-byte granules of x), N = ldw = 500 and N = 4096
    take the two-launch path instead."""
    A, W = workloads.random_case(M + K + N, M, K, N, a_scale=30.0)
    note(f"linear fused split {M}x{K}x{N}")
    y = run_linear(A, W)
    dx, dw = to_dev(A), to_dev(W)
    hi = torch.empty((M, K), dtype=torch.int16, device="cuda")
    lo = torch.empty((M, K), dtype=torch.int16, device="cuda")
    y2 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    assert cf.cfp32_split(dx.data_ptr(), K, hi.data_ptr(), lo.data_ptr(), K, M, K, stream_handle()) == cf.OK
    assert cf.cfp32_gemm(hi.data_ptr(), lo.data_ptr(), K, dw.data_ptr(), N, y2.data_ptr(), None, None, N,
                         M, N, K, stream_handle()) == cf.OK
    assert np.array_equal(y.view(np.uint32), to_host(y2).view(np.uint32))
    check_all_rows(A, W, y, None, f"fused {M}x{K}x{N}")
