"""cfp32_linear_noalloc: the projection for callers that cannot allocate
device memory, its scratch in a fixed array the library holds per device.

Through the C ABI, on two calls in a row with the second smaller than the
first (the array keeps the first call's contents, which must not matter),
its output equals cfp32_linear's with a workspace bit for bit, on each path:
the small-M dispatches (partial sums in the array; also for W rows that do
not allow 16-byte loads), split K over a small grid
(planes and partial sums), split + GEMM (planes exactly filling the 64 MiB),
the generic GEMM for unaligned shapes, split K above 64 rows, and, above 64
rows, a problem whose planes would not fit, which runs the GEMM that splits
inside (no scratch).  A problem that cannot run within the array (or whose
split of K needs more than it holds) is refused with CFP32_ERR_TOO_LARGE and
writes nothing.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
from compensated_fp32_projection_amd import workloads
from gpu_helpers import note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def with_workspace(A, W):
    M, K = A.shape
    N = W.shape[1]
    need = cf.cfp32_linear_workspace_bytes(M, N, K)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    dx, dw = to_dev(A), to_dev(W)  # held until the call has run
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    st = cf.cfp32_linear(dx.data_ptr(), K, dw.data_ptr(), N, y.data_ptr(), N, M, N, K,
                         ws.data_ptr(), need, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    return to_host(y)


def without(A, W):
    M, K = A.shape
    N = W.shape[1]
    dx, dw = to_dev(A), to_dev(W)
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    st = cf.cfp32_linear_noalloc(dx.data_ptr(), K, dw.data_ptr(), N, y.data_ptr(), N, M, N, K, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    return to_host(y)


# (first, second) shapes M, K, N; the second call is smaller.
PAIRS = [
    ((4096, 4096, 8192), (512, 768, 2304)),    # split + GEMM, planes of exactly 64 MiB; then no planes (split in registers)
    ((1, 4096, 14336), (3, 1000, 520)),        # small-M partial sums, twice
    ((64, 14336, 4096), (16, 2048, 3000)),     # split K (planes + partial sums); two groups of 8 rows
    ((8192, 4096, 14336), (333, 1000, 777)),   # planes of 128 MiB: split inside; then the generic GEMM
    ((256, 4096, 14336), (96, 4096, 14336)),   # split K above 64 rows (63 MB of planes and partial sums), twice
    ((1, 4096, 14335), (3, 1000, 777)),        # W rows not 16-byte loadable: chunked partial sums, twice
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_call(first, second):
    for M, K, N in (first, second):
        need = cf.cfp32_linear_workspace_bytes(M, N, K)
        A, W = workloads.random_case(M * 3 + K + N, M, K, N, a_scale=8.0)
        note(f"noalloc {M}x{K}x{N} (scratch {max(need - 256, 0)} of {SCRATCH} bytes)")
        y_ref = with_workspace(A, W)
        y = without(A, W)
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), f"{M}x{K}x{N}"


def test_noalloc_refuses_what_does_not_fit():
    """x with K % 4 != 0 cannot be split inside the GEMM, and its planes
    (2 x 5000 x 4008 FP16, 80 MB) exceed the array: refused, y untouched."""
    M, K, N = 5000, 4001, 300
    need = cf.cfp32_linear_workspace_bytes(M, N, K)
    assert need - 256 > SCRATCH
    A, W = workloads.random_case(1, M, K, N)
    dx, dw = to_dev(A), to_dev(W)
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    note("noalloc refusal 5000x4001x300")
    st = cf.cfp32_linear_noalloc(dx.data_ptr(), K, dw.data_ptr(), N, y.data_ptr(), N, M, N, K, stream_handle())
    assert st == cf.ERR_TOO_LARGE
    assert (to_host(y) == 7.0).all()


def test_noalloc_refuses_a_split_of_k_that_does_not_fit():
    """Above 64 rows on a small grid cfp32_linear splits K across blocks;
    when its planes and partial sums (here 21 MB and 50 MB) exceed the
    array, no path with its bits is left: refused, y untouched."""
    M, K, N = 256, 20480, 8192
    need = cf.cfp32_linear_workspace_bytes(M, N, K)
    assert need - 256 > SCRATCH
    dx = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    dw = torch.zeros((K, N), dtype=torch.int16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    note("noalloc refusal 256x20480x8192")
    st = cf.cfp32_linear_noalloc(dx.data_ptr(), K, dw.data_ptr(), N, y.data_ptr(), N, M, N, K, stream_handle())
    assert st == cf.ERR_TOO_LARGE
    assert (to_host(y) == 7.0).all()
