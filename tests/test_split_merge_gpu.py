"""GPU split and merge against the oracle, bit for bit (NaN by class).

The split is checked on every one of the 2^32 FP32 bit patterns through the
vectorised kernel, on 46 whole binades through the element-wise kernel, on
the hand-derived vectors, on every workload's activations, and with strided
leading dimensions (padding left untouched).  The merge is checked on random
values over the whole exponent range, planted ties, and the golden vectors.
"""
import os

import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_split(x: np.ndarray, ldh_pad: int = 0):
    """Split a host FP32 [rows, cols] array on the GPU; returns uint16 planes."""
    x = np.ascontiguousarray(x, np.float32)
    rows, cols = x.shape
    d = to_dev(x)
    ldh = cols + ldh_pad
    hi = torch.full((rows, ldh), 0x5A5A, dtype=torch.int16, device="cuda")
    lo = torch.full((rows, ldh), 0x5A5A, dtype=torch.int16, device="cuda")
    st = cf.cfp32_split(d.data_ptr(), cols, hi.data_ptr(), lo.data_ptr(), ldh, rows, cols, stream_handle())
    assert st == cf.OK, cf.cfp32_status_string(st)
    h = to_host(hi, np.uint16)
    l = to_host(lo, np.uint16)
    if ldh_pad:
        assert (h[:, cols:] == 0x5A5A).all() and (l[:, cols:] == 0x5A5A).all(), "padding was written"
    return h[:, :cols], l[:, :cols]


def _check_split(x, hi, lo, what):
    bad, first = oracle.split_mismatches(x, hi, lo)
    if bad:
        xf = np.ascontiguousarray(x, np.float32).reshape(-1)
        raise AssertionError(f"{what}: {bad} mismatches; first x=0x{xf[first].view(np.uint32):08X} "
                             f"gpu=(0x{hi.reshape(-1)[first]:04X}, 0x{lo.reshape(-1)[first]:04X})")


def test_split_golden_vectors():
    rows = []
    with open(os.path.join(GOLDEN, "split_vectors.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                p = line.split()
                rows.append((int(p[0], 16), int(p[1], 16), int(p[2], 16), p[3]))
    x = np.array([r[0] for r in rows], np.uint32).view(np.float32)
    for shape in [(1, len(rows)), (3, 4)]:          # element-wise and vectorised kernels
        note(f"split golden vectors shape={shape}")
        h, l = gpu_split(x.reshape(shape))
        for i, r in enumerate(rows):
            assert h.reshape(-1)[i] == r[1], r[3]
            assert l.reshape(-1)[i] == r[2], r[3]


@pytest.mark.parametrize("quarter", range(4))
def test_split_all_fp32_patterns(quarter):
    """Every FP32 bit pattern through the vectorised split kernel."""
    chunk = 1 << 27
    per_q = (1 << 32) // 4
    for start in range(quarter * per_q, (quarter + 1) * per_q, chunk):
        note(f"split exhaustive chunk start=0x{start:08X}")
        x = np.arange(start, start + chunk, dtype=np.uint32).view(np.float32).reshape(1 << 13, 1 << 14)
        h, l = gpu_split(x)
        _check_split(x, h, l, f"chunk 0x{start:08X}")


SCALAR_BINADES = [0, 1, 2, 90, 100, 101, 102, 103, 104, 105, 106, 107, 108, 109, 110, 111, 112, 113, 114,
                  115, 120, 125, 126, 127, 128, 129, 130, 135, 138, 139, 140, 141, 142, 143, 144, 145, 150,
                  160, 180, 200, 220, 240, 250, 253, 254, 255]


def test_split_elementwise_kernel_binades():
    """Whole binades (both signs) through the element-wise kernel: the row
    length 8191 is odd, so the vectorised kernel cannot be used."""
    m = np.arange(1 << 23, dtype=np.uint32)
    for expo in SCALAR_BINADES:
        note(f"split element-wise binade {expo}")
        u = np.concatenate([(np.uint32(expo << 23) | m), (np.uint32((256 + expo) << 23) | m)])
        u = np.concatenate([u, np.zeros(8191 * 2049 - u.size, np.uint32)])
        x = u.view(np.float32).reshape(2049, 8191)
        h, l = gpu_split(x)
        _check_split(x, h, l, f"binade {expo}")


@pytest.mark.parametrize("name", ["single_linear", "qkv_projection", "unaligned", "square"])
def test_split_workload_activations(name):
    wl = workloads.ALL[name]()
    note(f"split workload {name}")
    h, l = gpu_split(wl.A[0], ldh_pad=3)
    _check_split(wl.A[0], h, l, name)


def test_split_decode_ffn_activations():
    wl = workloads.decode_ffn_pair()
    for A in wl.A:
        note(f"split decode_ffn A{A.shape}")
        h, l = gpu_split(A)
        _check_split(A, h, l, f"decode_ffn {A.shape}")


def test_split_strided_input():
    """x with a leading dimension larger than its rows, hi/lo padded."""
    rng = np.random.default_rng(3)
    big = rng.standard_normal((37, 200)).astype(np.float32)
    d = to_dev(big)
    rows, cols, ldx, ldh = 37, 150, 200, 157
    hi = torch.full((rows, ldh), 0x1234, dtype=torch.int16, device="cuda")
    lo = torch.full((rows, ldh), 0x1234, dtype=torch.int16, device="cuda")
    note("split strided")
    st = cf.cfp32_split(d.data_ptr(), ldx, hi.data_ptr(), lo.data_ptr(), ldh, rows, cols, stream_handle())
    assert st == cf.OK
    h = to_host(hi, np.uint16)
    l = to_host(lo, np.uint16)
    assert (h[:, cols:] == 0x1234).all() and (l[:, cols:] == 0x1234).all()
    _check_split(big[:, :cols], np.ascontiguousarray(h[:, :cols]), np.ascontiguousarray(l[:, :cols]), "strided")


def test_split_tensor_helper_matches():
    x = np.random.default_rng(9).standard_normal((64, 96)).astype(np.float32) * 1000
    note("split tensor helper")
    hi, lo = cf.split(to_dev(x))
    _check_split(x, to_host(hi).view(np.uint16), to_host(lo).view(np.uint16), "helper")


# -- merge ---------------------------------------------------------------------

def gpu_merge(a, b, pad=0):
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    rows, cols = a.shape
    da, db = to_dev(a), to_dev(b)
    y = torch.full((rows, cols + pad), 7.0, dtype=torch.float32, device="cuda")
    st = cf.cfp32_merge(da.data_ptr(), db.data_ptr(), cols, y.data_ptr(), cols + pad, rows, cols, stream_handle())
    assert st == cf.OK
    out = to_host(y)
    if pad:
        assert (out[:, cols:] == 7.0).all()
    return np.ascontiguousarray(out[:, :cols])


def _merge_inputs(n, seed):
    rng = np.random.default_rng(seed)
    e1 = rng.integers(-149, 100, n)
    e2 = e1 + rng.integers(-40, 20, n)
    a = (rng.uniform(-1, 1, n) * np.exp2(e1)).astype(np.float32)
    b = (rng.uniform(-1, 1, n) * np.exp2(np.clip(e2, -149, 127))).astype(np.float32)
    t = rng.integers(0, n, n // 16)
    a[t] = np.float32(1.0) + np.float32(2.0 ** -23) * rng.integers(0, 2, t.size).astype(np.float32)
    b[t] = np.float32(2.0 ** -14)
    return a, b


@pytest.mark.parametrize("shape,pad", [((1024, 4096), 0), ((999, 1001), 5), ((1, 7), 0)])
def test_merge_against_oracle(shape, pad):
    n = shape[0] * shape[1]
    a, b = _merge_inputs(n, n)
    a, b = a.reshape(shape), b.reshape(shape)
    note(f"merge {shape} pad={pad}")
    got = gpu_merge(a, b, pad)
    want = oracle.merge(a, b)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_merge_golden_vectors():
    rows = []
    with open(os.path.join(GOLDEN, "merge_vectors.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                p = line.split()
                rows.append((int(p[0], 16), int(p[1], 16), int(p[2], 16)))
    a = np.array([r[0] for r in rows], np.uint32).view(np.float32).reshape(1, -1)
    b = np.array([r[1] for r in rows], np.uint32).view(np.float32).reshape(1, -1)
    note("merge golden")
    got = gpu_merge(a, b)
    assert np.array_equal(got.view(np.uint32).ravel(), np.array([r[2] for r in rows], np.uint32))
