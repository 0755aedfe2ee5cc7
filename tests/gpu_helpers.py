"""Helpers shared by the GPU tests: moving numpy arrays to and from the
device, and the acceptance measures the tests apply.

Acceptance (same on every path):
  * split and merge outputs: bit-exact against the oracle (NaN by class);
  * merged projection y: finite and |y - y64| <= 1e-5 * sum_k |a_k w_k|
    elementwise, exact zero where that sum is zero;
  * "measurably below a single FP16 conversion": max and RMS of
    |.-y64| / sum|a w| at least 16 times smaller for y than for C_hi;
  * determinism: a repeated call gives identical bits.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import compensated_fp32_projection_amd as cf

TOL = 1e-5
RATIO = 16.0


def note(msg: str):
    """Name the case before a GPU step, so a crash report still says what ran."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.int16)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def to_host(t: torch.Tensor, dtype=None) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def stream_handle():
    return torch.cuda.current_stream().cuda_stream


def rel_errors(y, y64, abs64):
    e = np.abs(np.asarray(y, np.float64) - y64) / np.where(abs64 > 0, abs64, 1.0)
    return float(e.max()), float(np.sqrt(np.mean(e ** 2)))


def assert_within_tolerance(y, y64, abs64, what=""):
    y = np.asarray(y)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    diff = np.abs(y.astype(np.float64) - y64)
    bad = diff > TOL * abs64
    if bad.any():
        i = np.unravel_index(np.flatnonzero(bad.ravel())[0], y.shape) if y.ndim > 1 else np.flatnonzero(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside 1e-5*sum|aw|; first at {i}: "
                             f"y={y[i]!r} y64={y64[i]!r} sum|aw|={abs64[i]!r}")
    zero = abs64 == 0
    assert (y[zero] == 0).all(), f"{what}: nonzero output where sum|aw| = 0"


def assert_better_than_single(y, c_hi, y64, abs64, what=""):
    ymax, yrms = rel_errors(y, y64, abs64)
    smax, srms = rel_errors(c_hi, y64, abs64)
    assert ymax * RATIO <= smax, f"{what}: max error {ymax:.3g} not {RATIO}x below single-FP16 {smax:.3g}"
    assert yrms * RATIO <= srms, f"{what}: rms error {yrms:.3g} not {RATIO}x below single-FP16 {srms:.3g}"
    return ymax, smax


def check_all_rows(A, W, y, c_hi=None, what="", block=1024):
    """Every element of y [M, N] against the FP64 reference, a block of rows
    at a time (the float64 products of a full 8192 x 4096 x 14336 output
    would need several GB at once): tolerance, finiteness and exact zeros as
    assert_within_tolerance.  With c_hi (the same call's single-FP16
    product), also the 16x error ratio over the whole output.  Returns the
    max and RMS normalised errors of y (and of c_hi, or None)."""
    import oracle
    M = A.shape[0]
    ymax = ysq = 0.0
    smax = ssq = 0.0
    for r0 in range(0, M, block):
        r1 = min(M, r0 + block)
        y64, abs64 = oracle.y64(A[r0:r1], W)
        yb = np.asarray(y[r0:r1])
        assert_within_tolerance(yb, y64, abs64, f"{what} rows {r0}:{r1}")
        den = np.where(abs64 > 0, abs64, 1.0)
        e = np.abs(yb.astype(np.float64) - y64) / den
        ymax = max(ymax, float(e.max()))
        ysq += float(np.sum(e * e))
        if c_hi is not None:
            s = np.abs(np.asarray(c_hi[r0:r1], np.float64) - y64) / den
            smax = max(smax, float(s.max()))
            ssq += float(np.sum(s * s))
    n = y.shape[0] * y.shape[1]
    yrms = (ysq / n) ** 0.5
    if c_hi is None:
        return ymax, yrms, None, None
    srms = (ssq / n) ** 0.5
    assert ymax * RATIO <= smax, f"{what}: max error {ymax:.3g} not {RATIO}x below single-FP16 {smax:.3g}"
    assert yrms * RATIO <= srms, f"{what}: rms error {yrms:.3g} not {RATIO}x below single-FP16 {srms:.3g}"
    return ymax, yrms, smax, srms
