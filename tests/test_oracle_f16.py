"""Pins for the oracle's binary16 rounding (O1), widening (O2) and split (O3).

Each check compares the oracle with something other than itself: numpy's and
PyTorch's own float16 casts (independent RNE implementations; PyTorch's CPU
cast runs on the x86 F16C hardware), hand-derived vectors, midpoint tables
built from the FP16 grid, and invariants of the definition in the laya.cpp
Vulkan guide's split/merge paragraph.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _nan16(h):
    h = np.asarray(h, np.uint16)
    return ((h & 0x7C00) == 0x7C00) & ((h & 0x03FF) != 0)


def _same16(want, got):
    """Bitwise equality, except that any NaN matches any NaN."""
    want = np.asarray(want, np.uint16)
    got = np.asarray(got, np.uint16)
    return np.where(_nan16(want), _nan16(got), want == got)


def _torch_f16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float16).numpy().view(np.uint16)


def _numpy_f16(x):
    with np.errstate(all="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def _load_vectors(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            rows.append((int(parts[0], 16), int(parts[1], 16), int(parts[2], 16), parts[3]))
    return rows


def test_fp_environment():
    assert oracle._load().o_fp_env_ok() == 1


def test_widen_all_patterns_against_numpy():
    """O2 on all 65,536 patterns equals numpy's float16 -> float32 widening."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_round_trip_all_patterns():
    """RNE16 of every exactly-representable FP16 value gives that pattern back."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.f16_to_f32(h)
    back = oracle.f16_rne(x)
    assert _same16(h, back).all()


def test_midpoints_tie_to_even_and_neighbours():
    """At every midpoint of two adjacent finite FP16 values the result is the
    even one; one FP32 step either side goes to the nearer neighbour.  The
    midpoint between 65504 and 65536 (the next value with an unbounded
    exponent) ties to the even 65536, i.e. overflows to infinity."""
    pos = np.arange(0, 0x7C00, dtype=np.uint16)             # +0 .. 65504
    vals = pos.view(np.float16).astype(np.float64)
    nxt = np.append(vals[1:], 65536.0)
    nxt_bits = np.append(pos[1:], np.uint16(0x7C00))
    mid = ((vals + nxt) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (vals + nxt) / 2)   # midpoints are exact in FP32
    even = np.where(pos % 2 == 0, pos, nxt_bits)
    for sign in (0, 0x8000):
        s = -1.0 if sign else 1.0
        m = (mid * np.float32(s)).astype(np.float32)
        assert np.array_equal(oracle.f16_rne(m), even | np.uint16(sign))
        up = np.nextafter(m, np.float32(s * np.inf))
        dn = np.nextafter(m, np.float32(-s * np.inf))
        assert np.array_equal(oracle.f16_rne(up), nxt_bits | np.uint16(sign))
        assert np.array_equal(oracle.f16_rne(dn), pos | np.uint16(sign))


@pytest.mark.slow
def test_rne16_all_fp32_inputs_against_f16c():
    """O1 on all 2^32 FP32 inputs equals the x86 F16C conversion (through
    PyTorch's CPU cast), NaN matched by class; numpy's software cast agrees on
    a spread sample of each chunk."""
    chunk = 1 << 26
    rng = np.random.default_rng(123)
    for c in range((1 << 32) // chunk):
        u = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint32)
        x = u.view(np.float32)
        got = oracle.f16_rne(x)
        want = _torch_f16(x)
        diff = np.flatnonzero(want != got)
        ok = _same16(want[diff], got[diff])
        if not ok.all():
            i = int(diff[np.flatnonzero(~ok)[0]])
            pytest.fail(f"RNE16 mismatch at x=0x{u[i]:08X}: oracle 0x{got[i]:04X}")
        pick = rng.integers(0, chunk, 4096)
        assert _same16(_numpy_f16(x[pick]), got[pick]).all()


def test_golden_split_vectors():
    """Hand-derived vectors (tests/golden/split_vectors.txt): the oracle and
    numpy's independent cast both give the stated bits."""
    rows = _load_vectors("split_vectors.txt")
    assert len(rows) == 12
    x = np.array([r[0] for r in rows], np.uint32).view(np.float32)
    hi, lo = oracle.split(x.reshape(1, -1))
    for i, (xb, hb, lb, name) in enumerate(rows):
        assert hi[0, i] == hb, f"{name}: hi 0x{hi[0, i]:04X} != 0x{hb:04X}"
        assert lo[0, i] == lb, f"{name}: lo 0x{lo[0, i]:04X} != 0x{lb:04X}"
    np_hi = _numpy_f16(x)
    with np.errstate(all="ignore"):
        np_lo = _numpy_f16((x - np_hi.view(np.float16).astype(np.float32)) * np.float32(1024))
    assert np.array_equal(np_hi, np.array([r[1] for r in rows], np.uint16))
    assert np.array_equal(np_lo, np.array([r[2] for r in rows], np.uint16))


def _split_reference_f32(x):
    """The split restated with single-precision arithmetic and the F16C cast:
    hi = f16(x), lo = f16(fp32(fp32(x - hi) * 1024)).  It equals the
    definition exactly when x - hi is exact in FP32, which is the property
    the agreement below pins (together with the rounding of both parts)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    h = t.to(torch.float16)
    r = (t - h.to(torch.float32)) * 1024.0
    return h.numpy().view(np.uint16), r.to(torch.float16).numpy().view(np.uint16)


BINADES = [0, 1, 2, 100, 101, 102, 103, 104, 108, 112, 113, 114, 126, 127, 128,
           140, 141, 142, 143, 144, 200, 254, 255]


@pytest.mark.slow
@pytest.mark.parametrize("expo", BINADES)
def test_split_exhaustive_binade(expo):
    """O3 over every mantissa of a binade, both signs: equals the FP32/F16C
    restatement bitwise (NaN by class).  The binades cover FP32 subnormals,
    the FP16 subnormal range, 2^-14, 1, the values above 32,000 and the
    overflow binade 2^16, and infinities/NaN."""
    m = np.arange(1 << 23, dtype=np.uint32)
    for sign in (0, 1):
        u = (np.uint32(sign << 31) | np.uint32(expo << 23) | m).astype(np.uint32)
        x = u.view(np.float32)
        hi, lo = oracle.split(x.reshape(1, -1))
        rh, rl = _split_reference_f32(x)
        ok = _same16(rh, hi[0]) & _same16(rl, lo[0])
        if not ok.all():
            i = int(np.flatnonzero(~ok)[0])
            pytest.fail(f"split mismatch at x=0x{u[i]:08X}: oracle (0x{hi[0, i]:04X}, 0x{lo[0, i]:04X})"
                        f" reference (0x{rh[i]:04X}, 0x{rl[i]:04X})")


def test_split_random_against_numpy_and_bound():
    """O3 on 2^22 random bit patterns equals numpy's restatement; for finite
    |x| < 65520 the reconstruction error obeys the representation bound
    |x - (hi + lo/1024)| <= max(2^-23 |x|, 2^-35) and the residual x - hi is
    exactly representable in FP32."""
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    hi, lo = oracle.split(x.reshape(1, -1))
    hi, lo = hi[0], lo[0]
    np_hi = _numpy_f16(x)
    with np.errstate(all="ignore"):
        r32 = x - np_hi.view(np.float16).astype(np.float32)
        np_lo = _numpy_f16(r32 * np.float32(1024))
    assert (_same16(np_hi, hi) & _same16(np_lo, lo)).all()

    fin = np.isfinite(x) & (np.abs(x) < 65520)
    xf = x[fin].astype(np.float64)
    hv = hi[fin].view(np.float16).astype(np.float64)
    lv = lo[fin].view(np.float16).astype(np.float64)
    err = np.abs(xf - (hv + lv / 1024.0))
    bound = np.maximum(2.0 ** -23 * np.abs(xf), 2.0 ** -35)
    assert (err <= bound).all()
    assert np.array_equal((xf - hv).astype(np.float32).astype(np.float64), xf - hv)


def test_split_bound_is_tight_on_log_uniform():
    """The representation bound is reached (ratio 1) somewhere on a log-uniform
    sample, so it is not loose: the split keeps about 23 of FP32's 24 bits."""
    rng = np.random.default_rng(11)
    x = (np.exp(rng.uniform(np.log(1e-6), np.log(6e4), 1 << 21)) *
         rng.choice([-1.0, 1.0], 1 << 21)).astype(np.float32)
    hi, lo = oracle.split(x.reshape(1, -1))
    xf = x.astype(np.float64)
    rec = hi[0].view(np.float16).astype(np.float64) + lo[0].view(np.float16).astype(np.float64) / 1024
    ratio = np.abs(xf - rec) / np.maximum(2.0 ** -23 * np.abs(xf), 2.0 ** -35)
    assert ratio.max() <= 1.0
    assert ratio.max() >= 0.99


def test_split_mismatch_checker_flags_planted_errors():
    """The checker used by the GPU tests reports a planted wrong bit, and
    accepts NaN with another payload."""
    x = np.array([1.0, 3.0, np.nan, 1e-30], np.float32)
    hi, lo = oracle.split(x.reshape(1, -1))
    hi, lo = hi[0].copy(), lo[0].copy()
    assert oracle.split_mismatches(x, hi, lo) == (0, -1)
    hi2 = hi.copy()
    hi2[2] = 0x7C01 | 0x8000    # another NaN
    assert oracle.split_mismatches(x, hi2, lo) == (0, -1)
    lo2 = lo.copy()
    lo2[3] ^= 0x8000            # wrong sign of zero
    assert oracle.split_mismatches(x, hi, lo2) == (1, 3)
