"""CPU oracle for the compensated-FP32 projection (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
imports nothing from the GPU library.

It follows the laya.cpp Vulkan backend guide (docs/vulkan.md): the
compensated-FP32 paragraph (split each FP32 projection input into two FP16
parts, take both products against the exact FP16 weights with FP32
accumulators, combine in FP32) and the split/merge paragraph (round to nearest
even, keep subnormals, scale the residual by 1024).  For an FP32 value x:

    hi = RNE16(x),  lo = RNE16((x - hi) * 1024),
    y  = C_hi + C_lo / 1024,  C_hi = A_hi W,  C_lo = A_lo W.

Functions (arrays are numpy; FP16 travels as uint16 bit patterns):

* ``f16_rne``, ``f16_to_f32``  -- O1/O2, binary16 rounding and widening.
* ``split``                    -- O3, bit-exact split.
* ``split_mismatches``         -- O3 used as a checker (NaN matched by class).
* ``merge``                    -- O4, y = C_hi + C_lo * 2^-10 in IEEE FP32.
* ``linear_cf32``              -- O5(b), the method on the CPU, FP32 sums.
* ``linear_f32``               -- O5(c), the plain FP32 product.
* ``y64``                      -- O5(a), FP64 reference and sum |a w| for a
                                  whole output, via a float64 matmul.
* ``y64_at``, ``ideal64_at``   -- O5(a)/(e) at chosen output positions.
* ``gelu64``, ``geglu64``      -- the GEGLU step after an FFN projection
                                  (exact GELU, g * Phi(g)), in double.
* ``qkv_rotary``               -- Q/K/V packing with the rotary multiplication
                                  after a QKV projection, in double.

Pins (what this oracle is checked against, apart from itself) live in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cfp32_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.o_fp_env_ok.restype = ctypes.c_int
    lib.o_num_threads.restype = ctypes.c_int
    lib.o_f16_rne.argtypes = [ctypes.c_float]
    lib.o_f16_rne.restype = ctypes.c_uint16
    lib.o_rne16.argtypes = [ctypes.c_double]
    lib.o_rne16.restype = ctypes.c_uint16
    lib.o_f16_value.argtypes = [ctypes.c_uint16]
    lib.o_f16_value.restype = ctypes.c_double
    lib.o_f16_rne_array.argtypes = [P, P, I64]
    lib.o_f16_rne_array.restype = None
    lib.o_f16_widen_array.argtypes = [P, P, I64]
    lib.o_f16_widen_array.restype = None
    lib.o_merge1.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.o_merge1.restype = ctypes.c_float
    lib.o_split.argtypes = [P, I64, P, P, I64, I64, I64]
    lib.o_split.restype = None
    lib.o_split_mismatches.argtypes = [P, P, P, I64, P]
    lib.o_split_mismatches.restype = I64
    lib.o_merge.argtypes = [P, P, I64, P, I64, I64, I64]
    lib.o_merge.restype = None
    lib.o_linear_cf32.argtypes = [P, I64, P, I64, P, P, P, I64, I64, I64, I64]
    lib.o_linear_cf32.restype = None
    lib.o_linear_f32.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64]
    lib.o_linear_f32.restype = None
    lib.o_dot64_at.argtypes = [P, I64, P, I64, I64, P, P, I64, P, P]
    lib.o_dot64_at.restype = None
    lib.o_ideal64_at.argtypes = [P, I64, P, I64, I64, P, P, I64, P]
    lib.o_ideal64_at.restype = None
    lib.o_gelu64.argtypes = [ctypes.c_double]
    lib.o_gelu64.restype = ctypes.c_double
    lib.o_geglu64.argtypes = [P, P, I64, P]
    lib.o_geglu64.restype = None
    lib.o_qkv_rotary.argtypes = [P, I64, P, ctypes.c_double, I64, I64, I64, P, P, P]
    lib.o_qkv_rotary.restype = None
    if not lib.o_fp_env_ok():
        raise RuntimeError("oracle: host FP environment has FTZ/DAZ or a non-nearest rounding mode")
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _as_f16_bits(w) -> np.ndarray:
    w = np.asarray(w)
    if w.dtype == np.float16:
        w = w.view(np.uint16)
    if w.dtype != np.uint16:
        raise TypeError("FP16 operands are numpy float16 or uint16 bit patterns")
    return np.ascontiguousarray(w)


def num_threads() -> int:
    """Threads the OpenMP loops of the oracle use."""
    return int(_load().o_num_threads())


# -- O1 / O2 -----------------------------------------------------------------

def f16_rne(x) -> np.ndarray:
    """RNE16 of each FP32 element, as uint16 bit patterns (O1)."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().o_f16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_to_f32(h) -> np.ndarray:
    """Exact widening of binary16 bit patterns to FP32 (O2)."""
    h = _as_f16_bits(h)
    out = np.empty(h.shape, np.float32)
    _load().o_f16_widen_array(_ptr(h), _ptr(out), h.size)
    return out


def f16_table() -> np.ndarray:
    """FP32 value of every one of the 65,536 binary16 patterns (O2)."""
    return f16_to_f32(np.arange(65536, dtype=np.uint16))


# -- O3 ----------------------------------------------------------------------

def split(x, ldh: int | None = None):
    """Split a 2-D FP32 array into (hi, lo) uint16 planes (O3)."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    rows, cols = x.shape
    hi = np.empty((rows, cols), np.uint16)
    lo = np.empty((rows, cols), np.uint16)
    _load().o_split(_ptr(x), cols, _ptr(hi), _ptr(lo), cols, rows, cols)
    return hi, lo


def split_mismatches(x, hi, lo):
    """Number of elements where (hi, lo) differ from O3, and the first index."""
    x = _c(x, np.float32).reshape(-1)
    hi = _as_f16_bits(hi).reshape(-1)
    lo = _as_f16_bits(lo).reshape(-1)
    if not (x.size == hi.size == lo.size):
        raise ValueError("size mismatch")
    first = np.zeros(1, np.int64)
    bad = _load().o_split_mismatches(_ptr(x), _ptr(hi), _ptr(lo), x.size, _ptr(first))
    return int(bad), int(first[0])


# -- O4 ----------------------------------------------------------------------

def merge(c_hi, c_lo) -> np.ndarray:
    """y = C_hi + C_lo * 2^-10 in IEEE FP32 (O4)."""
    c_hi = _c(c_hi, np.float32)
    c_lo = _c(c_lo, np.float32)
    if c_hi.shape != c_lo.shape:
        raise ValueError("shape mismatch")
    a = c_hi.reshape(1, -1) if c_hi.ndim < 2 else c_hi
    b = c_lo.reshape(a.shape)
    y = np.empty(a.shape, np.float32)
    rows, cols = a.shape
    _load().o_merge(_ptr(a), _ptr(b), cols, _ptr(y), cols, rows, cols)
    return y.reshape(c_hi.shape)


# -- O5 ----------------------------------------------------------------------

def linear_cf32(A, W):
    """The method on the CPU (O5(b)): returns (y, c_hi, c_lo), FP32 [M,N]."""
    A = _c(A, np.float32)
    W = _as_f16_bits(W)
    M, K = A.shape
    K2, N = W.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    y = np.empty((M, N), np.float32)
    ch = np.empty((M, N), np.float32)
    cl = np.empty((M, N), np.float32)
    _load().o_linear_cf32(_ptr(A), K, _ptr(W), N, _ptr(y), _ptr(ch), _ptr(cl), N, M, N, K)
    return y, ch, cl


def linear_f32(A, W) -> np.ndarray:
    """Plain FP32 product with fused multiply-adds, k ascending (O5(c))."""
    A = _c(A, np.float32)
    W = _as_f16_bits(W)
    M, K = A.shape
    K2, N = W.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    y = np.empty((M, N), np.float32)
    _load().o_linear_f32(_ptr(A), K, _ptr(W), N, _ptr(y), N, M, N, K)
    return y


def y64(A, W):
    """FP64 reference (O5(a)) for the whole output: (y64, abs64).

    A float64 matrix product serves as the summation step: every product of an
    FP32 and an FP16 value is exact in float64, so the only rounding is the
    float64 summation, about K * 2^-53 relative to sum |a w|."""
    A64 = np.asarray(A, dtype=np.float32).astype(np.float64)
    W64 = _as_f16_bits(W).view(np.float16).astype(np.float64)
    return A64 @ W64, np.abs(A64) @ np.abs(W64)


def y64_at(A, W, rows, cols):
    """FP64 reference and sum |a w| at positions (rows[i], cols[i]) (O5(a))."""
    A = _c(A, np.float32)
    W = _as_f16_bits(W)
    rows = _c(rows, np.int64).reshape(-1)
    cols = _c(cols, np.int64).reshape(-1)
    K = A.shape[1]
    if W.shape[0] != K:
        raise ValueError("inner dimensions differ")
    out = np.empty(rows.size, np.float64)
    absv = np.empty(rows.size, np.float64)
    _load().o_dot64_at(_ptr(A), A.shape[1], _ptr(W), W.shape[1], K, _ptr(rows), _ptr(cols),
                       rows.size, _ptr(out), _ptr(absv))
    return out, absv


def ideal64_at(A, W, rows, cols):
    """sum (hi + lo/1024) w in float64 at chosen positions (O5(e))."""
    A = _c(A, np.float32)
    W = _as_f16_bits(W)
    rows = _c(rows, np.int64).reshape(-1)
    cols = _c(cols, np.int64).reshape(-1)
    out = np.empty(rows.size, np.float64)
    _load().o_ideal64_at(_ptr(A), A.shape[1], _ptr(W), W.shape[1], A.shape[1], _ptr(rows),
                         _ptr(cols), rows.size, _ptr(out))
    return out


def gelu64(g) -> np.ndarray:
    """gelu(g) = g/2 (1 + erf(g / sqrt 2)) in double, elementwise."""
    lib = _load()
    g = np.asarray(g, np.float64)
    return np.vectorize(lib.o_gelu64, otypes=[np.float64])(g) if g.size else g.copy()


def geglu64(gate, up) -> np.ndarray:
    """gelu(gate) * up in double from FP32 gate and up of one shape."""
    lib = _load()
    gate = _c(gate, np.float32)
    up = _c(up, np.float32)
    if gate.shape != up.shape:
        raise ValueError("gate and up differ in shape")
    out = np.empty(gate.shape, np.float64)
    lib.o_geglu64(_ptr(gate), _ptr(up), gate.size, _ptr(out))
    return out


def qkv_rotary(qkv, H: int, D: int, pos=None, theta: float = 10000.0):
    """(q, k, v), each float64 [H, T, D], from the FP32 QKV projection output
    [T, 3 H D] (row t = [q | k | v], head h at h*D): q and k rotated in the
    half-split pairing (d, d + D/2) by pos[t] * theta^(-2i/D); v copied."""
    lib = _load()
    qkv = _c(qkv, np.float32)
    T = qkv.shape[0]
    if qkv.shape[1] < 3 * H * D or D % 2:
        raise ValueError("qkv must be [T, >= 3 H D] with D even")
    pos = np.arange(T, dtype=np.int64) if pos is None else _c(pos, np.int64)
    q = np.empty((H, T, D), np.float64)
    k = np.empty((H, T, D), np.float64)
    v = np.empty((H, T, D), np.float64)
    lib.o_qkv_rotary(_ptr(qkv), qkv.shape[1], _ptr(pos), float(theta), T, H, D, _ptr(q), _ptr(k), _ptr(v))
    return q, k, v
