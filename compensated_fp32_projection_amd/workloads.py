"""Seeded synthetic projection workloads.

This module only draws inputs; it holds none of the split/product/merge
arithmetic, so both the GPU library's tests and the CPU oracle can be fed the
same bytes from it.  It needs numpy only.

Why synthetic: the laya.cpp Vulkan guide measures full checkpoints over a fixed
question corpus (its performance tables), and neither the checkpoints nor the
corpus nor the layer shapes are given.  These five shapes stand in for the
projections such a model runs: a small single linear, a QKV-style encoder
projection, a deliberately unaligned shape, a compute-bound square, and a
decoder FFN weight used both at decode (M = 1) and prefill (M = 8192).

Recipe (numpy ``default_rng(seed)``, draws in the order listed):

* normals are ``standard_normal(shape, dtype=float32)``; a normal of standard
  deviation s is that times ``float32(s)``;
* FP16 weights are an FP32 normal rounded to FP16 by numpy's cast (round to
  nearest even);
* "a fraction p of the entries" means the first ``round(p * size)`` positions
  of one ``permutation(size)``; scalings are exact powers of two.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Workload:
    name: str
    description: str
    seed: int
    M: int
    K: int
    N: int
    # One or more activation matrices sharing the weight (config 5 has two).
    A: list = field(default_factory=list)
    W: np.ndarray | None = None

    @property
    def W_bits(self) -> np.ndarray:
        return self.W.view(np.uint16)


def _weights(rng, K, N, sigma):
    return (rng.standard_normal((K, N), dtype=np.float32) * np.float32(sigma)).astype(np.float16)


def _scale_fraction(rng, A, fractions_and_scales):
    """Scale disjoint sets of entries (first counts of one permutation)."""
    flat = A.reshape(-1)
    perm = rng.permutation(flat.size)
    start = 0
    for p, scale in fractions_and_scales:
        cnt = int(round(p * flat.size))
        idx = perm[start:start + cnt]
        flat[idx] = flat[idx] * np.float32(scale)
        start += cnt
    return A


def single_linear() -> Workload:
    """A [16,256] ~ N(0,1) with 1 % of entries x 2^12 and 1 % x 2^-18 (the
    latter land in the FP16 subnormal range); W [256,384] ~ N(0, 0.02)."""
    rng = np.random.default_rng(0)
    A = rng.standard_normal((16, 256), dtype=np.float32)
    _scale_fraction(rng, A, [(0.01, 2.0 ** 12), (0.01, 2.0 ** -18)])
    W = _weights(rng, 256, 384, 0.02)
    return Workload("single_linear", "single linear 16x256x384 with outliers and FP16-subnormal entries",
                    0, 16, 256, 384, [A], W)


def qkv_projection() -> Workload:
    """A [512,768] ~ N(0,1) with 0.5 % of entries x 2^10; W [768,2304] ~ N(0,0.02)."""
    rng = np.random.default_rng(1)
    A = rng.standard_normal((512, 768), dtype=np.float32)
    _scale_fraction(rng, A, [(0.005, 2.0 ** 10)])
    W = _weights(rng, 768, 2304, 0.02)
    return Workload("qkv_projection", "QKV-style projection 512x768x2304", 1, 512, 768, 2304, [A], W)


def unaligned() -> Workload:
    """A [333,1000]: half U(-3e4, 3e4), half N(0, 1e-5) at permuted positions;
    W [1000,777] ~ N(0, 0.05)."""
    rng = np.random.default_rng(2)
    M, K, N = 333, 1000, 777
    size = M * K
    perm = rng.permutation(size)
    half = size // 2
    A = np.empty(size, np.float32)
    A[perm[:half]] = rng.uniform(-3e4, 3e4, half).astype(np.float32)
    A[perm[half:]] = rng.standard_normal(size - half, dtype=np.float32) * np.float32(1e-5)
    A = A.reshape(M, K)
    W = _weights(rng, K, N, 0.05)
    return Workload("unaligned", "non-aligned 333x1000x777, U(+-3e4) mixed with N(0,1e-5)",
                    2, M, K, N, [A], W)


def square() -> Workload:
    """A [4096,4096] ~ N(0,1); W [4096,4096] ~ N(0, 0.02)."""
    rng = np.random.default_rng(3)
    A = rng.standard_normal((4096, 4096), dtype=np.float32)
    W = _weights(rng, 4096, 4096, 0.02)
    return Workload("square", "compute-bound square 4096x4096x4096", 3, 4096, 4096, 4096, [A], W)


def decode_ffn_pair(prefill_rows: int = 8192) -> Workload:
    """W [4096,14336] ~ N(0, 0.02) drawn first; then A [1,4096] (decode) and
    A [8192,4096] (prefill), both ~ N(0,1).  ``prefill_rows`` below 8192 draws
    only the leading rows of the same stream (used for smaller smoke runs)."""
    rng = np.random.default_rng(4)
    W = _weights(rng, 4096, 14336, 0.02)
    A1 = rng.standard_normal((1, 4096), dtype=np.float32)
    A2 = rng.standard_normal((prefill_rows, 4096), dtype=np.float32)
    return Workload("decode_ffn_pair", "decode GEMV 1x4096x14336 + FFN GEMM 8192x4096x14336",
                    4, 8192, 4096, 14336, [A1, A2], W)


ALL = {
    "single_linear": single_linear,
    "qkv_projection": qkv_projection,
    "unaligned": unaligned,
    "square": square,
    "decode_ffn_pair": decode_ffn_pair,
}


def random_case(seed: int, M: int, K: int, N: int, a_scale: float = 1.0, w_sigma: float = 0.05):
    """Small random case for edge-shape sweeps: A ~ N(0, a_scale), W ~ N(0, w_sigma)."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K), dtype=np.float32) * np.float32(a_scale)
    W = _weights(rng, K, N, w_sigma)
    return A, W
