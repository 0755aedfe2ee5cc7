"""The seeded input generators: deterministic, and shaped as stated."""
import numpy as np

from compensated_fp32_projection_amd import workloads


def test_generators_are_deterministic():
    for name in ("single_linear", "qkv_projection", "unaligned"):
        a = workloads.ALL[name]()
        b = workloads.ALL[name]()
        assert np.array_equal(a.A[0].view(np.uint32), b.A[0].view(np.uint32))
        assert np.array_equal(a.W_bits, b.W_bits)


def test_single_linear_recipe():
    wl = workloads.single_linear()
    A, W = wl.A[0], wl.W
    assert A.shape == (16, 256) and A.dtype == np.float32
    assert W.shape == (256, 384) and W.dtype == np.float16
    big = np.abs(A) > 8            # 41 entries scaled by 2^12 (N(0,1) alone never reaches 8 here)
    tiny = np.abs(A) < 2.0 ** -12  # 41 entries scaled by 2^-18: FP16-subnormal hi
    assert 36 <= big.sum() <= 41
    assert 38 <= tiny.sum() <= 43
    assert 0.015 < W.astype(np.float64).std() < 0.025


def test_qkv_recipe():
    wl = workloads.qkv_projection()
    A = wl.A[0]
    assert A.shape == (512, 768)
    assert 1850 <= (np.abs(A) > 8).sum() <= 1966     # 1966 entries scaled by 2^10
    assert wl.W.shape == (768, 2304)


def test_unaligned_recipe():
    wl = workloads.unaligned()
    A = wl.A[0]
    assert A.shape == (333, 1000) and wl.W.shape == (1000, 777)
    small = np.abs(A) < 1e-3
    assert abs(small.sum() - 166500) < 50
    assert np.abs(A).max() <= 3e4


def test_decode_pair_shares_weight_stream():
    """The smaller prefill draw is the prefix of the full one."""
    small = workloads.decode_ffn_pair(prefill_rows=4)
    assert small.W.shape == (4096, 14336)
    assert small.A[0].shape == (1, 4096) and small.A[1].shape == (4, 4096)
