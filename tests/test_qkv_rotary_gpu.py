"""GPU tests of cfp32_qkv_rotary (Q/K/V packing with the rotary
multiplication, one dispatch) after a QKV projection of the 512 x 768 x 2304
workload (12 heads of 64).

The reference is the oracle's packing and rotation in double applied to the
same FP32 projection output.  v is a copy, so it must match exactly.  q and k
differ from the reference by the FP32 evaluation of the angle (frequency and
product: about 12 * 2^-24 of the angle) and of sincosf and the four products
and two sums: |out - ref| <= 1e-6 * (|x1| + |x2|) * (1 + |angle|) per pair.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import note, stream_handle, to_dev, to_host

pytestmark = pytest.mark.gpu


def check(qkv, H, D, pos, theta, q, k, v):
    rq, rk, rv = oracle.qkv_rotary(qkv, H, D, pos=pos, theta=theta)
    T = qkv.shape[0]
    assert np.array_equal(v, rv.astype(np.float32))
    p = np.arange(T) if pos is None else np.asarray(pos)
    ang = np.abs(p[:, None].astype(np.float64) * theta ** (-2.0 * np.arange(D // 2) / D))  # [T, D/2]
    for part, (got, ref) in enumerate(((q, rq), (k, rk))):
        src = qkv[:, part * H * D:(part + 1) * H * D].reshape(T, H, D).transpose(1, 0, 2).astype(np.float64)
        mag = np.abs(src[..., :D // 2]) + np.abs(src[..., D // 2:])          # [H, T, D/2]
        bound = 1e-6 * mag * (1.0 + ang[None])
        bound = np.concatenate([bound, bound], axis=-1)
        err = np.abs(got.astype(np.float64) - ref)
        assert (err <= bound + 1e-30).all(), f"part {part}: worst {(err - bound).max():.3g} over bound"


@pytest.mark.parametrize("positions", ["default", "random"])
def test_after_qkv_projection(positions):
    wl = workloads.qkv_projection()
    A, W = wl.A[0], wl.W
    H, D = 12, 64
    note(f"qkv rotary after projection, positions={positions}")
    qkv_t = cf.linear(to_dev(A), to_dev(W).view(torch.float16))
    qkv = to_host(qkv_t)
    T = qkv.shape[0]
    pos = None if positions == "default" else np.random.default_rng(5).integers(0, 8192, T).astype(np.int64)
    q, k, v = cf.qkv_rotary(qkv_t, H, D, positions=None if pos is None else to_dev(pos))
    check(qkv, H, D, pos, 10000.0, to_host(q), to_host(k), to_host(v))


def test_edges_and_padded_rows():
    for T, H, D, pad, theta in [(1, 1, 2, 0, 10000.0), (37, 3, 10, 5, 500000.0), (5, 2, 128, 1, 10000.0)]:
        note(f"qkv rotary T={T} H={H} D={D} pad={pad}")
        rows = np.random.default_rng(T + D).normal(0, 2, (T, 3 * H * D + pad)).astype(np.float32)
        dq = to_dev(rows)
        q, k, v = (torch.full((H, T, D), 7.0, dtype=torch.float32, device="cuda") for _ in range(3))
        st = cf.cfp32_qkv_rotary(dq.data_ptr(), 3 * H * D + pad, None, theta, q.data_ptr(), k.data_ptr(),
                                 v.data_ptr(), T, H, D, stream_handle())
        assert st == cf.OK
        check(rows[:, :3 * H * D], H, D, None, theta, to_host(q), to_host(k), to_host(v))
