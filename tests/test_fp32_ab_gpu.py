"""Compensated FP32 next to true FP32 on the GPU (accuracy side of the A/B;
the speed side is the ``fp32_ab_4096`` entry of bench.py's output).

The laya.cpp Vulkan guide offers the two FP16 products as a stand-in for
FP32 arithmetic on tensor hardware (compensated-FP32 paragraph).  Here the
true-FP32 side is this library's own FP32 kernel (cfp32_linear_f32) and,
for reference, the FP32 library GEMM (torch.matmul on FP32 operands with
TF32 off), both fed the same FP32 activations and the same weights widened
exactly from FP16.

What the arithmetic fixes: hi + lo/1024 represents each activation to within
about 2^-24 of its magnitude (hi holds 11 significant bits, lo the next 11 of
the residual, which is at most half an FP16 ulp of hi), about the rounding of
one FP32 operation, and both sides accumulate in FP32.  So both results must
meet the 1e-5 * sum|a w| bound, and the compensated error must be of the same
order as the FP32 library's: its RMS within 4x of it.
"""
import numpy as np
import pytest
import torch

import compensated_fp32_projection_amd as cf
import oracle
from compensated_fp32_projection_amd import workloads
from gpu_helpers import assert_within_tolerance, note, rel_errors, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["single_linear", "qkv_projection", "unaligned", "square"])
def test_compensated_error_matches_true_fp32(name):
    wl = workloads.ALL[name]()
    A, W = wl.A[0], wl.W
    note(f"fp32 A/B {name}")
    dx, dw = to_dev(A), to_dev(W).view(torch.float16)
    y_c = to_host(cf.linear(dx, dw))
    prev = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        y_f = to_host(torch.matmul(dx, dw.float()))
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev
    y_o = to_host(cf.linear_f32(dx, dw))
    y64, abs64 = oracle.y64(A, W)
    assert_within_tolerance(y_c, y64, abs64, f"{name} compensated")
    assert_within_tolerance(y_f, y64, abs64, f"{name} fp32 library")
    assert_within_tolerance(y_o, y64, abs64, f"{name} fp32 own kernel")
    c_max, c_rms = rel_errors(y_c, y64, abs64)
    f_max, f_rms = rel_errors(y_f, y64, abs64)
    o_max, o_rms = rel_errors(y_o, y64, abs64)
    note(f"{name}: compensated max {c_max:.3g} rms {c_rms:.3g}; fp32 library max {f_max:.3g} rms {f_rms:.3g}; "
         f"fp32 own kernel max {o_max:.3g} rms {o_rms:.3g}")
    assert c_rms <= 4.0 * f_rms, (name, c_rms, f_rms)
    assert c_rms <= 4.0 * o_rms, (name, c_rms, o_rms)
