"""The C-ABI library: it loads, exports every function include/cfp32.h
declares, and its host-side argument checks run before any device work.

No kernel is launched here.  Calls that fail validation, or that are empty,
return before the library touches the GPU; on a machine without a gfx950 GPU
a valid call must report CFP32_ERR_UNSUPPORTED_DEVICE (there is no CPU
fallback).
"""
import ctypes
import os
import re

import pytest

import compensated_fp32_projection_amd as cf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cfp32.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"CFP32_API\s+[\w\s\*]*?\b(cfp32_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cf.LIB_PATH):
        from compensated_fp32_projection_amd import build
        build.build()
    return cf.load_library()


def test_header_declares_the_boundary():
    assert _declared() == sorted(cf.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for s in (cf.OK, cf.ERR_INVALID_VALUE, cf.ERR_UNSUPPORTED_DEVICE, cf.ERR_HIP, cf.ERR_TOO_LARGE):
        assert cf.cfp32_status_string(s)
    assert cf.cfp32_status_string(99) == "unknown status"


FAKE = 1 << 20  # never dereferenced: these calls fail or return before any device work


def test_invalid_arguments_are_rejected_on_the_host(lib):
    E = cf.ERR_INVALID_VALUE
    # negative sizes
    assert cf.cfp32_split(FAKE, 4, FAKE, FAKE, 4, -1, 4, None) == E
    assert cf.cfp32_gemm(FAKE, FAKE, 4, FAKE, 4, FAKE, None, None, 4, 4, 4, -4, None) == E
    # null pointers
    assert cf.cfp32_split(None, 4, FAKE, FAKE, 4, 2, 4, None) == E
    assert cf.cfp32_merge(FAKE, None, 4, FAKE, 4, 2, 4, None) == E
    assert cf.cfp32_linear(FAKE, 8, None, 8, FAKE, 8, 2, 8, 8, None, 0, None) == E
    # leading dimension below the row length
    assert cf.cfp32_split(FAKE, 3, FAKE, FAKE, 4, 2, 4, None) == E
    assert cf.cfp32_gemm(FAKE, FAKE, 7, FAKE, 8, FAKE, None, None, 8, 4, 8, 8, None) == E
    assert cf.cfp32_merge(FAKE, FAKE, 8, FAKE, 7, 2, 8, None) == E
    # separate-addition gemm: unsupported depth per addition, missing outputs
    for kpa in (-16, 8, 32, 128, 512):
        assert cf.cfp32_gemm_separate_add(FAKE, FAKE, 8, FAKE, 8, FAKE, None, None, 8, 4, 8, 8, kpa, None) == E
    assert cf.cfp32_gemm_separate_add(FAKE, FAKE, 8, FAKE, 8, None, None, None, 8, 4, 8, 8, 16, None) == E
    assert cf.cfp32_gemm_separate_add(FAKE, FAKE, 7, FAKE, 8, FAKE, None, None, 8, 4, 8, 8, 16, None) == E
    # gemm: no output, or only one of c_hi / c_lo
    assert cf.cfp32_gemm(FAKE, FAKE, 8, FAKE, 8, None, None, None, 8, 4, 8, 8, None) == E
    assert cf.cfp32_gemm(FAKE, FAKE, 8, FAKE, 8, None, FAKE, None, 8, 4, 8, 8, None) == E
    # linear: workspace missing or too small, M > 8 and M <= 8
    for M in (64, 1):
        need = cf.cfp32_linear_workspace_bytes(M, 64, 64)
        assert need > 0
        assert cf.cfp32_linear(FAKE, 64, FAKE, 64, FAKE, 64, M, 64, 64, None, 0, None) == E
        assert cf.cfp32_linear(FAKE, 64, FAKE, 64, FAKE, 64, M, 64, 64, FAKE, need - 1, None) == E
    # linear_noalloc: null pointers, short leading dimensions, negative sizes
    assert cf.cfp32_linear_noalloc(None, 8, FAKE, 8, FAKE, 8, 2, 8, 8, None) == E
    assert cf.cfp32_linear_noalloc(FAKE, 7, FAKE, 8, FAKE, 8, 2, 8, 8, None) == E
    assert cf.cfp32_linear_noalloc(FAKE, 8, FAKE, 8, FAKE, 7, 2, 8, 8, None) == E
    assert cf.cfp32_linear_noalloc(FAKE, 8, FAKE, 8, FAKE, 8, -2, 8, 8, None) == E
    # linear_noalloc: scratch beyond its 64 MiB with at most 64 rows is
    # refused before the device is looked at (M = 64, K = 2^20: planes of
    # 2 x 64 x 2^20 x 2 bytes = 256 MiB)
    assert cf.cfp32_linear_noalloc(FAKE, 1 << 20, FAKE, 8, FAKE, 8, 64, 8, 1 << 20, None) == cf.ERR_TOO_LARGE
    # linear_ex: unknown layout; [N, K] weights need ldw >= K
    assert cf.cfp32_linear_ex(FAKE, 64, FAKE, 64, 2, None, FAKE, 64, 2, 64, 64, None, 0, None) == E
    assert cf.cfp32_linear_ex(FAKE, 64, FAKE, 63, cf.W_NK, None, FAKE, 64, 2, 64, 64, None, 0, None) == E
    assert cf.cfp32_linear_ex(FAKE, 64, FAKE, 32, cf.W_NK, None, FAKE, 64, 2, 16, 64, None, 0, None) == E
    # linear_geglu: w narrower than 2F, out narrower than F, small workspace
    assert cf.cfp32_linear_geglu(FAKE, 64, FAKE, 63, None, FAKE, 32, 2, 32, 64, None, 0, None) == E
    assert cf.cfp32_linear_geglu(FAKE, 64, FAKE, 64, None, FAKE, 31, 2, 32, 64, None, 0, None) == E
    need = cf.cfp32_linear_geglu_workspace_bytes(2, 32, 64)
    assert need > 0
    assert cf.cfp32_linear_geglu(FAKE, 64, FAKE, 64, None, FAKE, 32, 2, 32, 64, FAKE, need - 1, None) == E
    # qkv_rotary: odd D, non-positive theta, ldq below 3*H*D
    assert cf.cfp32_qkv_rotary(FAKE, 96, None, 10000.0, FAKE, FAKE, FAKE, 4, 2, 15, None) == E
    assert cf.cfp32_qkv_rotary(FAKE, 96, None, 0.0, FAKE, FAKE, FAKE, 4, 2, 16, None) == E
    assert cf.cfp32_qkv_rotary(FAKE, 95, None, 10000.0, FAKE, FAKE, FAKE, 4, 2, 16, None) == E
    assert cf.cfp32_qkv_rotary(None, 96, None, 10000.0, FAKE, FAKE, FAKE, 4, 2, 16, None) == E
    # dimensions or rows x ld extents of 2^48 elements or more
    big = 1 << 40
    assert cf.cfp32_split(FAKE, big, FAKE, FAKE, big, big, 4, None) == E
    assert cf.cfp32_split(FAKE, 1 << 48, FAKE, FAKE, 1 << 48, 1, 1 << 48, None) == E
    assert cf.cfp32_gemm(FAKE, FAKE, 1 << 47, FAKE, 8, FAKE, None, None, 8, 2, 8, 8, None) == E
    assert cf.cfp32_gemm(FAKE, FAKE, 8, FAKE, 8, FAKE, None, None, 8, 2, 8, 1 << 48, None) == E
    assert cf.cfp32_linear(FAKE, (1 << 47) + 8, FAKE, 8, FAKE, 8, 2, 8, 8, FAKE, 1 << 20, None) == E
    assert cf.cfp32_merge(FAKE, FAKE, 1 << 46, FAKE, 8, 4, 8, None) == E


def test_workspace_sizes(lib):
    # M <= 8: FP32 partial sums [chunks][M][2][N rounded up to 512] + 256 B
    # slack.  512-column tiles, at most 256 blocks over tiles x chunks (the
    # largest count within 8 of that which is a multiple of 8 blocks), chunks
    # of whole 32-row stages; a single chunk merges in place and needs nothing.
    # M=1, N=14336 (28 tiles), K=4096: 256 // 28 = 9, 9 * 28 = 252 is not a
    # multiple of 8, 8 * 28 = 224 is: 8 chunks.
    assert cf.cfp32_linear_workspace_bytes(1, 14336, 4096) == 8 * 1 * 2 * 14336 * 4 + 256
    # M=8, N=4096 (8 tiles): 32 chunks of 4 stages.
    assert cf.cfp32_linear_workspace_bytes(8, 4096, 4096) == 32 * 8 * 2 * 4096 * 4 + 256
    # M=1, N=5, K=1: one tile, one stage, one chunk.
    assert cf.cfp32_linear_workspace_bytes(1, 5, 1) == 0
    # M=4, N=300000 (586 tiles): one chunk.
    assert cf.cfp32_linear_workspace_bytes(4, 300000, 4096) == 0
    # M=3, N=1000 (2 tiles), K=777: 128 chunks wanted, ceil(777 / 32) = 25 stages.
    assert cf.cfp32_linear_workspace_bytes(3, 1000, 777) == 25 * 3 * 2 * 1024 * 4 + 256
    assert cf.cfp32_linear_workspace_bytes(8, 4096, 0) == 0
    # cfp32_linear_ex: [K, N] as cfp32_linear; [N, K] needs nothing for M <= 8
    # (one dispatch) and the hi/lo planes above; unknown layouts give 0.
    for shape in [(1, 14336, 4096), (8, 4096, 4096), (3, 1000, 777), (4096, 4096, 4096), (9, 5, 1)]:
        assert cf.cfp32_linear_ex_workspace_bytes(*shape, cf.W_KN) == cf.cfp32_linear_workspace_bytes(*shape)
    assert cf.cfp32_linear_ex_workspace_bytes(1, 14336, 4096, cf.W_NK) == 0
    assert cf.cfp32_linear_ex_workspace_bytes(8, 4096, 4096, cf.W_NK) == 0
    assert cf.cfp32_linear_ex_workspace_bytes(9, 5, 1, cf.W_NK) == 2 * 256 + 256  # no W copy for [N, K]
    assert cf.cfp32_linear_ex_workspace_bytes(9, 5, 1, 7) == 0
    # cfp32_linear_geglu: M <= 8 holds partial sums for all 2F columns, even
    # for a single chunk; M > 8 the hi/lo planes, and up to 16 rows at least
    # those partial sums (the small-M dispatches when W allows 16-byte loads).
    assert cf.cfp32_linear_geglu_workspace_bytes(1, 7168, 4096) == 8 * 1 * 2 * 14336 * 4 + 256
    assert cf.cfp32_linear_geglu_workspace_bytes(2, 16, 8) == 1 * 2 * 2 * 512 * 4 + 256
    # F % 8 != 0 above 8 rows: then a padded copy of W for the small-grid
    # kernel, K x 2 roundup(F, 8) FP16 (here 1 x 16), 256-byte aligned.
    assert cf.cfp32_linear_geglu_workspace_bytes(9, 5, 1) == 1 * 9 * 2 * 512 * 4 + 256 + 256
    assert cf.cfp32_linear_geglu_workspace_bytes(17, 5, 1) == 2 * 512 + 256 + 256  # planes of 17 x 8 FP16
    assert cf.cfp32_linear_geglu_workspace_bytes(17, 8, 1) == 2 * 512 + 256
    assert cf.cfp32_linear_geglu_workspace_bytes(2, 16, 0) == 0
    assert cf.cfp32_linear_workspace_bytes(0, 10, 10) == 0
    assert cf.cfp32_linear_workspace_bytes(100, 10, 0) == 0
    assert cf.cfp32_linear_workspace_bytes(-1, 10, 10) == 0
    # two FP16 planes of M x roundup(K, 8), 256-byte aligned, plus alignment
    # slack; N not a multiple of 8: then a padded copy of W, K x roundup(N, 8)
    # FP16 (here 1 x 8), 256-byte aligned
    assert cf.cfp32_linear_workspace_bytes(9, 5, 1) == 2 * 256 + 256 + 256
    assert cf.cfp32_linear_workspace_bytes(9, 8, 1) == 2 * 256 + 256
    assert cf.cfp32_linear_workspace_bytes(4096, 4096, 4096) == 2 * 4096 * 4096 * 2 + 256
    # M > 8 with fewer than 128 output tiles of 128 x 256 and K % 8 == 0: K is
    # split (chunks x tiles about 256, a multiple of 8 where within reach, at
    # least four 64-deep units per chunk) and FP32 partial sums
    # [chunks][M][2][N rounded up to 64] follow the planes.  M=64, N=4096
    # (16 tiles), K=4096 (64 units): 16 chunks wanted, 4096 // (16 * 64) = 4
    # by the partial-sum bytes.
    planes = 2 * 64 * 4096 * 2
    assert cf.cfp32_linear_workspace_bytes(64, 4096, 4096) == planes + 4 * 64 * 2 * 4096 * 4 + 256
    # From 17 rows, no split where 32 x 128 tiles alone give 192 blocks or
    # more: M=64, N=14336 (2 x 112 = 224 of them): the planes only.
    assert cf.cfp32_linear_workspace_bytes(64, 14336, 4096) == planes + 256
    # At the edge: 33 rows x 12288 columns make exactly 2 x 96 = 192 such
    # tiles (no split), 12160 columns 2 x 95 = 190 (split); 32 rows x 14336
    # columns one row of 112 tiles (split).
    planes33 = 2 * ((33 * 4096 * 2 + 255) // 256 * 256)
    assert cf.cfp32_linear_workspace_bytes(33, 12288, 4096) == planes33 + 256
    assert cf.cfp32_linear_workspace_bytes(33, 12160, 4096) > planes33 + 256
    assert cf.cfp32_linear_workspace_bytes(32, 14336, 4096) > 2 * 32 * 4096 * 2 + 256
    # Above 256 such tiles (40 x 28672: 448), or K above 4096, K is split.
    assert cf.cfp32_linear_workspace_bytes(40, 28672, 4096) > 2 * 40 * 4096 * 2 + 256
    assert cf.cfp32_linear_workspace_bytes(64, 16384, 4096) == planes + 256
    assert cf.cfp32_linear_workspace_bytes(64, 16512, 4096) > planes + 256
    assert cf.cfp32_linear_workspace_bytes(64, 14336, 4104) > 2 * 64 * 4104 * 2 + 256
    # M=40, N=520 (3 tiles), K=4104 (65 units): 85 chunks wanted, 80 for a
    # multiple of 8 blocks, 65 // 4 = 16 by length, 4104 // (16 * 40) = 6 by
    # the partial-sum bytes: 6 chunks, N rounded up to 576.
    planes = 2 * ((40 * 4104 * 2 + 255) // 256 * 256)
    assert cf.cfp32_linear_workspace_bytes(40, 520, 4104) == planes + 6 * 40 * 2 * 576 * 4 + 256
    # M > 64, K % 8 != 0, K too short for two chunks, or enough tiles: planes
    # only (and the padded W copy, 1000 x 784 FP16, when N % 8 != 0).
    assert cf.cfp32_linear_workspace_bytes(300, 777, 1000) == \
        2 * ((300 * 1000 * 2 + 255) // 256 * 256) + 1000 * 784 * 2 + 256
    assert cf.cfp32_linear_workspace_bytes(300, 776, 1000) == 2 * ((300 * 1000 * 2 + 255) // 256 * 256) + 256
    assert cf.cfp32_linear_workspace_bytes(64, 14336, 4100) == 2 * ((64 * 4104 * 2 + 255) // 256 * 256) + 256
    assert cf.cfp32_linear_workspace_bytes(64, 14336, 256) == 2 * 64 * 256 * 2 + 256
    assert cf.cfp32_linear_workspace_bytes(512, 14336, 4096) == 2 * 512 * 4096 * 2 + 256


def test_empty_problems_are_no_ops(lib):
    assert cf.cfp32_split(None, 0, None, None, 0, 0, 5, None) == cf.OK
    assert cf.cfp32_gemm(None, None, 0, None, 0, None, None, None, 0, 0, 8, 8, None) == cf.OK
    assert cf.cfp32_gemm_separate_add(None, None, 0, None, 0, None, None, None, 0, 0, 8, 8, 64, None) == cf.OK
    assert cf.cfp32_linear_geglu(None, 0, None, 0, None, None, 0, 0, 8, 8, None, 0, None) == cf.OK
    assert cf.cfp32_qkv_rotary(None, 0, None, 10000.0, None, None, None, 0, 4, 8, None) == cf.OK
    assert cf.cfp32_linear_geglu(None, 0, None, 0, None, None, 0, 3, 0, 8, None, 0, None) == cf.OK
    assert cf.cfp32_merge(None, None, 0, None, 0, 4, 0, None) == cf.OK
    assert cf.cfp32_linear(None, 0, None, 0, None, 0, 0, 8, 8, None, 0, None) == cf.OK
    assert cf.cfp32_linear_noalloc(None, 0, None, 0, None, 0, 0, 8, 8, None) == cf.OK
    assert cf.cfp32_linear_noalloc(None, 0, None, 0, None, 0, 5, 0, 8, None) == cf.OK


def test_no_cpu_fallback_without_gfx950():
    """With no gfx950 device visible, a valid call must refuse to run."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the refusal path needs a machine without one")
    cf.load_library()
    st = cf.cfp32_split(FAKE, 4, FAKE, FAKE, 4, 1, 4, None)
    assert st == cf.ERR_UNSUPPORTED_DEVICE


def test_binding_raises_without_library(tmp_path, monkeypatch):
    """The Python layer fails loudly when the HIP library is missing."""
    monkeypatch.setattr(cf, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(cf, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        cf.load_library()
