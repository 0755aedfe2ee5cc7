"""Python binding of libcfp32, the compensated-FP32 projection for MI355X.

Argument marshalling only: every step of the projection runs in the HIP
kernels of ``libcfp32.so`` (built by ``compensated_fp32_projection_amd.build``).
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: if the library is missing or the device is not gfx950, calls raise.

Low-level entry points carry the C names and take raw integers (device
pointers, sizes, stream handle):

    cfp32_split, cfp32_gemm, cfp32_gemm_separate_add, cfp32_merge,
    cfp32_linear, cfp32_linear_noalloc, cfp32_linear_workspace_bytes, cfp32_linear_ex,
    cfp32_linear_ex_workspace_bytes, cfp32_linear_geglu,
    cfp32_linear_geglu_workspace_bytes, cfp32_linear_f32, cfp32_qkv_rotary, cfp32_status_string,
    cfp32_last_hip_error

Tensor-level helpers (``split``, ``gemm``, ``merge``, ``linear``) check dtype,
device and layout, pass ``data_ptr()`` and the current stream, and raise
``Cfp32Error`` on a non-zero status.  FP16 tensors may be ``torch.float16``
or ``torch.int16``/``torch.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcfp32.so")

OK, ERR_INVALID_VALUE, ERR_UNSUPPORTED_DEVICE, ERR_HIP, ERR_TOO_LARGE = 0, 1, 2, 3, 4

EXPORTS = (
    "cfp32_status_string",
    "cfp32_last_hip_error",
    "cfp32_split",
    "cfp32_gemm",
    "cfp32_gemm_separate_add",
    "cfp32_merge",
    "cfp32_linear_workspace_bytes",
    "cfp32_linear",
    "cfp32_linear_noalloc",
    "cfp32_linear_ex_workspace_bytes",
    "cfp32_linear_ex",
    "cfp32_linear_geglu_workspace_bytes",
    "cfp32_linear_geglu",
    "cfp32_linear_f32",
    "cfp32_qkv_rotary",
)

W_KN, W_NK = 0, 1


class Cfp32Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = cfp32_status_string(status)
        if status == ERR_HIP:
            msg += f" (hipError_t {cfp32_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


_lib = None


def load_library():
    """Load libcfp32.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m compensated_fp32_projection_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.cfp32_status_string.argtypes = [I32]
    lib.cfp32_status_string.restype = ctypes.c_char_p
    lib.cfp32_last_hip_error.argtypes = []
    lib.cfp32_last_hip_error.restype = I32
    lib.cfp32_split.argtypes = [P, I64, P, P, I64, I64, I64, P]
    lib.cfp32_split.restype = I32
    lib.cfp32_gemm.argtypes = [P, P, I64, P, I64, P, P, P, I64, I64, I64, I64, P]
    lib.cfp32_gemm.restype = I32
    lib.cfp32_gemm_separate_add.argtypes = [P, P, I64, P, I64, P, P, P, I64, I64, I64, I64, I64, P]
    lib.cfp32_gemm_separate_add.restype = I32
    lib.cfp32_merge.argtypes = [P, P, I64, P, I64, I64, I64, P]
    lib.cfp32_merge.restype = I32
    lib.cfp32_linear_workspace_bytes.argtypes = [I64, I64, I64]
    lib.cfp32_linear_workspace_bytes.restype = ctypes.c_size_t
    lib.cfp32_linear.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.cfp32_linear.restype = I32
    lib.cfp32_linear_noalloc.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.cfp32_linear_noalloc.restype = I32
    lib.cfp32_linear_ex_workspace_bytes.argtypes = [I64, I64, I64, I32]
    lib.cfp32_linear_ex_workspace_bytes.restype = ctypes.c_size_t
    lib.cfp32_linear_ex.argtypes = [P, I64, P, I64, I32, P, P, I64, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.cfp32_linear_ex.restype = I32
    lib.cfp32_linear_geglu_workspace_bytes.argtypes = [I64, I64, I64]
    lib.cfp32_linear_geglu_workspace_bytes.restype = ctypes.c_size_t
    lib.cfp32_linear_geglu.argtypes = [P, I64, P, I64, P, P, I64, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.cfp32_linear_geglu.restype = I32
    lib.cfp32_linear_f32.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.cfp32_linear_f32.restype = I32
    lib.cfp32_qkv_rotary.argtypes = [P, I64, P, ctypes.c_double, P, P, P, I64, I64, I64, P]
    lib.cfp32_qkv_rotary.restype = I32
    _lib = lib
    return lib


# -- C entry points, same names, raw integers ------------------------------------

def cfp32_status_string(status: int) -> str:
    return load_library().cfp32_status_string(int(status)).decode()


def cfp32_last_hip_error() -> int:
    return int(load_library().cfp32_last_hip_error())


def cfp32_split(x, ldx, hi, lo, ldh, rows, cols, stream) -> int:
    return int(load_library().cfp32_split(x, ldx, hi, lo, ldh, rows, cols, stream))


def cfp32_gemm(a_hi, a_lo, lda, w, ldw, y, c_hi, c_lo, ldc, M, N, K, stream) -> int:
    return int(load_library().cfp32_gemm(a_hi, a_lo, lda, w, ldw, y, c_hi, c_lo, ldc, M, N, K, stream))


def cfp32_gemm_separate_add(a_hi, a_lo, lda, w, ldw, y, c_hi, c_lo, ldc, M, N, K, k_per_add, stream) -> int:
    return int(load_library().cfp32_gemm_separate_add(a_hi, a_lo, lda, w, ldw, y, c_hi, c_lo, ldc, M, N, K,
                                                      k_per_add, stream))


def cfp32_merge(c_hi, c_lo, ldc, y, ldy, M, N, stream) -> int:
    return int(load_library().cfp32_merge(c_hi, c_lo, ldc, y, ldy, M, N, stream))


def cfp32_linear_workspace_bytes(M, N, K) -> int:
    return int(load_library().cfp32_linear_workspace_bytes(M, N, K))


def cfp32_linear(x, ldx, w, ldw, y, ldy, M, N, K, workspace, workspace_bytes, stream) -> int:
    return int(load_library().cfp32_linear(x, ldx, w, ldw, y, ldy, M, N, K, workspace, workspace_bytes, stream))


def cfp32_linear_noalloc(x, ldx, w, ldw, y, ldy, M, N, K, stream) -> int:
    return int(load_library().cfp32_linear_noalloc(x, ldx, w, ldw, y, ldy, M, N, K, stream))


def cfp32_linear_ex_workspace_bytes(M, N, K, w_layout) -> int:
    return int(load_library().cfp32_linear_ex_workspace_bytes(M, N, K, w_layout))


def cfp32_linear_ex(x, ldx, w, ldw, w_layout, bias, y, ldy, M, N, K, workspace, workspace_bytes, stream) -> int:
    return int(load_library().cfp32_linear_ex(x, ldx, w, ldw, w_layout, bias, y, ldy, M, N, K, workspace,
                                              workspace_bytes, stream))


def cfp32_linear_geglu_workspace_bytes(M, F, K) -> int:
    return int(load_library().cfp32_linear_geglu_workspace_bytes(M, F, K))


def cfp32_linear_geglu(x, ldx, w, ldw, bias, out, ldo, M, F, K, workspace, workspace_bytes, stream) -> int:
    return int(load_library().cfp32_linear_geglu(x, ldx, w, ldw, bias, out, ldo, M, F, K, workspace,
                                                 workspace_bytes, stream))


def cfp32_linear_f32(x, ldx, w, ldw, y, ldy, M, N, K, stream) -> int:
    return int(load_library().cfp32_linear_f32(x, ldx, w, ldw, y, ldy, M, N, K, stream))


def cfp32_qkv_rotary(qkv, ldq, positions, theta, q, k, v, T, H, D, stream) -> int:
    return int(load_library().cfp32_qkv_rotary(qkv, ldq, positions, theta, q, k, v, T, H, D, stream))


# -- tensor helpers -------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _mat(t, dtypes, name):
    """(pointer, rows, cols, ld) of a 2-D device tensor with unit column stride."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name}: expected a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D tensor")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: columns must be contiguous (stride(1) == 1)")
    ld = t.stride(0) if rows > 1 else max(cols, 1)
    return t.data_ptr(), rows, cols, max(ld, cols)


def _f16_dtypes():
    torch = _torch()
    d = [torch.float16, torch.int16]
    if hasattr(torch, "uint16"):
        d.append(torch.uint16)
    return tuple(d)


def _check(status, where):
    if status != OK:
        raise Cfp32Error(status, where)


def split(x, hi=None, lo=None, stream=None):
    """(hi, lo) = split(x): FP32 [rows, cols] -> two FP16 planes (float16)."""
    torch = _torch()
    px, rows, cols, ldx = _mat(x, (torch.float32,), "x")
    if hi is None:
        hi = torch.empty((rows, cols), dtype=torch.float16, device=x.device)
    if lo is None:
        lo = torch.empty((rows, cols), dtype=torch.float16, device=x.device)
    ph, r1, c1, ldh = _mat(hi, _f16_dtypes(), "hi")
    pl, r2, c2, ldl = _mat(lo, _f16_dtypes(), "lo")
    if (r1, c1) != (rows, cols) or (r2, c2) != (rows, cols) or ldh != ldl:
        raise ValueError("hi/lo must be [rows, cols] with one leading dimension")
    _check(cfp32_split(px, ldx, ph, pl, ldh, rows, cols, _stream(stream)), "cfp32_split")
    return hi, lo


def gemm(a_hi, a_lo, w, y=None, c_hi=None, c_lo=None, want_y=True, want_parts=False, stream=None):
    """Dual-product GEMM with fused merge.  Returns (y, c_hi, c_lo); entries not
    requested are None."""
    torch = _torch()
    pa, M, K, lda = _mat(a_hi, _f16_dtypes(), "a_hi")
    pb, M2, K2, lda2 = _mat(a_lo, _f16_dtypes(), "a_lo")
    pw, K3, N, ldw = _mat(w, _f16_dtypes(), "w")
    if (M2, K2) != (M, K) or lda2 != lda or K3 != K:
        raise ValueError("shape mismatch between a_hi, a_lo and w")
    dev = a_hi.device
    if want_y and y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    if want_parts and c_hi is None:
        c_hi = torch.empty((M, N), dtype=torch.float32, device=dev)
        c_lo = torch.empty((M, N), dtype=torch.float32, device=dev)
    outs = [t for t in (y, c_hi, c_lo) if t is not None]
    lds = {(_mat(t, (torch.float32,), "out")[3]) for t in outs}
    if len(lds) != 1:
        raise ValueError("all outputs must share one leading dimension")
    ldc = lds.pop()
    py = y.data_ptr() if y is not None else None
    ph = c_hi.data_ptr() if c_hi is not None else None
    pl = c_lo.data_ptr() if c_lo is not None else None
    _check(cfp32_gemm(pa, pb, lda, pw, ldw, py, ph, pl, ldc, M, N, K, _stream(stream)), "cfp32_gemm")
    return y, c_hi, c_lo


def merge(c_hi, c_lo, y=None, stream=None):
    torch = _torch()
    ph, M, N, ldc = _mat(c_hi, (torch.float32,), "c_hi")
    pl, M2, N2, ldc2 = _mat(c_lo, (torch.float32,), "c_lo")
    if (M2, N2) != (M, N) or ldc2 != ldc:
        raise ValueError("c_hi and c_lo must match")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=c_hi.device)
    py, _, _, ldy = _mat(y, (torch.float32,), "y")
    _check(cfp32_merge(ph, pl, ldc, py, ldy, M, N, _stream(stream)), "cfp32_merge")
    return y


class Workspace:
    """Grow-only device scratch for ``linear`` and ``linear_geglu``.

    The library's kernels read and write the workspace asynchronously, in the
    order of the stream they are launched on, so one Workspace serves one
    stream at a time: calls on different streams that may overlap need one
    each (the helpers' default keeps one per device and stream).  The buffer
    is marked as used by every stream it is handed to (``record_stream``), so
    when it grows, the caching allocator does not give the old buffer to
    anyone else before the work queued on those streams is done."""

    def __init__(self):
        self.buf = None
        self._lock = threading.Lock()

    def get(self, nbytes, device, stream=None):
        torch = _torch()
        if nbytes == 0:
            return None
        with self._lock:
            if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
                self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            buf = self.buf
        if stream is not None and hasattr(stream, "cuda_stream"):
            buf.record_stream(stream)
        return buf


_default_lock = threading.Lock()
_default_ws: dict = {}


def _default_workspace(device, stream) -> Workspace:
    """The helpers' own workspace for (device, stream): calls on different
    streams never share scratch memory."""
    key = (device.index if device.index is not None else -1, _stream(stream))
    with _default_lock:
        ws = _default_ws.get(key)
        if ws is None:
            ws = _default_ws[key] = Workspace()
        return ws


def _stream_obj(stream):
    """The torch stream a helper call runs on (the current one by default)."""
    if stream is None:
        return _torch().cuda.current_stream()
    return stream


def linear(x, w, out=None, workspace: Workspace | None = None, stream=None, bias=None, w_layout: str = "kn"):
    """y = x W (+ bias) with the compensated-FP32 method: x FP32 [M,K]; w FP16
    [K,N] (w_layout "kn") or [N,K] ("nk", a torch.nn.Linear weight); bias
    FP32 [N] or None."""
    torch = _torch()
    if w_layout not in ("kn", "nk"):
        raise ValueError("w_layout must be 'kn' or 'nk'")
    px, M, K, ldx = _mat(x, (torch.float32,), "x")
    pw, r, c, ldw = _mat(w, _f16_dtypes(), "w")
    K2, N = (r, c) if w_layout == "kn" else (c, r)
    if K2 != K:
        raise ValueError("inner dimensions differ")
    pb = None
    if bias is not None:
        if bias.dtype != torch.float32 or bias.device != x.device or bias.dim() != 1 or bias.shape[0] != N \
                or (N > 1 and bias.stride(0) != 1):
            raise ValueError("bias must be a contiguous FP32 [N] tensor on x's device")
        pb = bias.data_ptr()
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    py, M3, N3, ldy = _mat(out, (torch.float32,), "out")
    if (M3, N3) != (M, N):
        raise ValueError("out has the wrong shape")
    layout = W_KN if w_layout == "kn" else W_NK
    need = cfp32_linear_ex_workspace_bytes(M, N, K, layout)
    st = _stream_obj(stream)
    ws = (workspace or _default_workspace(x.device, st)).get(need, x.device, st)
    pws = ws.data_ptr() if ws is not None else None
    _check(cfp32_linear_ex(px, ldx, pw, ldw, layout, pb, py, ldy, M, N, K, pws, need, _stream(st)),
           "cfp32_linear_ex")
    return out


def linear_geglu(x, w, bias=None, out=None, workspace: Workspace | None = None, stream=None):
    """out = gelu(x W[:, :F] + b[:F]) * (x W[:, F:] + b[F:]): x FP32 [M,K], w FP16
    [K, 2F] (gate columns, then up columns), bias FP32 [2F] or None."""
    torch = _torch()
    px, M, K, ldx = _mat(x, (torch.float32,), "x")
    pw, K2, N2, ldw = _mat(w, _f16_dtypes(), "w")
    if K2 != K or N2 % 2:
        raise ValueError("w must be [K, 2F]")
    F = N2 // 2
    pb = None
    if bias is not None:
        if bias.dtype != torch.float32 or bias.device != x.device or bias.dim() != 1 or bias.shape[0] != 2 * F \
                or (F > 0 and bias.stride(0) != 1):
            raise ValueError("bias must be a contiguous FP32 [2F] tensor on x's device")
        pb = bias.data_ptr()
    if out is None:
        out = torch.empty((M, F), dtype=torch.float32, device=x.device)
    po, M3, F3, ldo = _mat(out, (torch.float32,), "out")
    if (M3, F3) != (M, F):
        raise ValueError("out has the wrong shape")
    need = cfp32_linear_geglu_workspace_bytes(M, F, K)
    st = _stream_obj(stream)
    ws = (workspace or _default_workspace(x.device, st)).get(need, x.device, st)
    pws = ws.data_ptr() if ws is not None else None
    _check(cfp32_linear_geglu(px, ldx, pw, ldw, pb, po, ldo, M, F, K, pws, need, _stream(st)),
           "cfp32_linear_geglu")
    return out


def linear_f32(x, w, out=None, stream=None):
    """The true-FP32 projection y = x W: x FP32 [M, K] used as FP32, w FP16
    [K, N] widened exactly, FP32 matrix-unit products and sums."""
    torch = _torch()
    px, M, K, ldx = _mat(x, (torch.float32,), "x")
    pw, K2, N, ldw = _mat(w, _f16_dtypes(), "w")
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    py, M3, N3, ldy = _mat(out, (torch.float32,), "out")
    if (M3, N3) != (M, N):
        raise ValueError("out has the wrong shape")
    _check(cfp32_linear_f32(px, ldx, pw, ldw, py, ldy, M, N, K, _stream(stream)), "cfp32_linear_f32")
    return out


def qkv_rotary(qkv, H: int, D: int, positions=None, theta: float = 10000.0, stream=None):
    """(q, k, v), each FP32 [H, T, D], from a QKV projection output [T, 3 H D]
    (row t = [q | k | v]); q and k rotated (half-split pairs), v copied."""
    torch = _torch()
    pq, T, C, ldq = _mat(qkv, (torch.float32,), "qkv")
    if C < 3 * H * D:
        raise ValueError("qkv has fewer than 3*H*D columns")
    pp = None
    if positions is not None:
        if positions.dtype != torch.int64 or positions.device != qkv.device or positions.numel() != T \
                or not positions.is_contiguous():
            raise ValueError("positions must be a contiguous int64 [T] tensor on qkv's device")
        pp = positions.data_ptr()
    q, k, v = (torch.empty((H, T, D), dtype=torch.float32, device=qkv.device) for _ in range(3))
    _check(cfp32_qkv_rotary(pq, ldq, pp, float(theta), q.data_ptr(), k.data_ptr(), v.data_ptr(), T, H, D,
                            _stream(stream)), "cfp32_qkv_rotary")
    return q, k, v
