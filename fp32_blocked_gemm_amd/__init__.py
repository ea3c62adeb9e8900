"""Python binding of libog: exact and fast fp32 matrix product and NCHW
convolution on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libog.so`` behind the C ABI of ``include/og.h``.  Torch supplies
device memory and the stream (the current torch stream of the tensors'
device).  There is no CPU path: without the built library, or off gfx950,
the calls raise.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libog.so")

OG_OK = 0
OG_ERR_INVALID_ARG = -1
OG_ERR_NOT_EXACT = -2
OG_ERR_DEVICE = -3
OG_ERR_TOO_LARGE = -4

EXACT = 0
FAST = 1
FAST_MFMA = 2  # fast under a stated tolerance (split k, fp32 matrix cores); see og.h
ACT_NONE = 0
ACT_RELU = 1
_ACTS = {None: ACT_NONE, "none": ACT_NONE, "relu": ACT_RELU, ACT_NONE: ACT_NONE, ACT_RELU: ACT_RELU}
_MODES = {"exact": EXACT, "fast": FAST, "fast_mfma": FAST_MFMA, EXACT: EXACT, FAST: FAST,
          FAST_MFMA: FAST_MFMA}

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_lib = None


class OgError(RuntimeError):
    """A non-zero status from libog, with the library's own message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libog status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libog.so.  Raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python fp32_blocked_gemm_amd/build.py` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    L.og_gemm_f32.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, ctypes.c_int]
    L.og_gemm_f32.restype = ctypes.c_int
    L.og_gemm_nt_f32.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, ctypes.c_int]
    L.og_gemm_nt_f32.restype = ctypes.c_int
    L.og_conv2d_f32_ex.argtypes = [_i64] * 16 + [_vp, _vp, _vp, ctypes.c_int]
    L.og_conv2d_f32_ex.restype = ctypes.c_int
    L.og_conv2d_f32_epi.argtypes = [_i64] * 16 + [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int]
    L.og_conv2d_f32_epi.restype = ctypes.c_int
    L.og_conv2d_f32.argtypes = [_i64] * 11 + [_vp, _vp, _vp, ctypes.c_int]
    L.og_conv2d_f32.restype = ctypes.c_int
    L.og_conv2d_out_size.argtypes = [_i64] * 6
    L.og_conv2d_out_size.restype = _i64
    L.og_set_stream.argtypes = [_vp]
    L.og_set_stream.restype = ctypes.c_int
    L.og_get_stream.argtypes = []
    L.og_get_stream.restype = _vp
    L.og_set_variant.argtypes = [ctypes.c_int]
    L.og_set_variant.restype = ctypes.c_int
    L.og_get_variant.argtypes = []
    L.og_get_variant.restype = ctypes.c_int
    L.og_gemm_choice.argtypes = [_i64, _i64, _i64, ctypes.c_int]
    L.og_gemm_choice.restype = ctypes.c_int
    L.og_last_error.argtypes = []
    L.og_last_error.restype = ctypes.c_char_p
    L.og_version.argtypes = []
    L.og_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != OG_OK:
        raise OgError(status, lib().og_last_error().decode(errors="replace"))


def _mode(mode) -> int:
    try:
        return _MODES[mode]
    except KeyError:
        raise ValueError(f"mode must be 'exact', 'fast' or 'fast_mfma', not {mode!r}") from None


def version() -> str:
    return lib().og_version().decode()


def conv2d_out_size(size: int, k: int, stride: int, pad_before: int, pad_after: int,
                    dil: int) -> int:
    return int(lib().og_conv2d_out_size(size, k, stride, pad_before, pad_after, dil))


def set_variant(variant: int):
    """Kernel variant for this thread's later calls (0 = chosen from the shape)."""
    _check(lib().og_set_variant(variant))


def get_variant() -> int:
    return int(lib().og_get_variant())


# ---------------------------------------------------------------------------
# Raw entry points: device pointers and sizes, exactly the C ABI.
# ---------------------------------------------------------------------------

def gemm_choice(m: int, n: int, k: int, mode="fast") -> int:
    """The variant og_gemm_f32's automatic choice runs for an m x n x k
    product (n >= 2) in `mode` (og_gemm_choice)."""
    v = lib().og_gemm_choice(m, n, k, _mode(mode))
    _check(min(v, 0))
    return v


def set_stream(stream_handle: int | None):
    _check(lib().og_set_stream(stream_handle))


def gemm_f32(m, n, k, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, mode):
    _check(lib().og_gemm_f32(m, n, k, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, _mode(mode)))


def gemm_nt_f32(m, n, k, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, mode):
    _check(lib().og_gemm_nt_f32(m, n, k, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, _mode(mode)))


def conv2d_f32_ex(N, Cin, H, W, Cout, G, KH, KW, sH, sW, pT, pL, pB, pR, dH, dW, x_ptr, w_ptr,
                  y_ptr, mode):
    _check(lib().og_conv2d_f32_ex(N, Cin, H, W, Cout, G, KH, KW, sH, sW, pT, pL, pB, pR, dH, dW,
                                  x_ptr, w_ptr, y_ptr, _mode(mode)))


def conv2d_f32(N, Cin, H, W, Cout, G, KH, KW, stride, pad, dil, x_ptr, w_ptr, y_ptr, mode):
    _check(lib().og_conv2d_f32(N, Cin, H, W, Cout, G, KH, KW, stride, pad, dil, x_ptr, w_ptr,
                               y_ptr, _mode(mode)))


# ---------------------------------------------------------------------------
# Torch-tensor conveniences (still only marshalling).
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _use_stream_of(t):
    torch = _torch()
    set_stream(torch.cuda.current_stream(t.device).cuda_stream)


def _ld(t) -> int:
    """Row stride of a 2-D float32 view whose columns are contiguous.

    A view with more than one column must have stride(1) == 1, whatever its
    number of rows (a single row of a column slice is not contiguous); a
    single row's stride is never used, so it passes max(1, cols)."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("columns must be contiguous (stride(1) == 1)")
    if rows <= 1 or cols == 0:
        return max(1, cols)
    return t.stride(0)


def _check_f32_cuda(*ts):
    torch = _torch()
    dev = None
    for t in ts:
        if t.dtype != torch.float32 or not t.is_cuda:
            raise ValueError("tensors must be float32 CUDA tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must be on one device")
    return dev


def gemm(A, B, mode="exact", out=None):
    """C = A @ B on 2-D float32 CUDA tensors (row strides as lda/ldb/ldc)."""
    torch = _torch()
    m, k = A.shape
    k2, n = B.shape
    if k != k2:
        raise ValueError(f"inner sizes differ: {k} vs {k2}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=A.device)
    if tuple(out.shape) != (m, n):
        raise ValueError("out has the wrong shape")
    dev = _check_f32_cuda(A, B, out)
    with torch.cuda.device(dev):
        _use_stream_of(out)
        gemm_f32(m, n, k, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), out.data_ptr(), _ld(out),
                 mode)
    return out


def gemm_nt(A, B, mode="exact", out=None):
    """C = A @ B.T on 2-D float32 CUDA tensors, B given as n x k (row strides as lda/ldb/ldc)."""
    torch = _torch()
    m, k = A.shape
    n, k2 = B.shape
    if k != k2:
        raise ValueError(f"inner sizes differ: {k} vs {k2}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=A.device)
    if tuple(out.shape) != (m, n):
        raise ValueError("out has the wrong shape")
    dev = _check_f32_cuda(A, B, out)
    with torch.cuda.device(dev):
        _use_stream_of(out)
        gemm_nt_f32(m, n, k, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), out.data_ptr(),
                    _ld(out), mode)
    return out


def conv2d(x, w, stride=(1, 1), pad=(0, 0, 0, 0), dil=(1, 1), groups=1, mode="exact",
           out=None, bias=None, act=None, residual=None):
    """NCHW convolution; pad = (top, left, bottom, right).  With bias (Cout),
    act ('relu') or residual (the output's shape) the epilogue runs in the
    same kernels: bias, then activation, then residual."""
    torch = _torch()
    if isinstance(stride, int):
        stride = (stride, stride)
    if isinstance(dil, int):
        dil = (dil, dil)
    if isinstance(pad, int):
        pad = (pad, pad, pad, pad)
    N, Cin, H, W = x.shape
    Cout, cin_g, KH, KW = w.shape
    if not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x and w must be contiguous")
    if cin_g * groups != Cin:
        raise ValueError(f"w.shape[1] * groups = {cin_g * groups} != Cin = {Cin}")
    OH = conv2d_out_size(H, KH, stride[0], pad[0], pad[2], dil[0])
    OW = conv2d_out_size(W, KW, stride[1], pad[1], pad[3], dil[1])
    if OH < 1 or OW < 1:
        raise ValueError("the window does not fit the padded input")
    if out is None:
        out = torch.empty((N, Cout, OH, OW), dtype=torch.float32, device=x.device)
    if tuple(out.shape) != (N, Cout, OH, OW) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [N, Cout, OH, OW] tensor")
    dev = _check_f32_cuda(x, w, out)
    if act not in _ACTS:
        raise ValueError(f"act must be None or 'relu', not {act!r}")
    if bias is not None:
        _check_f32_cuda(bias, out)
        if tuple(bias.shape) != (Cout,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous tensor of Cout floats")
    if residual is not None:
        _check_f32_cuda(residual, out)
        if tuple(residual.shape) != tuple(out.shape) or not residual.is_contiguous():
            raise ValueError("residual must be a contiguous tensor of the output's shape")
    with torch.cuda.device(dev):
        _use_stream_of(out)
        if bias is None and residual is None and _ACTS[act] == ACT_NONE:
            conv2d_f32_ex(N, Cin, H, W, Cout, groups, KH, KW, stride[0], stride[1], pad[0],
                          pad[1], pad[2], pad[3], dil[0], dil[1], x.data_ptr(), w.data_ptr(),
                          out.data_ptr(), mode)
        else:
            _check(lib().og_conv2d_f32_epi(
                N, Cin, H, W, Cout, groups, KH, KW, stride[0], stride[1], pad[0], pad[1], pad[2],
                pad[3], dil[0], dil[1], x.data_ptr(), w.data_ptr(),
                None if bias is None else bias.data_ptr(), _ACTS[act],
                None if residual is None else residual.data_ptr(), out.data_ptr(), _mode(mode)))
    return out
