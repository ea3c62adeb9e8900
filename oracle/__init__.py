"""The CPU oracle: ctypes binding of ``oracle/ogref.c`` on numpy arrays.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check and the
benchmark's CPU-baseline leg import this package.  It never imports the GPU
package and the GPU package never imports it.

The arithmetic lives in ``ogref.c`` (its header names the passages of the
pages it restates); this module only marshals arrays: a 2-D float32 view with
unit column stride passes its row stride as ld.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ogref.c")
LIB = os.path.join(HERE, "libogref.so")

EXACT = 0
FAST = 1

# The flags are part of the oracle's definition: no contraction, no fast-math.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def compile_lib(src: str, out: str, verbose: bool = False) -> str:
    """Compile one oracle source into a shared library with the oracle's flags."""
    cmd = ["gcc", *CFLAGS, "-I", HERE, src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    """Compile ``libogref.so`` (always, as the build step asks)."""
    return compile_lib(SRC, LIB, verbose)


_i64 = ctypes.c_int64
_fp = ctypes.c_void_p


def _ld(a: np.ndarray) -> int:
    """Row stride in elements of a 2-D float32 view with unit column stride."""
    assert a.dtype == np.float32 and a.ndim == 2
    rows, cols = a.shape
    assert a.strides[1] == 4 or cols <= 1 or rows == 0, "columns must be contiguous"
    if rows <= 1 or cols == 0:
        return max(1, cols)  # the row stride is never used
    assert a.strides[0] % 4 == 0 and a.strides[0] // 4 >= cols
    return a.strides[0] // 4


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Oracle:
    """One loaded oracle library.  ``selftest`` runs the fused/unfused check at load."""

    def __init__(self, path: str = LIB, selftest: bool = True):
        L = ctypes.CDLL(path)
        gemm_args = [_i64, _i64, _i64, _fp, _i64, _fp, _i64, _fp, _i64, ctypes.c_int]
        L.ogref_gemm_f32.argtypes = gemm_args
        L.ogref_gemm_f32_rowwise.argtypes = gemm_args
        L.ogref_gemm_f32_at.argtypes = [_i64, _i64, _i64, _fp, _i64, _fp, _i64, _i64, _fp,
                                        _fp, _fp, ctypes.c_int]
        conv_args = [_i64] * 16 + [_fp, _fp, _fp, ctypes.c_int]
        L.ogref_conv2d_f32_ex.argtypes = conv_args
        L.ogref_conv2d_im2col_f32_ex.argtypes = conv_args
        L.ogref_conv2d_f32_at.argtypes = [_i64] * 16 + [_fp, _fp, _i64, _fp, _fp, ctypes.c_int]
        L.ogref_conv_epilogue_f32.argtypes = [_i64, _i64, _i64, _fp, _fp, ctypes.c_int, _fp]
        L.ogref_conv_out_size.argtypes = [_i64] * 6
        L.ogref_conv_out_size.restype = _i64
        for name in ("ogref_gemm_f32", "ogref_gemm_f32_rowwise", "ogref_gemm_f32_at",
                     "ogref_conv2d_f32_ex", "ogref_conv2d_im2col_f32_ex",
                     "ogref_conv2d_f32_at", "ogref_conv_epilogue_f32", "ogref_selftest",
                     "ogref_num_threads",
                     "ogref_set_num_threads"):
            getattr(L, name).restype = ctypes.c_int
        L.ogref_set_num_threads.argtypes = [ctypes.c_int]
        self.L = L
        if selftest:
            rc = L.ogref_selftest()
            if rc != 0:
                raise RuntimeError(f"oracle self-test failed ({rc}): the compiled library does not "
                                   "tell fused from unfused arithmetic")

    def num_threads(self) -> int:
        return int(self.L.ogref_num_threads())

    def set_num_threads(self, n: int) -> int:
        """Threads of later calls (over outputs only: results do not change)."""
        return int(self.L.ogref_set_num_threads(int(n)))

    def gemm(self, A: np.ndarray, B: np.ndarray, mode: int, out: np.ndarray | None = None,
             rowwise: bool = False) -> np.ndarray:
        """C = A*B on 2-D float32 views (row strides taken as lda/ldb/ldc)."""
        m, k = A.shape
        k2, n = B.shape
        assert k == k2
        if out is None:
            out = np.empty((m, n), np.float32)
        assert out.shape == (m, n)
        f = self.L.ogref_gemm_f32_rowwise if rowwise else self.L.ogref_gemm_f32
        rc = f(m, n, k, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(out), _ld(out), mode)
        if rc != 0:
            raise ValueError("oracle gemm: invalid arguments")
        return out

    def gemm_at(self, A: np.ndarray, B: np.ndarray, rows, cols, mode: int) -> np.ndarray:
        """The outputs (rows[t], cols[t]) of A*B, one by one."""
        m, k = A.shape
        n = B.shape[1]
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        out = np.empty(rows.shape[0], np.float32)
        rc = self.L.ogref_gemm_f32_at(m, n, k, _ptr(A), _ld(A), _ptr(B), _ld(B), rows.shape[0],
                                      _ptr(rows), _ptr(cols), _ptr(out), mode)
        if rc != 0:
            raise ValueError("oracle gemm_at: invalid arguments")
        return out

    def conv_out_size(self, size: int, k: int, stride: int, pad_before: int, pad_after: int,
                      dil: int) -> int:
        return int(self.L.ogref_conv_out_size(size, k, stride, pad_before, pad_after, dil))

    def _conv_args(self, x, w, groups, stride, pad, dil):
        N, Cin, H, W = x.shape
        Cout, cin_g, KH, KW = w.shape
        assert x.dtype == np.float32 and w.dtype == np.float32
        assert x.flags.c_contiguous and w.flags.c_contiguous
        assert cin_g * groups == Cin
        sH, sW = stride
        pT, pL, pB, pR = pad
        dH, dW = dil
        OH = self.conv_out_size(H, KH, sH, pT, pB, dH)
        OW = self.conv_out_size(W, KW, sW, pL, pR, dW)
        return ((N, Cin, H, W, Cout, groups, KH, KW, sH, sW, pT, pL, pB, pR, dH, dW),
                (N, Cout, OH, OW))

    def conv2d(self, x: np.ndarray, w: np.ndarray, mode: int, groups: int = 1, stride=(1, 1),
               pad=(0, 0, 0, 0), dil=(1, 1), route: str = "direct") -> np.ndarray:
        """NCHW convolution; pad = (top, left, bottom, right); route 'direct' or 'im2col'."""
        args, yshape = self._conv_args(x, w, groups, stride, pad, dil)
        if yshape[2] < 1 or yshape[3] < 1:
            raise ValueError("oracle conv2d: empty output")
        y = np.empty(yshape, np.float32)
        f = self.L.ogref_conv2d_f32_ex if route == "direct" else self.L.ogref_conv2d_im2col_f32_ex
        rc = f(*args, _ptr(x), _ptr(w), _ptr(y), mode)
        if rc != 0:
            raise ValueError("oracle conv2d: invalid arguments")
        return y

    def conv2d_at(self, x: np.ndarray, w: np.ndarray, flat, mode: int, groups: int = 1,
                  stride=(1, 1), pad=(0, 0, 0, 0), dil=(1, 1)) -> np.ndarray:
        """The outputs at flat indices of y [N, Cout, OH, OW], one by one."""
        args, _ = self._conv_args(x, w, groups, stride, pad, dil)
        flat = np.ascontiguousarray(flat, dtype=np.int64)
        out = np.empty(flat.shape[0], np.float32)
        rc = self.L.ogref_conv2d_f32_at(*args, _ptr(x), _ptr(w), flat.shape[0], _ptr(flat),
                                        _ptr(out), mode)
        if rc != 0:
            raise ValueError("oracle conv2d_at: invalid arguments")
        return out


    def conv_epilogue(self, y: np.ndarray, bias=None, act: int = 0, residual=None) -> np.ndarray:
        """A copy of y [N, Cout, OH, OW] with the convolution epilogue applied:
        + bias[oc], then ReLU (act 1), then + residual, then canonical NaN."""
        y = np.ascontiguousarray(y, dtype=np.float32).copy()
        N, Cout = y.shape[0], y.shape[1]
        ohw = y.shape[2] * y.shape[3]
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        r = None if residual is None else np.ascontiguousarray(residual, dtype=np.float32)
        assert b is None or b.shape == (Cout,)
        assert r is None or r.shape == y.shape
        rc = self.L.ogref_conv_epilogue_f32(N, Cout, ohw, _ptr(y), None if b is None else _ptr(b),
                                            act, None if r is None else _ptr(r))
        if rc != 0:
            raise ValueError("oracle conv_epilogue: invalid activation")
        return y


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``ogref.c`` (compiled first if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default
