"""FP64 CPU oracle for the dense projection GEMMs and the BF16x3 router GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and never imports it.

The passes are those of the dense projection GEMM family on the pages
("plan the 4096 -> 12288 input gradient with the row-half-release program",
description: forward with a K-major B, input gradient with an MN-major B;
"restore the K1 weight-gradient routes", description: the weight gradient
reduces over T in 64-token K blocks):

    forward          Y[t,n]  = sum_k X[t,k]  W[n,k]
    input gradient   dX[t,k] = sum_n dY[t,n] W[n,k]
    weight gradient  dW[n,k] = sum_t dY[t,n] X[t,k]

BF16 operands are numpy ``uint16`` arrays of bit patterns; FP32 operands are
``float32`` arrays.  Every result is float64.  The summation is in ascending
order of the reduction index, in FP64, from exact operand values.

``mode="bf16x3"`` gives the exact-arithmetic value of the router's BF16x3
emulation (hi = bf16(a), lo = bf16(a - hi), products hi*hi + hi*lo + lo*hi);
``mode="abs"`` gives sum |a*b|, the scale that error bounds are stated in.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dpg_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_MODES = {"exact": 0, "bf16x3": 1, "abs": 2}


def build(force=False, src=_SRC, out=_LIB_PATH):
    """Compile the oracle's C source with gcc (OpenMP, -O3); returns the library path.

    -O3 vectorizes the loop over output columns; every output is still the
    same ascending-index FP64 sum (products of BF16 or FP32 values are exact
    in FP64, so contraction into FMA changes no result)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-Wall", src, "-o", tmp])
        os.replace(tmp, out)
    return out


def _dtype_code(a):
    if a.dtype == np.uint16:
        return 0
    if a.dtype == np.float32:
        return 1
    raise TypeError("oracle operands are uint16 (bf16 bits) or float32, got %s" % a.dtype)


def _view(a):
    """(array, dtype code, row stride, col stride) of a 2-D operand, in elements."""
    if a.ndim != 2:
        raise ValueError("2-D operand expected")
    if a.strides[0] < 0 or a.strides[1] < 0:
        a = np.ascontiguousarray(a)
    it = a.itemsize
    return a, _dtype_code(a), a.strides[0] // it, a.strides[1] // it


class Oracle:
    """One loaded copy of the oracle library (tests may load a second, altered copy)."""

    def __init__(self, lib_path=None):
        lib = ctypes.CDLL(lib_path or build())
        i64, vp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.orc_matmul.argtypes = [i64, i64, i64, vp, ip, i64, i64, vp, ip, i64, i64, ip, vp, i64]
        lib.orc_matmul.restype = ip
        lib.orc_matmul_sampled.argtypes = [i64, vp, ip, i64, i64, vp, ip, i64, i64, ip, vp, vp, i64, vp]
        lib.orc_matmul_sampled.restype = ip
        lib.orc_f32_to_bf16_array.argtypes = [vp, vp, i64]
        lib.orc_f64_to_bf16_via_f32.argtypes = [vp, vp, i64]
        lib.orc_split_bf16x3.argtypes = [vp, vp, vp, i64]
        lib.orc_num_threads.restype = ip
        lib.orc_set_num_threads.argtypes = [ip]
        lib.orc_set_num_threads.restype = None
        self._lib = lib

    def num_threads(self):
        return self._lib.orc_num_threads()

    def set_num_threads(self, n):
        """OpenMP threads of later calls (timing only; results do not depend on it)."""
        self._lib.orc_set_num_threads(int(n))

    def _matmul(self, M, N, R, a, asi, asr, b, bsr, bsj, mode):
        a_arr, adt = a
        b_arr, bdt = b
        out = np.empty((M, N), dtype=np.float64)
        rc = self._lib.orc_matmul(M, N, R, a_arr.ctypes.data, adt, asi, asr,
                                  b_arr.ctypes.data, bdt, bsr, bsj, _MODES[mode], out.ctypes.data, N)
        if rc:
            raise ValueError("oracle rejected the shapes")
        return out

    def _sampled(self, R, a, asi, asr, b, bsr, bsj, mode, ii, jj):
        a_arr, adt = a
        b_arr, bdt = b
        ii = np.ascontiguousarray(ii, dtype=np.int64)
        jj = np.ascontiguousarray(jj, dtype=np.int64)
        out = np.empty(ii.shape[0], dtype=np.float64)
        rc = self._lib.orc_matmul_sampled(R, a_arr.ctypes.data, adt, asi, asr, b_arr.ctypes.data, bdt, bsr, bsj,
                                          _MODES[mode], ii.ctypes.data, jj.ctypes.data, ii.shape[0],
                                          out.ctypes.data)
        if rc:
            raise ValueError("oracle rejected the shapes")
        return out

    def forward(self, x, w, mode="exact", rows=None, cols=None):
        """Y[t,n] = sum_k X[t,k] W[n,k].  X is [T,K], W is [N,K].

        With ``rows``/``cols`` (equal-length index arrays) only Y[rows[p], cols[p]]
        is computed."""
        x, xd, xs0, xs1 = _view(x)
        w, wd, ws0, ws1 = _view(w)
        T, K = x.shape
        N, K2 = w.shape
        if K != K2:
            raise ValueError("K mismatch")
        # A(t,k) = X[t,k]; B(k,n) = W[n,k]
        if rows is not None:
            return self._sampled(K, (x, xd), xs0, xs1, (w, wd), ws1, ws0, mode, rows, cols)
        return self._matmul(T, N, K, (x, xd), xs0, xs1, (w, wd), ws1, ws0, mode)

    def dgrad(self, dy, w, mode="exact", rows=None, cols=None):
        """dX[t,k] = sum_n dY[t,n] W[n,k].  dY is [T,N], W is [N,K]."""
        dy, dd, ds0, ds1 = _view(dy)
        w, wd, ws0, ws1 = _view(w)
        T, N = dy.shape
        N2, K = w.shape
        if N != N2:
            raise ValueError("N mismatch")
        # A(t,n) = dY[t,n]; B(n,k) = W[n,k]
        if rows is not None:
            return self._sampled(N, (dy, dd), ds0, ds1, (w, wd), ws0, ws1, mode, rows, cols)
        return self._matmul(T, K, N, (dy, dd), ds0, ds1, (w, wd), ws0, ws1, mode)

    def wgrad(self, dy, x, mode="exact", rows=None, cols=None):
        """dW[n,k] = sum_t dY[t,n] X[t,k].  dY is [T,N], X is [T,K]; reduces over T."""
        dy, dd, ds0, ds1 = _view(dy)
        x, xd, xs0, xs1 = _view(x)
        T, N = dy.shape
        T2, K = x.shape
        if T != T2:
            raise ValueError("T mismatch")
        # A(n,t) = dY[t,n]; B(t,k) = X[t,k]
        if rows is not None:
            return self._sampled(T, (dy, dd), ds1, ds0, (x, xd), xs0, xs1, mode, rows, cols)
        return self._matmul(N, K, T, (dy, dd), ds1, ds0, (x, xd), xs0, xs1, mode)

    def f32_to_bf16(self, x):
        """Round FP32 values to BF16 (nearest, ties to even); returns uint16 bits."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self._lib.orc_f32_to_bf16_array(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def f64_to_bf16(self, x):
        """FP64 -> FP32 (nearest even) -> BF16 (nearest even); uint16 bits."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        self._lib.orc_f64_to_bf16_via_f32(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def split_bf16x3(self, a):
        """BF16x3 split of FP32 values: (hi, lo) as float32 arrays holding BF16 values."""
        a = np.ascontiguousarray(a, dtype=np.float32)
        hi = np.empty_like(a)
        lo = np.empty_like(a)
        self._lib.orc_split_bf16x3(a.ctypes.data, hi.ctypes.data, lo.ctypes.data, a.size)
        return hi, lo


def bf16_to_f64(bits):
    """BF16 bit patterns -> exact float64 values (a bit shift, no rounding)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def forward(*a, **k):
    return default().forward(*a, **k)


def dgrad(*a, **k):
    return default().dgrad(*a, **k)


def wgrad(*a, **k):
    return default().wgrad(*a, **k)


def f32_to_bf16(x):
    return default().f32_to_bf16(x)


def f64_to_bf16(x):
    return default().f64_to_bf16(x)


def split_bf16x3(a):
    return default().split_bf16x3(a)


def num_threads():
    return default().num_threads()


def set_num_threads(n):
    default().set_num_threads(n)
