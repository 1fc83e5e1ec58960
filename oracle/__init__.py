"""CPU oracle for im2win convolution (ctypes wrapper around liboracle.so).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this package; the HIP library never does. It shares no
code with the HIP path. What each function computes, and the readings of the
pages it rests on, are stated in oracle.c.

A stride argument is either one int (the same stride along rows and
columns) or a pair (sh, sw): row stride, then column stride.

All float inputs are passed as float32 arrays: fp16 inputs are widened to
float32 first, which is exact, so the oracle multiplies the very values the
GPU multiplies and accumulates them in float64.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_i = ctypes.c_int
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float32)


def strides(s):
    """(sh, sw) from one int or a pair."""
    if isinstance(s, (tuple, list)):
        sh, sw = s
        return int(sh), int(sw)
    return int(s), int(s)


class Oracle:
    """The oracle's functions bound to one compiled liboracle.so."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        L.oracle_out_extent.argtypes = [_i, _i, _i]
        L.oracle_out_extent.restype = _i
        for f in (L.oracle_im2win_elems, L.oracle_im2col_elems):
            f.argtypes = [_i] * 8
            f.restype = _i64
        L.oracle_im2win_pack.argtypes = [_p, _p] + [_i] * 9
        L.oracle_im2win_pack.restype = None
        L.oracle_im2col_pack.argtypes = [_p, _p] + [_i] * 10
        L.oracle_im2win_pack_nhwc.argtypes = [_p, _p] + [_i] * 9
        L.oracle_im2win_pack_nhwc.restype = None
        L.oracle_im2col_pack.restype = None
        L.oracle_conv_direct_f64.argtypes = [_p, _p, _p, _p] + [_i] * 9
        L.oracle_conv_direct_f32acc.argtypes = [_p, _p, _p] + [_i] * 9
        L.oracle_conv_im2win_f64.argtypes = [_p, _p, _p] + [_i] * 9
        L.oracle_conv_im2win_f32acc.argtypes = [_p, _p, _p] + [_i] * 9
        L.oracle_conv_points_f64.argtypes = [_p, _p, _p, _i64, _p, _p] + [_i] * 9
        for f in (L.oracle_conv_direct_f64, L.oracle_conv_direct_f32acc,
                  L.oracle_conv_im2win_f64, L.oracle_conv_im2win_f32acc,
                  L.oracle_conv_points_f64):
            f.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = _i
        self.L = L
        self.path = path

    # ---- sizes -----------------------------------------------------------
    def out_extent(self, n_in: int, f: int, s: int) -> int:
        return self.L.oracle_out_extent(n_in, f, s)

    def out_hw(self, Hi, Wi, Hf, Wf, s):
        sh, sw = strides(s)
        return self.out_extent(Hi, Hf, sh), self.out_extent(Wi, Wf, sw)

    def im2win_elems(self, N, Ci, Hi, Wi, Hf, Wf, s) -> int:
        return self.L.oracle_im2win_elems(N, Ci, Hi, Wi, Hf, Wf, *strides(s))

    def im2col_elems(self, N, Ci, Hi, Wi, Hf, Wf, s) -> int:
        return self.L.oracle_im2col_elems(N, Ci, Hi, Wi, Hf, Wf, *strides(s))

    # ---- transform -------------------------------------------------------
    def im2win_pack(self, x: np.ndarray, Hf: int, Wf: int, s) -> np.ndarray:
        """Bit copy of x (N, Ci, Hi, Wi) into the im2win tensor (N, Ci, Ho, Wi*Hf).

        Any 2- or 4-byte element type (float16/uint16/float32/uint32); the
        result has x's dtype.
        """
        x = np.ascontiguousarray(x)
        N, Ci, Hi, Wi = x.shape
        Ho, Wo = self.out_hw(Hi, Wi, Hf, Wf, s)
        if Ho == 0 or Wo == 0:
            raise ValueError("filter larger than input")
        ws = np.empty((N, Ci, Ho, Wi * Hf), dtype=x.dtype)
        self.L.oracle_im2win_pack(_ptr(x), _ptr(ws), N, Ci, Hi, Wi, Hf, Wf, *strides(s),
                                  x.dtype.itemsize)
        return ws

    def im2win_pack_nhwc(self, x: np.ndarray, Hf: int, Wf: int, s) -> np.ndarray:
        """Bit copy of an NHWC x (N, Hi, Wi, Ci) into the NHWC im2win tensor
        (N, Ho, Wi, Hf, Ci): ws[n, ho, w, kh, c] = x[n, ho*sh + kh, w, c]."""
        x = np.ascontiguousarray(x)
        N, Hi, Wi, Ci = x.shape
        Ho, Wo = self.out_hw(Hi, Wi, Hf, Wf, s)
        if Ho == 0 or Wo == 0:
            raise ValueError("filter larger than input")
        ws = np.empty((N, Ho, Wi, Hf, Ci), dtype=x.dtype)
        self.L.oracle_im2win_pack_nhwc(_ptr(x), _ptr(ws), N, Ci, Hi, Wi, Hf, Wf, *strides(s),
                                       x.dtype.itemsize)
        return ws

    def im2col_pack(self, x: np.ndarray, Hf: int, Wf: int, s, KP: int | None = None) -> np.ndarray:
        """Bit copy of x (N, Ci, Hi, Wi) into the im2col matrix (N*Ho*Wo, KP):
        each row one output pixel's receptive field in (ci, kh, kw) order, then
        zeros (KP defaults to Ci*Hf*Wf)."""
        x = np.ascontiguousarray(x)
        N, Ci, Hi, Wi = x.shape
        Ho, Wo = self.out_hw(Hi, Wi, Hf, Wf, s)
        if Ho == 0 or Wo == 0:
            raise ValueError("filter larger than input")
        K = Ci * Hf * Wf
        KP = K if KP is None else KP
        if KP < K:
            raise ValueError("row pitch below Ci*Hf*Wf")
        col = np.empty((N * Ho * Wo, KP), dtype=x.dtype)
        self.L.oracle_im2col_pack(_ptr(x), _ptr(col), N, Ci, Hi, Wi, Hf, Wf, *strides(s), KP,
                                  x.dtype.itemsize)
        return col

    # ---- convolution -----------------------------------------------------
    def _dims(self, x, w, s):
        N, Ci, Hi, Wi = x.shape
        Co, Ci2, Hf, Wf = w.shape
        if Ci2 != Ci:
            raise ValueError("channel mismatch")
        Ho, Wo = self.out_hw(Hi, Wi, Hf, Wf, s)
        if Ho == 0 or Wo == 0:
            raise ValueError("filter larger than input")
        return N, Ci, Hi, Wi, Co, Hf, Wf, Ho, Wo

    def conv_direct(self, x, w, s, with_absdot: bool = False):
        """Direct convolution in float64: y (N, Co, Ho, Wo) [, sum |x*w| per output]."""
        x, w = _f32(x), _f32(w)
        N, Ci, Hi, Wi, Co, Hf, Wf, Ho, Wo = self._dims(x, w, s)
        y = np.empty((N, Co, Ho, Wo), dtype=np.float64)
        a = np.empty_like(y) if with_absdot else None
        self.L.oracle_conv_direct_f64(_ptr(x), _ptr(w), _ptr(y), _ptr(a),
                                      N, Ci, Hi, Wi, Co, Hf, Wf, *strides(s))
        return (y, a) if with_absdot else y

    def conv_direct_f32acc(self, x, w, s):
        x, w = _f32(x), _f32(w)
        N, Ci, Hi, Wi, Co, Hf, Wf, Ho, Wo = self._dims(x, w, s)
        y = np.empty((N, Co, Ho, Wo), dtype=np.float32)
        self.L.oracle_conv_direct_f32acc(_ptr(x), _ptr(w), _ptr(y), N, Ci, Hi, Wi, Co, Hf, Wf,
                                         *strides(s))
        return y

    def _im2win_dims(self, ws, w, Hi, Wi, s):
        N, Ci = ws.shape[0], ws.shape[1]
        Co, Ci2, Hf, Wf = w.shape
        Ho, Wo = self.out_hw(Hi, Wi, Hf, Wf, s)
        if Ci2 != Ci or ws.shape != (N, Ci, Ho, Wi * Hf):
            raise ValueError("im2win tensor does not match the shapes")
        return N, Ci, Co, Hf, Wf, Ho, Wo

    def conv_im2win(self, ws, w, Hi: int, Wi: int, s):
        """im2win convolution (float64) on a packed tensor from im2win_pack."""
        ws, w = _f32(ws), _f32(w)
        N, Ci, Co, Hf, Wf, Ho, Wo = self._im2win_dims(ws, w, Hi, Wi, s)
        y = np.empty((N, Co, Ho, Wo), dtype=np.float64)
        self.L.oracle_conv_im2win_f64(_ptr(ws), _ptr(w), _ptr(y), N, Ci, Hi, Wi, Co, Hf, Wf,
                                      *strides(s))
        return y

    def conv_im2win_f32acc(self, ws, w, Hi: int, Wi: int, s):
        ws, w = _f32(ws), _f32(w)
        N, Ci, Co, Hf, Wf, Ho, Wo = self._im2win_dims(ws, w, Hi, Wi, s)
        y = np.empty((N, Co, Ho, Wo), dtype=np.float32)
        self.L.oracle_conv_im2win_f32acc(_ptr(ws), _ptr(w), _ptr(y), N, Ci, Hi, Wi, Co,
                                         Hf, Wf, *strides(s))
        return y

    def conv_points(self, x, w, s, idx: np.ndarray):
        """Direct convolution (float64) at flat NCHW output indices: (y, absdot)."""
        x, w = _f32(x), _f32(w)
        N, Ci, Hi, Wi, Co, Hf, Wf, Ho, Wo = self._dims(x, w, s)
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        if idx.size and (idx.min() < 0 or idx.max() >= N * Co * Ho * Wo):
            raise ValueError("output index out of range")
        y = np.empty(idx.shape, dtype=np.float64)
        a = np.empty(idx.shape, dtype=np.float64)
        self.L.oracle_conv_points_f64(_ptr(x), _ptr(w), _ptr(idx), idx.size, _ptr(y), _ptr(a),
                                      N, Ci, Hi, Wi, Co, Hf, Wf, *strides(s))
        return y, a

    def num_threads(self) -> int:
        return self.L.oracle_num_threads()


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (compiled with gcc on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def __getattr__(name):
    # Module-level shortcuts: oracle.conv_direct(...) == oracle.default().conv_direct(...)
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
