"""ctypes wrappers of the oracle's C loops (oracle/gemv.c).

TEST INFRASTRUCTURE ONLY."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .formats import E2M1, E4M3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "_gemv.so")
_E8M0 = np.ldexp(1.0, np.arange(256) - 127)  # byte 255 (NaN) never occurs in the inputs
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(os.path.join(_HERE, "gemv.c")):
            from .build import build
            build(verbose=False)
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _rows(x):
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
    assert x.shape[0] <= 64
    return x


def gemv_mxfp8(w, s, x):
    """x [R, K] float64 times the dequantized MXFP8 tile32 weight [N, K] -> [R, N] float64."""
    w = np.ascontiguousarray(w, dtype=np.uint8); s = np.ascontiguousarray(s, dtype=np.uint8)
    N, K = w.shape
    x = _rows(x)
    y = np.empty((x.shape[0], N))
    _load().oracle_gemv_mxfp8(_p(w), _p(s), N, K, _p(E4M3), _p(_E8M0), _p(x), x.shape[0], _p(y))
    return y


def gemv_fp8b128(w, s, x):
    w = np.ascontiguousarray(w, dtype=np.uint8); s = np.ascontiguousarray(s, dtype=np.float32)
    N, K = w.shape
    x = _rows(x)
    y = np.empty((x.shape[0], N))
    _load().oracle_gemv_fp8b128(_p(w), _p(s), N, K, _p(E4M3), _p(x), x.shape[0], _p(y))
    return y


def gemv_mxfp4(w, s, x):
    w = np.ascontiguousarray(w, dtype=np.uint8); s = np.ascontiguousarray(s, dtype=np.uint8)
    N, K2 = w.shape
    x = _rows(x)
    y = np.empty((x.shape[0], N))
    _load().oracle_gemv_mxfp4(_p(w), _p(s), N, 2 * K2, _p(E2M1), _p(_E8M0), _p(x), x.shape[0], _p(y))
    return y
