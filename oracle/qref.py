"""ctypes binding of the C half of the CPU oracle (qref.c).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qref.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile qref.c into liboracle.so (plain gcc, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-std=c99", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_half_to_double.restype = ctypes.c_double
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_dequant.restype = ctypes.c_int
        L.orc_dequant.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_void_p]
        L.orc_gemv.restype = ctypes.c_int
        L.orc_gemv.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def half_to_double(bits: int) -> float:
    return lib().orc_half_to_double(int(bits) & 0xFFFF)


def dequant(qtype: int, raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Decode GGUF blocks [rows, cols/32*bb] -> fp64 [rows, cols]."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.float64)
    rc = lib().orc_dequant(qtype, raw.ctypes.data, rows, cols, out.ctypes.data)
    if rc:
        raise ValueError("orc_dequant: bad arguments")
    return out


def gemv(qtype: int, raw: np.ndarray, rows: int, cols: int, x: np.ndarray) -> np.ndarray:
    """y = W x in fp64.  x: [cols] or [n, cols] (n <= 64); returns the same leading shape."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    xx = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
    if xx.shape[1] != cols:
        raise ValueError("x has the wrong length")
    n = xx.shape[0]
    y = np.empty((n, rows), dtype=np.float64)
    rc = lib().orc_gemv(qtype, raw.ctypes.data, rows, cols, n, xx.ctypes.data, y.ctypes.data)
    if rc:
        raise ValueError("orc_gemv: bad arguments")
    return y[0] if np.ndim(x) == 1 else y
