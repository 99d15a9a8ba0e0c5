"""Build and call the plain-C fp64 oracle (grinqh_oracle.c) through ctypes.

TEST INFRASTRUCTURE ONLY (tests, smoke check, bench CPU baseline).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "grinqh_oracle.c")
LIB = os.path.join(HERE, "libgrinqh_oracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        d = ctypes.POINTER(ctypes.c_double)
        u8 = ctypes.POINTER(ctypes.c_uint8)
        u32 = ctypes.POINTER(ctypes.c_uint32)
        i = ctypes.c_int
        lib.oracle_assign_bits.argtypes = [d, d, i, i, u8]
        lib.oracle_assign_bits.restype = None
        lib.oracle_pack.argtypes = [u8, i, i, i, u32]
        lib.oracle_pack.restype = None
        lib.oracle_gemv.argtypes = [d, d, u8, d, d, i, i, i, u8, d]
        lib.oracle_gemv.restype = None
        _lib = lib
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def assign_bits(x, theta, b_max: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    th = np.ascontiguousarray(theta, dtype=np.float64)
    out = np.zeros(x.size, dtype=np.uint8)
    _load().oracle_assign_bits(_ptr(x, ctypes.c_double), _ptr(th, ctypes.c_double),
                               x.size, b_max, _ptr(out, ctypes.c_uint8))
    return out


def pack_planes(q, b_max: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    d_out, d_in = q.shape
    W = ((d_out + 63) // 64) * 4
    planes = np.zeros((d_in, b_max // 2, W), dtype=np.uint32)
    _load().oracle_pack(_ptr(q, ctypes.c_uint8), d_in, d_out, b_max,
                        _ptr(planes, ctypes.c_uint32))
    return planes


def gemv(x, theta, q_rows, s, z, b_max: int) -> np.ndarray:
    """y for the output channels whose code rows are given (q_rows = q[cols, :])."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    th = np.ascontiguousarray(theta, dtype=np.float64)
    q_rows = np.ascontiguousarray(q_rows, dtype=np.uint8)
    n_out, d_in = q_rows.shape
    s = np.ascontiguousarray(s, dtype=np.float64)
    z = np.ascontiguousarray(z, dtype=np.float64)
    bits = np.zeros(d_in, dtype=np.uint8)
    y = np.zeros(n_out, dtype=np.float64)
    _load().oracle_gemv(_ptr(x, ctypes.c_double), _ptr(th, ctypes.c_double),
                        _ptr(q_rows, ctypes.c_uint8), _ptr(s, ctypes.c_double),
                        _ptr(z, ctypes.c_double), d_in, n_out, b_max,
                        _ptr(bits, ctypes.c_uint8), _ptr(y, ctypes.c_double))
    return y
