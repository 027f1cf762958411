"""ORACLE (test infrastructure only): loader of oracle/e4m3_cast.c, the plain-C e4m3 cast used to
check the device cast over every fp32 bit pattern (the build step compiles it with gcc; a test
that finds no build compiles it itself)."""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "e4m3_cast.c")
LIB = os.path.join(HERE, "libe4m3_oracle.so")
_lib = None


def build() -> str:
    """Compile e4m3_cast.c into oracle/libe4m3_oracle.so (plain IEEE arithmetic: no fast-math, no
    contraction of the fp32 product)."""
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-o", tmp, SRC, "-lm"],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = ctypes.CDLL(LIB)
        _lib.oracle_e4m3_cast.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
        _lib.oracle_e4m3_cast.restype = None
        _lib.oracle_e4m3_cast_patterns.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
        _lib.oracle_e4m3_cast_patterns.restype = None
    return _lib


def cast(x, scale: float) -> np.ndarray:
    """e4m3fn codes of the fp32 values x at `scale` (module docstring of e4m3_cast.c)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_cast(x.ctypes.data, x.size, float(scale), q.ctypes.data)
    return q


def cast_patterns(first: int, n: int, scale: float, threads: int = 8) -> np.ndarray:
    """Codes of the fp32 bit patterns first .. first + n - 1 at `scale`, split over threads (the
    C calls release the interpreter lock)."""
    q = np.empty(n, np.uint8)
    L = lib()
    parts = max(1, min(threads, n // (1 << 16)))
    bounds = [n * i // parts for i in range(parts + 1)]

    def run(i):
        a, b = bounds[i], bounds[i + 1]
        L.oracle_e4m3_cast_patterns((first + a) & 0xFFFFFFFF, b - a, float(scale), q.ctypes.data + a)

    with ThreadPoolExecutor(parts) as ex:
        list(ex.map(run, range(parts)))
    return q
