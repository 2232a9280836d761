"""CPU oracle for the persistent tile-scheduled GEMM -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP path (persistent_tile_scheduled_amd)
and never imports it.

Contents
  * ``gemm_f64`` / ``gemm_entries_f64``: the fp64 triple-loop product of
    oracle_gemm.c (C = A @ B as in the page "[Feature] Introduce tile scheduler
    #2441", example main(), checked there against torch ``a @ b``).
  * ``round_to``: single round-to-nearest-even of binary64 values into fp16 or
    bf16 bits (IEEE 754 definition, oracle_gemm.c).
  * ``reference_c``: the two steps together, giving the expected C bits.
  * ``schedule`` (module ``oracle.schedule``): the reference tile schedule.

The C part is compiled with gcc into ``liboracle.so`` next to this file
(``build()``); it is rebuilt on first use if missing.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import schedule  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FP16 = 1
BF16 = 2


def build(force: bool = True) -> str:
    """Compile oracle_gemm.c with gcc (-O2, OpenMP, strict IEEE: no fast-math,
    no FMA contraction so every product and sum rounds exactly once)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-shared", "-fPIC", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    d = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_gemm_f64.argtypes = [i64, i64, i64, d, d, d]
    lib.oracle_gemm_f64.restype = None
    lib.oracle_gemm_entries_f64.argtypes = [i64, i64, d, d, i64,
                                            ctypes.POINTER(i64), ctypes.POINTER(i64), d]
    lib.oracle_gemm_entries_f64.restype = None
    lib.oracle_round_one.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.oracle_round_one.restype = ctypes.c_uint16
    lib.oracle_round_array.argtypes = [d, ctypes.POINTER(ctypes.c_uint16), i64, ctypes.c_int]
    lib.oracle_round_array.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def gemm_f64(A, B) -> np.ndarray:
    """C64 = A @ B summed in ascending k in binary64.  A: [M,K], B: [K,N]
    (anything numpy can view as float64; fp16/bf16 inputs must be widened by the
    caller, which is exact)."""
    A = _f64(A)
    B = _f64(B)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm_f64(M, N, K, _ptr(A, ctypes.c_double), _ptr(B, ctypes.c_double),
                            _ptr(C, ctypes.c_double))
    return C


def gemm_entries_f64(A, B, rows, cols) -> np.ndarray:
    """C64 at the given (rows[t], cols[t]) positions only."""
    A = _f64(A)
    B = _f64(B)
    K = A.shape[1]
    N = B.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and equally long")
    if len(rows) and (rows.min() < 0 or rows.max() >= A.shape[0] or cols.min() < 0 or cols.max() >= N):
        raise ValueError("sample position out of range")
    out = np.empty(len(rows), dtype=np.float64)
    _load().oracle_gemm_entries_f64(N, K, _ptr(A, ctypes.c_double), _ptr(B, ctypes.c_double),
                                    len(rows), _ptr(rows, ctypes.c_int64), _ptr(cols, ctypes.c_int64),
                                    _ptr(out, ctypes.c_double))
    return out


def round_to(x, fmt: int) -> np.ndarray:
    """Round binary64 values to fp16 (fmt=1) or bf16 (fmt=2); returns uint16 bits."""
    if fmt not in (FP16, BF16):
        raise ValueError("fmt must be 1 (fp16) or 2 (bf16)")
    x = _f64(x)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_round_array(_ptr(x, ctypes.c_double), _ptr(out, ctypes.c_uint16), x.size, fmt)
    return out


def round_one(x: float, fmt: int) -> int:
    return int(_load().oracle_round_one(float(x), fmt))


def reference_c(A, B, fmt: int):
    """Expected output: (C bits rounded once into fmt, the unrounded C64)."""
    c64 = gemm_f64(A, B)
    return round_to(c64, fmt), c64
