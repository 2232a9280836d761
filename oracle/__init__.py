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
  * ``e4m3_decode`` / ``e8m0_decode`` / ``mx_gemm_f64`` / ``mx_reference_c``:
    the block-scaled FP8 (OCP MX) product of oracle_mx.c.

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
_SRC_MX = os.path.join(_HERE, "oracle_mx.c")
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
            "-shared", "-fPIC", "-std=c11", _SRC, _SRC_MX, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
            os.path.getmtime(_SRC), os.path.getmtime(_SRC_MX)):
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
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    u8 = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_decode.restype = ctypes.c_double
    lib.oracle_mx_gemm_f64.argtypes = [i64, i64, i64, u8, u8, u8, u8, d]
    lib.oracle_mx_gemm_f64.restype = ctypes.c_int
    lib.oracle_mx_gemm_entries_f64.argtypes = [i64, u8, u8, u8, u8, i64, ctypes.POINTER(i64),
                                               ctypes.POINTER(i64), d]
    lib.oracle_mx_gemm_entries_f64.restype = None
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads used by later oracle calls (timing only; results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


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


# ---------------------------------------------------------------- MX (block-scaled FP8)
def e4m3_decode(codes) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> binary64 values (oracle_mx.c)."""
    lib = _load()
    table = np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e8m0_decode(codes) -> np.ndarray:
    """OCP E8M0 scale codes (uint8) -> binary64 values 2^(c-127), NaN for 255."""
    lib = _load()
    table = np.array([lib.oracle_e8m0_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def _u8(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.uint8)


def _mx_args(A, SFA, B, SFB):
    A, SFA, B, SFB = _u8(A), _u8(SFA), _u8(B), _u8(SFB)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2 or K % 32 or SFA.shape != (M, K // 32) or SFB.shape != (N, K // 32):
        raise ValueError("MX shapes: A[M,K], SFA[M,K/32], B[N,K], SFB[N,K/32], K % 32 == 0")
    return A, SFA, B, SFB, M, N, K


def mx_gemm_f64(A, SFA, B, SFB) -> np.ndarray:
    """C64[i,j] = sum_k x(A[i,k]) s(SFA[i,k/32]) x(B[j,k]) s(SFB[j,k/32]) in binary64,
    ascending k (operands decoded once; every term is exact, so the order of a
    term's four factors does not matter)."""
    A, SFA, B, SFB, M, N, K = _mx_args(A, SFA, B, SFB)
    C = np.empty((M, N), dtype=np.float64)
    u8 = ctypes.c_uint8
    if _load().oracle_mx_gemm_f64(M, N, K, _ptr(A, u8), _ptr(SFA, u8), _ptr(B, u8), _ptr(SFB, u8),
                                  _ptr(C, ctypes.c_double)) != 0:
        raise MemoryError("MX oracle: cannot allocate the decoded operands")
    return C


def mx_gemm_entries_f64(A, SFA, B, SFB, rows, cols) -> np.ndarray:
    A, SFA, B, SFB, M, N, K = _mx_args(A, SFA, B, SFB)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if len(rows) and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise ValueError("sample position out of range")
    out = np.empty(len(rows), dtype=np.float64)
    u8 = ctypes.c_uint8
    _load().oracle_mx_gemm_entries_f64(K, _ptr(A, u8), _ptr(SFA, u8), _ptr(B, u8), _ptr(SFB, u8),
                                       len(rows), _ptr(rows, ctypes.c_int64), _ptr(cols, ctypes.c_int64),
                                       _ptr(out, ctypes.c_double))
    return out


def mx_reference_c(A, SFA, B, SFB, fmt: int = BF16):
    """Expected MX output: (C bits rounded once into fmt, the unrounded C64)."""
    c64 = mx_gemm_f64(A, SFA, B, SFB)
    return round_to(c64, fmt), c64
