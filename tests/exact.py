"""Exact-arithmetic helpers for pinning the oracle (tests only).

Rounding here is a brute-force nearest search over the table of every finite
value of the format, compared with exact rationals -- a construction that
shares nothing with the oracle's bit-level rounding.
"""

from __future__ import annotations

import bisect
import struct
from fractions import Fraction

import numpy as np

_TABLES = {}


def decode(bits: int, fmt: int) -> float:
    """Exact value of one fp16 (fmt=1) or bf16 (fmt=2) bit pattern."""
    if fmt == 1:
        return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def table(fmt: int):
    """Sorted non-negative finite values of the format with their bit patterns."""
    if fmt not in _TABLES:
        max_bits = 0x7BFF if fmt == 1 else 0x7F7F
        vals = [decode(b, fmt) for b in range(0, max_bits + 1)]
        assert all(vals[i] < vals[i + 1] for i in range(len(vals) - 1))
        _TABLES[fmt] = vals
    return _TABLES[fmt]


def nearest_bits(x, fmt: int) -> int:
    """Round x (float or Fraction) to the nearest format value, ties to the even
    bit pattern, overflow to infinity -- by searching the value table."""
    sign = 0x8000 if (x < 0 or (isinstance(x, float) and np.signbit(x))) else 0
    if isinstance(x, float) and np.isinf(x):
        return sign | (0x7C00 if fmt == 1 else 0x7F80)
    ax = Fraction(abs(x))
    vals = table(fmt)
    top = Fraction(vals[-1])
    half_ulp_top = (top - Fraction(vals[-2])) / 2
    if ax >= top + half_ulp_top:
        return sign | (0x7C00 if fmt == 1 else 0x7F80)
    i = bisect.bisect_right(vals, float(ax)) - 1
    # float(ax) may round; step so that vals[i] <= ax < vals[i+1] exactly
    while i > 0 and Fraction(vals[i]) > ax:
        i -= 1
    while i + 1 < len(vals) and Fraction(vals[i + 1]) <= ax:
        i += 1
    if i + 1 >= len(vals):
        return sign | i
    lo, hi = Fraction(vals[i]), Fraction(vals[i + 1])
    dlo, dhi = ax - lo, hi - ax
    if dlo < dhi:
        pick = i
    elif dhi < dlo:
        pick = i + 1
    else:
        pick = i if i % 2 == 0 else i + 1
    return sign | pick
