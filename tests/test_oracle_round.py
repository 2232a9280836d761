"""Pins for the oracle's binary64 -> fp16/bf16 round-to-nearest-even.

Checked against: every bit pattern of both formats (round trip), numpy's own
binary64 -> binary16 conversion (a library routine), and a brute-force nearest
search with exact rationals (tests/exact.py) on random, midpoint,
near-midpoint, subnormal and overflow inputs.
"""

import math
import struct

import numpy as np
import pytest

import oracle
from tests import exact

FP16, BF16 = 1, 2


def _all_fp16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return bits, bits.view(np.float16).astype(np.float64)


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    return bits.astype(np.uint16), vals


@pytest.mark.parametrize("fmt", [FP16, BF16])
def test_round_trip_every_pattern(fmt):
    bits, vals = _all_fp16_values() if fmt == FP16 else _all_bf16_values()
    out = oracle.round_to(vals, fmt)
    nan = np.isnan(vals)
    assert np.array_equal(out[~nan], bits[~nan])
    # NaN stays NaN (exponent all ones, fraction non-zero)
    exp_mask, frac_mask = (0x7C00, 0x03FF) if fmt == FP16 else (0x7F80, 0x007F)
    assert np.all((out[nan] & exp_mask) == exp_mask)
    assert np.all((out[nan] & frac_mask) != 0)


def _probe_values(fmt, rng, count=20000):
    """Random doubles over the whole range plus exact midpoints and their
    binary64 neighbours, between every pair of adjacent format values."""
    _, vals = _all_fp16_values() if fmt == FP16 else _all_bf16_values()
    finite = vals[np.isfinite(vals)]
    pos = np.unique(finite[finite >= 0])
    idx = rng.integers(0, len(pos) - 1, size=count)
    lo, hi = pos[idx], pos[idx + 1]
    mid = (lo + hi) / 2                         # exact in binary64
    up = np.nextafter(mid, np.inf)
    dn = np.nextafter(mid, -np.inf)
    frac = lo + (hi - lo) * rng.random(count)
    top = pos[-1]
    edge = np.array([top, top + (top - pos[-2]) / 2, np.nextafter(top + (top - pos[-2]) / 2, 0),
                     top * 2, 1e300, np.inf, 5e-324, pos[1] / 2, np.nextafter(pos[1] / 2, 1),
                     pos[1] * 1.5, 0.0])
    x = np.concatenate([mid, up, dn, frac, edge])
    sign = np.where(rng.random(len(x)) < 0.5, -1.0, 1.0)
    return x * sign


def test_fp16_matches_numpy_conversion():
    rng = np.random.default_rng(11)
    x = _probe_values(FP16, rng)
    ref = x.astype(np.float16).view(np.uint16)
    out = oracle.round_to(x, FP16)
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("fmt", [FP16, BF16])
def test_matches_bruteforce_nearest(fmt):
    rng = np.random.default_rng(12 + fmt)
    x = _probe_values(fmt, rng, count=1500)
    out = oracle.round_to(x, fmt)
    ref = np.array([exact.nearest_bits(float(v), fmt) for v in x], dtype=np.uint16)
    assert np.array_equal(out, ref)


def test_ties_and_edges_by_hand():
    # fp16: 1 + 2^-11 sits half way between 1 and 1 + 2^-10: ties to even -> 1.0
    assert oracle.round_one(1 + 2 ** -11, FP16) == 0x3C00
    assert oracle.round_one(1 + 3 * 2 ** -11, FP16) == 0x3C02
    assert oracle.round_one(65504.0, FP16) == 0x7BFF
    assert oracle.round_one(65519.99, FP16) == 0x7BFF
    assert oracle.round_one(65520.0, FP16) == 0x7C00        # overflow to +inf
    assert oracle.round_one(-65520.0, FP16) == 0xFC00
    assert oracle.round_one(2 ** -24, FP16) == 0x0001       # smallest subnormal
    assert oracle.round_one(2 ** -25, FP16) == 0x0000       # tie -> even (zero)
    assert oracle.round_one(2 ** -25 * 1.0000001, FP16) == 0x0001
    assert oracle.round_one(-0.0, FP16) == 0x8000
    assert oracle.round_one(2 ** -14, FP16) == 0x0400       # smallest normal
    # bf16: 1 + 2^-8 is half way between 1 and 1 + 2^-7
    assert oracle.round_one(1 + 2 ** -8, BF16) == 0x3F80
    assert oracle.round_one(1 + 3 * 2 ** -8, BF16) == 0x3F82
    assert oracle.round_one(-2.0, BF16) == 0xC000
    big = struct.unpack("<f", struct.pack("<I", 0x7F7F0000))[0]
    assert oracle.round_one(big, BF16) == 0x7F7F
    assert oracle.round_one(big + 2.0 ** 119, BF16) == 0x7F80       # tie above max -> inf
    assert oracle.round_one(big + 2.0 ** 118, BF16) == 0x7F7F
    assert oracle.round_one(2.0 ** -133, BF16) == 0x0001            # smallest subnormal
    assert oracle.round_one(math.inf, BF16) == 0x7F80
