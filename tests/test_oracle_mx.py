"""Pins for the block-scaled FP8 oracle (oracle/oracle_mx.c).

The element and scale formats follow the OCP Microscaling Formats
specification (FP8 E4M3 elements, E8M0 scales, 32-element blocks along K).
Fixed independently of the oracle by: torch's own float8_e4m3fn decoding of all
256 codes, the landmark values the specification tabulates for E4M3 and E8M0,
products that reduce to a plain library matmul (unit scales), exact scaling
identities, and exact rational arithmetic on small cases.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))   # -0 for 0x80


def test_e4m3_specification_landmarks():
    d = lambda c: float(oracle.e4m3_decode([c])[0])
    assert d(0x7E) == 448.0                    # largest finite
    assert d(0x08) == 2.0 ** -6                # smallest normal
    assert d(0x07) == 0.875 * 2.0 ** -6        # largest subnormal
    assert d(0x01) == 2.0 ** -9                # smallest subnormal
    assert d(0x38) == 1.0 and d(0xB8) == -1.0
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)            # positive codes increase strictly
    neg = oracle.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def test_e8m0_is_a_power_of_two():
    for c in range(255):
        assert float(oracle.e8m0_decode([c])[0]) == math.ldexp(1.0, c - 127)
    assert math.isnan(float(oracle.e8m0_decode([255])[0]))


def _codes(rng, shape, lo_exp=4, hi_exp=10):
    """Random finite E4M3 codes with exponent fields in [lo_exp, hi_exp] (no NaN)."""
    s = rng.integers(0, 2, shape) << 7
    e = rng.integers(lo_exp, hi_exp + 1, shape) << 3
    m = rng.integers(0, 8, shape)
    return (s | e | m).astype(np.uint8)


def test_unit_scales_reduce_to_a_plain_matmul():
    """With every scale 2^0 the MX product is the ordinary product of the decoded
    elements; exponents are kept in a band where every sum is exact, so numpy's
    matmul (any summation order) must agree bit for bit."""
    rng = np.random.default_rng(1)
    M, N, K = 9, 7, 96
    A, B = _codes(rng, (M, K)), _codes(rng, (N, K))
    ones = lambda r: np.full((r, K // 32), 127, np.uint8)
    got = oracle.mx_gemm_f64(A, ones(M), B, ones(N))
    xa = torch.from_numpy(A).view(torch.float8_e4m3fn).double().numpy()
    xb = torch.from_numpy(B).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got, xa @ xb.T)


def test_scale_steps_are_exact_powers_of_two():
    """Raising one block's scale code by one doubles exactly that block's share."""
    rng = np.random.default_rng(2)
    M, N, K = 4, 5, 96
    A, B = _codes(rng, (M, K)), _codes(rng, (N, K))
    SA = np.full((M, 3), 127, np.uint8)
    SB = rng.integers(125, 130, (N, 3)).astype(np.uint8)
    base = oracle.mx_gemm_f64(A, SA, B, SB)
    for blk in range(3):
        SA2 = SA.copy()
        SA2[:, blk] += 1
        only = np.zeros_like(A)
        only[:, 32 * blk:32 * blk + 32] = A[:, 32 * blk:32 * blk + 32]
        share = oracle.mx_gemm_f64(only, SA, B, SB)
        assert np.array_equal(oracle.mx_gemm_f64(A, SA2, B, SB), base + share)


def test_brute_force_rationals():
    rng = np.random.default_rng(3)
    M, N, K = 3, 4, 64
    A, B = _codes(rng, (M, K), 1, 14), _codes(rng, (N, K), 1, 14)
    SA = rng.integers(110, 145, (M, 2)).astype(np.uint8)
    SB = rng.integers(110, 145, (N, 2)).astype(np.uint8)
    got = oracle.mx_gemm_f64(A, SA, B, SB)

    def q(c):  # E4M3 value as an exact fraction, from the bit fields
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        return -v if s else v

    for i in range(M):
        for j in range(N):
            exact = sum(q(int(A[i, k])) * Fraction(2) ** (int(SA[i, k // 32]) - 127) *
                        q(int(B[j, k])) * Fraction(2) ** (int(SB[j, k // 32]) - 127) for k in range(K))
            scale = sum(abs(q(int(A[i, k])) * q(int(B[j, k]))) * Fraction(2) ** (int(SA[i, k // 32]) + int(SB[j, k // 32]) - 254)
                        for k in range(K))
            assert abs(Fraction(got[i, j]) - exact) <= scale * Fraction(2) ** -50


def test_nan_scale_poisons_its_rows():
    rng = np.random.default_rng(4)
    A, B = _codes(rng, (3, 64)), _codes(rng, (2, 64))
    SA = np.full((3, 2), 127, np.uint8)
    SA[1, 0] = 255
    C = oracle.mx_gemm_f64(A, SA, B, np.full((2, 2), 127, np.uint8))
    assert np.isnan(C[1]).all() and np.isfinite(C[[0, 2]]).all()


def test_entries_match_full_product():
    rng = np.random.default_rng(5)
    M, N, K = 6, 5, 128
    A, B = _codes(rng, (M, K), 1, 14), _codes(rng, (N, K), 1, 14)
    SA = rng.integers(120, 135, (M, 4)).astype(np.uint8)
    SB = rng.integers(120, 135, (N, 4)).astype(np.uint8)
    full = oracle.mx_gemm_f64(A, SA, B, SB)
    rows, cols = np.array([0, 5, 3, 2]), np.array([4, 0, 2, 2])
    assert np.array_equal(oracle.mx_gemm_entries_f64(A, SA, B, SB, rows, cols), full[rows, cols])


def test_decoded_product_equals_term_by_term_sums():
    """The full product decodes each operand once and sums in i-k-j order; the
    per-entry routine multiplies the four factors of every term as it goes.
    Every term is exact in binary64, so both must give the same bits (NaN
    blocks, negative-zero rows and a wide spread of scales included)."""
    from workloads import make_mx_inputs
    A, SFA, B, SFB = make_mx_inputs(40, 36, 512, seed=11, spread=30)
    A[3, 7] = 0x7F
    SFB[5, 2] = 0xFF
    A[9, :] = 0x80
    full = oracle.mx_gemm_f64(A, SFA, B, SFB)
    r, c = np.meshgrid(np.arange(40), np.arange(36), indexing="ij")
    each = oracle.mx_gemm_entries_f64(A, SFA, B, SFB, r.ravel(), c.ravel()).reshape(40, 36)
    assert np.array_equal(np.isnan(full), np.isnan(each))
    fin = ~np.isnan(full)
    assert np.isnan(full[3]).all() and np.isnan(full[:, 5]).all() and fin.sum() > 0
    assert np.array_equal(full[fin].view(np.uint64), each[fin].view(np.uint64))


def test_shape_checks():
    with pytest.raises(ValueError):
        oracle.mx_gemm_f64(np.zeros((2, 48), np.uint8), np.zeros((2, 1), np.uint8),
                           np.zeros((2, 48), np.uint8), np.zeros((2, 1), np.uint8))
