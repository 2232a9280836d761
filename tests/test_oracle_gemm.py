"""Pins for the oracle's fp64 GEMM (oracle_gemm_f64 / oracle_gemm_entries_f64).

What fixes the expected values, independently of the oracle:
  * exact rational sums (fractions.Fraction) on tiny random fp16/bf16 shapes,
    with value ranges chosen so that binary64 sums are exact: the oracle must be
    exact there, and its rounded output bit-exact against a brute-force nearest
    search;
  * closed forms: identity, permutation and rank-1 products;
  * numpy's binary64 matmul (a library routine) on medium shapes.
Non-square shapes throughout, so a transposed operand cannot pass.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact

FP16, BF16 = 1, 2


def _to_dtype_f64(x: np.ndarray, fmt: int) -> np.ndarray:
    t = torch.from_numpy(x).to(torch.float16 if fmt == FP16 else torch.bfloat16)
    return t.to(torch.float64).numpy()


def _restricted(rng, shape, fmt):
    """Values with magnitude in [2^-6, 1) (fp16) / [2^-10, 1) (bf16): every
    product is a multiple of 2^-32 / 2^-34 below 2, so short sums are exact."""
    lo = 2.0 ** (-6 if fmt == FP16 else -10)
    mag = np.exp(rng.uniform(np.log(lo), 0.0, size=shape))
    sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    return _to_dtype_f64(mag * sign, fmt)


def _exact_product(A, B):
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(A[i, k])) for k in range(K)] for i in range(M)]
    Bf = [[Fraction(float(B[k, j])) for j in range(N)] for k in range(K)]
    return [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]


@pytest.mark.parametrize("fmt", [FP16, BF16])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (7, 2, 4), (5, 6, 1), (2, 7, 6)])
def test_bruteforce_exact_and_bitexact(fmt, shape):
    M, N, K = shape
    rng = np.random.default_rng(hash((fmt,) + shape) % (2 ** 32))
    A = _restricted(rng, (M, K), fmt)
    B = _restricted(rng, (K, N), fmt)
    C = oracle.gemm_f64(A, B)
    ex = _exact_product(A, B)
    bits = oracle.round_to(C, fmt)
    for i in range(M):
        for j in range(N):
            assert Fraction(float(C[i, j])) == ex[i][j], (i, j)
            assert int(bits[i, j]) == exact.nearest_bits(ex[i][j], fmt), (i, j)


@pytest.mark.parametrize("fmt", [FP16, BF16])
def test_bruteforce_wide_range_within_fp64_bound(fmt):
    """Full-range uniform[-1,1] inputs (fp16 subnormals included): the binary64
    sum may round, but stays within K * 2^-53 * sum|a*b| of the exact value."""
    rng = np.random.default_rng(21 + fmt)
    M, N, K = 4, 6, 7
    A = _to_dtype_f64(rng.uniform(-1, 1, (M, K)), fmt)
    B = _to_dtype_f64(rng.uniform(-1, 1, (K, N)), fmt)
    A[0, 0] = _to_dtype_f64(np.array([3e-7]), fmt)[0]   # a tiny (fp16 subnormal) entry
    C = oracle.gemm_f64(A, B)
    ex = _exact_product(A, B)
    absum = np.abs(A) @ np.abs(B)
    for i in range(M):
        for j in range(N):
            err = abs(Fraction(float(C[i, j])) - ex[i][j])
            assert err <= Fraction(K) * Fraction(2) ** -53 * Fraction(float(absum[i, j])) * 2


@pytest.mark.parametrize("fmt", [FP16, BF16])
def test_identity_and_permutation(fmt):
    rng = np.random.default_rng(31)
    K, N = 24, 40
    B = _to_dtype_f64(rng.uniform(-1, 1, (K, N)), fmt)
    assert np.array_equal(oracle.gemm_f64(np.eye(K), B), B)
    perm = rng.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0          # row i of P picks row perm[i] of B
    C = oracle.gemm_f64(P, B)
    assert np.array_equal(C, B[perm])
    # rectangular selection: 9 rows chosen with repetition
    pick = rng.integers(0, K, size=9)
    S = np.zeros((9, K))
    S[np.arange(9), pick] = 1.0
    assert np.array_equal(oracle.gemm_f64(S, B), B[pick])
    bits = oracle.round_to(oracle.gemm_f64(S, B), fmt)
    t = torch.from_numpy(B[pick]).to(torch.float16 if fmt == FP16 else torch.bfloat16)
    assert np.array_equal(bits, t.view(torch.int16).numpy().view(np.uint16))


@pytest.mark.parametrize("fmt", [FP16, BF16])
def test_rank_one_closed_form(fmt):
    """A[i,k] = a_i, B[k,j] = b_j with a, b in {0, +-2^e} and K = 64: C = K * a_i * b_j,
    a signed power of two (or zero), so exact in both output formats."""
    rng = np.random.default_rng(41)
    M, N, K = 13, 17, 64
    a = rng.choice([0.0, 1.0, -1.0, 0.5, -2.0, 4.0, 0.25], size=M)
    b = rng.choice([0.0, 1.0, -0.5, 2.0, -4.0, 0.125], size=N)
    A = np.repeat(a[:, None], K, axis=1)
    B = np.repeat(b[None, :], K, axis=0)
    C = oracle.gemm_f64(A, B)
    expect = K * np.outer(a, b) + 0.0    # an empty-magnitude sum is +0
    assert np.array_equal(C, expect)
    bits = oracle.round_to(C, fmt)
    t = torch.from_numpy(expect).to(torch.float16 if fmt == FP16 else torch.bfloat16)
    assert np.array_equal(bits, t.view(torch.int16).numpy().view(np.uint16))


def test_matches_numpy_matmul_medium():
    rng = np.random.default_rng(51)
    for (M, N, K) in [(64, 48, 96), (130, 70, 257), (1, 300, 33)]:
        A = _to_dtype_f64(rng.uniform(-1, 1, (M, K)), FP16)
        B = _to_dtype_f64(rng.standard_normal((K, N)), BF16)
        C = oracle.gemm_f64(A, B)
        ref = A @ B
        scale = np.abs(A) @ np.abs(B)
        assert np.all(np.abs(C - ref) <= 1e-12 * scale + 1e-300)


def test_entries_match_full_product():
    rng = np.random.default_rng(61)
    M, N, K = 37, 53, 71
    A = _to_dtype_f64(rng.uniform(-1, 1, (M, K)), BF16)
    B = _to_dtype_f64(rng.uniform(-1, 1, (K, N)), BF16)
    C = oracle.gemm_f64(A, B)
    rows = rng.integers(0, M, 500)
    cols = rng.integers(0, N, 500)
    assert np.array_equal(oracle.gemm_entries_f64(A, B, rows, cols), C[rows, cols])


def test_empty_and_zero_k():
    A = np.zeros((3, 0))
    B = np.zeros((0, 4))
    assert np.array_equal(oracle.gemm_f64(A, B), np.zeros((3, 4)))
    assert oracle.gemm_f64(np.zeros((0, 5)), np.zeros((5, 2))).shape == (0, 2)
