"""Pins of the oracle's MXFP4 GEMM (C = A · Bᵀ of two operands quantized
along K) against values fixed by the definition: exact rational brute force
on small random operands, closed forms, and the transpose identity."""
from fractions import Fraction

import numpy as np

import oracle

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def _value(codes, scales, r, k):
    byte = int(codes[r, k // 2])
    c = (byte >> (4 * (k & 1))) & 15
    v = E2M1[c & 7] * Fraction(2) ** (int(scales[r, k // 32]) - 127)
    return -v if c & 8 else v


def test_brute_force_exact():
    rng = np.random.default_rng(31)
    M, N, K = 5, 7, 128
    a = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = rng.integers(120, 135, (M, K // 32), dtype=np.uint8)
    sb = rng.integers(120, 135, (N, K // 32), dtype=np.uint8)
    got = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    for m in range(M):
        for n in range(N):
            want = sum(_value(a, sa, m, k) * _value(b, sb, n, k) for k in range(K))
            assert Fraction(got[m, n]) == want, (m, n)


def test_closed_forms():
    M, N, K = 3, 4, 256
    ones = np.full((M, K // 2), 0x22, dtype=np.uint8)   # every code 1.0
    onesb = np.full((N, K // 2), 0x22, dtype=np.uint8)
    got = oracle.gemm_mx(ones, np.full((M, K // 32), 128, np.uint8), onesb,
                         np.full((N, K // 32), 126, np.uint8), M, N, K)
    assert np.all(got == K)  # (1 * 2) * (1 * 1/2) summed over K
    neg = np.full((N, K // 2), 0xAA, dtype=np.uint8)    # every code -1.0
    got = oracle.gemm_mx(ones, np.full((M, K // 32), 127, np.uint8), neg,
                         np.full((N, K // 32), 127, np.uint8), M, N, K)
    assert np.all(got == -K)
    zero = np.full((N, K // 2), 0x88, dtype=np.uint8)   # -0 codes
    got = oracle.gemm_mx(ones, np.full((M, K // 32), 127, np.uint8), zero,
                         np.full((N, K // 32), 127, np.uint8), M, N, K)
    assert np.all(got == 0)


def test_transpose_identity():
    rng = np.random.default_rng(32)
    M, N, K = 6, 9, 96
    a = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = rng.integers(100, 150, (M, K // 32), dtype=np.uint8)
    sb = rng.integers(100, 150, (N, K // 32), dtype=np.uint8)
    assert np.array_equal(oracle.gemm_mx(a, sa, b, sb, M, N, K),
                          oracle.gemm_mx(b, sb, a, sa, N, M, K).T)
