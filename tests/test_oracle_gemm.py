"""Pins for the oracle GEMM (no GPU).

* exact rational brute force on tiny inputs (Fraction arithmetic, operands
  decoded independently through torch's float8 casts);
* float64 matmul of independently decoded operands (all scales 1);
* int64 matmul of integer-valued inputs (exact);
* invariants: raising one E8M0 code by 1 doubles exactly that block's
  contribution, +-k scales by 2^+-k, flipping all sign bits negates C,
  swapping the operands transposes C, NaN scale / NaN element patterns.
"""
from fractions import Fraction

import numpy as np
import pytest

import mxgen
import oracle
from tests import refdecode


def _rand(fmt, M, N, K, seed, lo=120, hi=134):
    a, sa = mxgen.random_codes(seed, fmt, M, K, lo, hi)
    b, sb = mxgen.random_codes(seed + 7, fmt, N, K, lo, hi)
    return a, b, sa, sb


def _exact(fmt, a, b, sa, sb, M, N, K):
    A = refdecode.values(fmt, a, M, K)
    B = refdecode.values(fmt, b, N, K)
    SA = refdecode.e8m0(sa)
    SB = refdecode.e8m0(sb)
    C = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            sacc = Fraction(0)
            for k in range(K):
                f = Fraction(SA[m, k // 32]) * Fraction(SB[n, k // 32])
                p = Fraction(A[m, k]) * Fraction(B[n, k]) * f
                acc += p
                sacc += abs(p)
            C[m][n] = acc
            S[m][n] = sacc
    return C, S


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("K", [128, 256])
def test_bruteforce_fraction(fmt, K):
    M, N = 3, 4
    a, b, sa, sb = _rand(fmt, M, N, K, seed=11 + K)
    c, s = oracle.gemm(fmt, a, b, sa, sb, M, N, K)
    C, S = _exact(fmt, a, b, sa, sb, M, N, K)
    for m in range(M):
        for n in range(N):
            Sx = float(S[m][n])
            assert abs(s[m, n] - Sx) <= 1e-15 * Sx
            assert abs(Fraction(c[m, n]) - C[m][n]) <= Fraction(K // 32) * Fraction(2) ** -53 * S[m][n]


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_unit_scales_equal_float64_matmul(fmt):
    M, N, K = 37, 29, 512
    a, b, _, _ = _rand(fmt, M, N, K, seed=3)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    c, s = oracle.gemm(fmt, a, b, sa, sb, M, N, K)
    A = refdecode.values(fmt, a, M, K)
    B = refdecode.values(fmt, b, N, K)
    ref = A @ B.T
    assert np.all(np.abs(c - ref) <= 1e-14 * s + 1e-300)
    assert np.allclose(s, np.abs(A) @ np.abs(B).T, rtol=1e-14, atol=0)


def test_integer_valued_fp4_exact_int64():
    # E2M1 values times 2 are integers; with both scales 2^1 every element is an integer
    M, N, K = 24, 40, 1024
    a, b, _, _ = _rand("fp4", M, N, K, seed=5)
    sa = np.full((M, K // 32), 128, np.uint8)
    sb = np.full((N, K // 32), 128, np.uint8)
    c, _ = oracle.gemm("fp4", a, b, sa, sb, M, N, K)
    Ai = (refdecode.values("fp4", a, M, K) * 2).astype(np.int64)
    Bi = (refdecode.values("fp4", b, N, K) * 2).astype(np.int64)
    assert np.array_equal(c, (Ai @ Bi.T).astype(np.float64))


def test_integer_valued_fp8_exact_int64():
    # E4M3 codes with exponent field >= 10 (values >= 8, multiples of 1) are integers
    rng = np.random.default_rng(6)
    M, N, K = 16, 20, 256
    def ints(rows):
        e = rng.integers(10, 13, size=(rows, K))
        m = rng.integers(0, 8, size=(rows, K))
        s = rng.integers(0, 2, size=(rows, K))
        return ((s << 7) | (e << 3) | m).astype(np.uint8)
    a, b = ints(M), ints(N)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    c, _ = oracle.gemm("fp8", a, b, sa, sb, M, N, K)
    Ai = refdecode.values("fp8", a, M, K).astype(np.int64)
    Bi = refdecode.values("fp8", b, N, K).astype(np.int64)
    assert np.array_equal(c, (Ai @ Bi.T).astype(np.float64))


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_scale_plus_one_doubles_exactly_that_block(fmt):
    M, N, K = 5, 6, 384
    a, b, sa, sb = _rand(fmt, M, N, K, seed=9, lo=125, hi=129)
    c0, _ = oracle.gemm(fmt, a, b, sa, sb, M, N, K)
    m, kb = 2, 7
    # contribution of block kb alone: every other block's A scale set so it vanishes exactly
    # is not possible in E8M0 (no zero), so isolate the block by zeroing the other A codes
    a_only = a.copy().reshape(M, -1)
    per_blk = 16 if fmt == "fp4" else 32
    keep = np.zeros_like(a_only)
    keep[:, kb * per_blk:(kb + 1) * per_blk] = a_only[:, kb * per_blk:(kb + 1) * per_blk]
    blk, _ = oracle.gemm(fmt, keep, b, sa, sb, M, N, K)
    sa2 = sa.copy()
    sa2[m, kb] += 1
    c1, _ = oracle.gemm(fmt, a, b, sa2, sb, M, N, K)
    # rows other than m unchanged, row m changes by exactly the block's contribution
    rows = [r for r in range(M) if r != m]
    assert np.array_equal(c1[rows], c0[rows])
    # the isolated-block identity is exact when the other blocks are zero
    blk2, _ = oracle.gemm(fmt, keep, b, sa2, sb, M, N, K)
    assert np.array_equal(blk2[m], 2.0 * blk[m])
    assert np.allclose(c1[m] - c0[m], blk[m], rtol=0, atol=1e-12 * np.abs(c0).max())


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("k", [-9, -1, 3, 20])
def test_uniform_scale_shift_is_exact_power_of_two(fmt, k):
    M, N, K = 4, 9, 256
    a, b, sa, sb = _rand(fmt, M, N, K, seed=21)
    c0, s0 = oracle.gemm(fmt, a, b, sa, sb, M, N, K)
    c1, s1 = oracle.gemm(fmt, a, b, (sa.astype(int) + k).astype(np.uint8), sb, M, N, K)
    assert np.array_equal(c1, np.ldexp(c0, k))
    assert np.array_equal(s1, np.ldexp(s0, k))


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_sign_flip_and_transpose(fmt):
    M, N, K = 6, 5, 256
    a, b, sa, sb = _rand(fmt, M, N, K, seed=33)
    c, s = oracle.gemm(fmt, a, b, sa, sb, M, N, K)
    flip = np.uint8(0x88 if fmt == "fp4" else 0x80)
    cn, sn = oracle.gemm(fmt, a ^ flip, b, sa, sb, M, N, K)
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    ct, st = oracle.gemm(fmt, b, a, sb, sa, N, M, K)
    assert np.array_equal(ct, c.T) and np.array_equal(st, s.T)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_nan_scale_pattern(fmt):
    M, N, K = 4, 6, 256
    a, b, sa, sb = _rand(fmt, M, N, K, seed=44)
    a[:] = 0                              # NaN scale poisons the block even when the codes are zero
    sa[1, 3] = 255
    sb[4, 0] = 255
    c, _ = oracle.gemm(fmt, a, b, sa, sb, M, N, K)
    expect = np.zeros((M, N), bool)
    expect[1, :] = True
    expect[:, 4] = True
    assert np.array_equal(np.isnan(c), expect)


def test_e4m3_nan_element():
    M, N, K = 3, 3, 128
    a, b, sa, sb = _rand("fp8", M, N, K, seed=55)
    a[2, 77] = 0xFF
    c, _ = oracle.gemm("fp8", a, b, sa, sb, M, N, K)
    assert np.all(np.isnan(c[2])) and not np.any(np.isnan(c[:2]))


def test_gemm_at_matches_full():
    M, N, K = 33, 47, 512
    for fmt in ("fp4", "fp8"):
        a, b, sa, sb = _rand(fmt, M, N, K, seed=66)
        c, s = oracle.gemm(fmt, a, b, sa, sb, M, N, K)
        rng = np.random.default_rng(1)
        ms = rng.integers(0, M, 50)
        ns = rng.integers(0, N, 50)
        c2, s2 = oracle.gemm_at(fmt, a, b, sa, sb, M, N, K, ms, ns)
        assert np.array_equal(c2, c[ms, ns]) and np.array_equal(s2, s[ms, ns])


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.gemm("fp4", np.zeros(10, np.uint8), np.zeros(10, np.uint8), np.zeros(1, np.uint8),
                    np.zeros(1, np.uint8), 1, 1, 128)
