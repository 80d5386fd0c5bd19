"""Pins for the oracle's grouped product (oracle.grouped_gemm, group_rows),
none of which re-types its definition: the row ranges written out by hand
for ordinary, empty, decreasing and out-of-range group ends; one group is
the plain GEMM; with unit scales each group equals a float64 matmul of
independently decoded operands (exact at these sizes); identical B for
every group reduces to one plain GEMM over all covered rows; reordering
the groups reorders the output rows; rows past the last group stay
uncovered.

The grouped operation: "PyTorch 接上 FlyDSL" (5ulink.com), support-matrix
row "Grouped GEMM" (groups of A of different lengths, empty groups skipped)
and the roadmap item "MXFP8 Grouped GEMM".
"""
import numpy as np
import pytest

import mxgen
import oracle
from tests import refdecode


def test_group_rows_table():
    assert oracle.group_rows([3, 3, 7, 10], 4, 10) == [(0, 3), (3, 3), (3, 7), (7, 10)]
    assert oracle.group_rows([0, 0, 5], 3, 5) == [(0, 0), (0, 0), (0, 5)]
    # a decreasing end gives an empty group; ends past M are clamped to M
    assert oracle.group_rows([4, 2, 6, 99], 4, 8) == [(0, 4), (4, 4), (4, 6), (6, 8)]
    # negative ends count as 0; rows past the last end are not covered
    assert oracle.group_rows([-5, 2, 3], 3, 9) == [(0, 0), (0, 2), (2, 3)]


def _grouped_inputs(fmt, sizes, N, K, seed, lo=120, hi=134):
    G = len(sizes)
    M = int(sum(sizes))
    a, sa = mxgen.random_codes(seed, fmt, max(M, 1), K, lo, hi)
    b, sb = mxgen.random_codes(seed + 1, fmt, G * N, K, lo, hi)
    offs = np.cumsum(sizes).astype(np.int32)
    return a[:M], b, sa[:M], sb, offs, G, M


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_single_group_is_plain_gemm(fmt):
    a, b, sa, sb, offs, G, M = _grouped_inputs(fmt, [37], 24, 256, 5)
    c, s, cov = oracle.grouped_gemm(fmt, a, b, sa, sb, offs, G, M, 24, 256)
    c0, s0 = oracle.gemm(fmt, a, b, sa, sb, M, 24, 256)
    assert cov.all()
    assert np.array_equal(c, c0) and np.array_equal(s, s0)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_unit_scales_groups_equal_decoded_matmul(fmt):
    sizes = [5, 0, 17, 1, 0, 9]
    N, K = 20, 256
    a, b, sa, sb, offs, G, M = _grouped_inputs(fmt, sizes, N, K, 11, 127, 127)
    c, _, cov = oracle.grouped_gemm(fmt, a, b, sa, sb, offs, G, M, N, K)
    A = refdecode.values(fmt, a, M, K)
    B = refdecode.values(fmt, b, G * N, K).reshape(G, N, K)
    r0 = 0
    for g, m in enumerate(sizes):
        if m:
            assert np.array_equal(c[r0:r0 + m], A[r0:r0 + m] @ B[g].T)
        r0 += m
    assert cov.all()


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_shared_b_is_one_gemm(fmt):
    sizes = [4, 0, 11, 3]
    N, K = 16, 128
    a, _, sa, _, offs, G, M = _grouped_inputs(fmt, sizes, N, K, 21)
    b1, sb1 = mxgen.random_codes(99, fmt, N, K, 120, 134)
    b = np.concatenate([b1] * G)
    sb = np.concatenate([sb1] * G)
    c, s, _ = oracle.grouped_gemm(fmt, a, b, sa, sb, offs, G, M, N, K)
    c0, s0 = oracle.gemm(fmt, a, b1, sa, sb1, M, N, K)
    assert np.array_equal(c, c0) and np.array_equal(s, s0)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_group_order_permutes_rows(fmt):
    sizes = [6, 2, 9]
    N, K = 12, 128
    a, b, sa, sb, offs, G, M = _grouped_inputs(fmt, sizes, N, K, 31)
    c, _, _ = oracle.grouped_gemm(fmt, a, b, sa, sb, offs, G, M, N, K)
    rb = a.shape[1]
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    perm = [2, 0, 1]
    rows = np.concatenate([np.arange(starts[g], starts[g] + sizes[g]) for g in perm])
    a2, sa2 = a[rows], sa[rows]
    b2 = b.reshape(G, N, rb)[perm].reshape(G * N, rb)
    sb2 = sb.reshape(G, N, -1)[perm].reshape(G * N, -1)
    offs2 = np.cumsum([sizes[g] for g in perm]).astype(np.int32)
    c2, _, _ = oracle.grouped_gemm(fmt, a2, b2, sa2, sb2, offs2, G, M, N, K)
    assert np.array_equal(c2, c[rows])


def test_rows_past_last_group_uncovered():
    fmt, N, K = "fp4", 8, 128
    a, sa = mxgen.random_codes(3, fmt, 10, K)
    b, sb = mxgen.random_codes(4, fmt, 2 * N, K)
    c, s, cov = oracle.grouped_gemm(fmt, a, b, sa, sb, np.array([3, 7], np.int32), 2, 10, N, K)
    assert list(cov) == [True] * 7 + [False] * 3
    assert np.isnan(c[7:]).all() and np.isfinite(c[:7]).all()
