"""Pins for the oracle's dense BF16 / FP16 product (oracle.dense_gemm), the
torch.mm row of the support matrix of "PyTorch 接上 FlyDSL" (FP16/BF16,
static 2-D, NN / NT / TN / TT): the decoders against torch's own casts
over every bit pattern, exact rational brute force on tiny inputs in all
four layouts, integer-valued inputs against int64 matmul, and the four
layouts of one product agreeing exactly."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def bits_of(x, dtype):
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decoder_matches_torch_every_pattern(dtype):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.dense_values(dtype, pats, (65536,))
    t = torch.tensor(pats.view(np.int16)).view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    ref = t.double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _stored(X, trans):
    return np.ascontiguousarray(X.T if trans else X)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_bruteforce_fraction_all_layouts(dtype, ta, tb):
    rng = np.random.default_rng(3 + 2 * ta + tb)
    M, N, K = 3, 4, 9
    A = rng.standard_normal((M, K)) * 3
    B = rng.standard_normal((K, N)) * 3
    ab, bb = bits_of(A, dtype), bits_of(B, dtype)
    Av, Bv = oracle.dense_values(dtype, ab, (M, K)), oracle.dense_values(dtype, bb, (K, N))
    c, s = oracle.dense_gemm(dtype, ta, tb, _stored(ab, ta), _stored(bb.T, 0) if tb else bb, M, N, K)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(Av[m, k]) * Fraction(Bv[k, n]) for k in range(K))
            sabs = sum(abs(Fraction(Av[m, k]) * Fraction(Bv[k, n])) for k in range(K))
            assert abs(Fraction(c[m, n]) - exact) <= Fraction(sabs) * Fraction(K, 2 ** 52)
            assert float(sabs) == pytest.approx(s[m, n], rel=1e-15)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_integer_valued_exact_int64(dtype):
    rng = np.random.default_rng(7)
    M, N, K = 17, 23, 300
    Ai = rng.integers(-64, 65, (M, K))
    Bi = rng.integers(-64, 65, (K, N))
    c, _ = oracle.dense_gemm(dtype, 0, 0, bits_of(Ai, dtype), bits_of(Bi, dtype), M, N, K)
    assert np.array_equal(c, (Ai @ Bi).astype(np.float64))


def test_layouts_agree():
    rng = np.random.default_rng(9)
    M, N, K = 13, 11, 40
    A = bits_of(rng.standard_normal((M, K)), "bf16")
    B = bits_of(rng.standard_normal((K, N)), "bf16")
    ref, _ = oracle.dense_gemm("bf16", 0, 0, A, B, M, N, K)
    for ta in (0, 1):
        for tb in (0, 1):
            c, _ = oracle.dense_gemm("bf16", ta, tb, _stored(A, ta), _stored(B, tb), M, N, K)
            assert np.array_equal(c, ref)
