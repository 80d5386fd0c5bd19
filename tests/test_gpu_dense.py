"""GPU parity of the dense BF16 / FP16 GEMM (mx_dense_gemm, through the C ABI)
against the oracle's double-precision product, in the four layouts.

Tolerance from the arithmetic: the products of two BF16 / FP16 values are
exact in FP32, each MFMA adds 16 of them into the FP32 accumulator, and K/16
such additions follow in sequence, so |c - c_ref| <= (K/16 + 16) 2^-24 S
(S = sum |a b|) plus subnormal flushing.  16-bit output must be the
round-to-nearest-even of the FP32 output bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mxgen
import oracle

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_scaled_precision_mm_amd as mx
    return mx


def bits(x, dtype):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(TDT[dtype]).view(torch.int16).numpy().view(np.uint16)


def stored(X, trans):
    return np.ascontiguousarray(X.T if trans else X)


def run(mx, dtype, ta, tb, a_st, b_st, M, N, K, out):
    a = torch.from_numpy(a_st.view(np.int16)).cuda().view(TDT[dtype])
    b = torch.from_numpy(b_st.view(np.int16)).cuda().view(TDT[dtype])
    c = torch.empty((M, N), dtype={"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out],
                    device="cuda")
    mx.mx_dense_gemm(a, b, c, M, N, K, ta, tb)
    torch.cuda.synchronize()
    if out == "f32":
        return c.cpu().numpy().astype(np.float64)
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


def check(mx, dtype, ta, tb, M, N, K, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    A = bits(rng.standard_normal((M, K)) * scale, dtype)
    B = bits(rng.standard_normal((K, N)) * scale, dtype)
    a_st, b_st = stored(A, ta), stored(B, tb)
    what = "%s %s%s %dx%dx%d" % (dtype, "NT"[ta], "NT"[tb], M, N, K)
    print("dense", what, flush=True)
    cref, S = oracle.dense_gemm(dtype, ta, tb, a_st, b_st, M, N, K)
    c32 = run(mx, dtype, ta, tb, a_st, b_st, M, N, K, "f32")
    tol = (K / 16 + 16) * 2.0 ** -24 * S + 2.0 ** -126 * K
    err = np.abs(c32 - cref)
    assert np.all(err <= tol), "%s: max err %g over tol (err/S %g)" % (what, (err - tol).max(), (err / np.maximum(S, 1e-300)).max())
    for out, rnd in (("bf16", oracle.round_bf16), ("f16", oracle.round_f16)):
        b16 = run(mx, dtype, ta, tb, a_st, b_st, M, N, K, out)
        assert np.array_equal(b16, rnd(c32)), what + " " + out + " != RNE(f32)"


LAYOUTS = [(0, 0), (0, 1), (1, 0), (1, 1)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=["NN", "NT", "TN", "TT"])
def test_layouts_small(mx, dtype, ta, tb):
    # every contiguous dimension a multiple of 8; ragged against the 128 tile
    # and the 32-deep stage; one stage, several stages, a K tail
    for (M, N, K) in ((8, 8, 8), (136, 264, 40), (128, 128, 32), (264, 72, 520), (40, 1000, 1032)):
        check(mx, dtype, ta, tb, M, N, K, seed=M + 3 * N + 7 * K + 11 * ta + 13 * tb)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_ragged_rows(mx, dtype):
    # M free when a is [M][K] (NN, NT); N free when b is [N][K] (NT, TT)
    check(mx, dtype, 0, 1, 37, 45, 264, seed=1)
    check(mx, dtype, 0, 0, 1, 64, 64, seed=2)
    check(mx, dtype, 1, 1, 16, 3, 96, seed=3)


def test_integer_valued_exact(mx):
    # small integers: every partial sum exact in FP32, so the result is exact
    rng = np.random.default_rng(5)
    M, N, K = 192, 136, 1024
    for ta, tb in LAYOUTS:
        Ai = rng.integers(-8, 9, (M, K)).astype(np.float32)
        Bi = rng.integers(-8, 9, (K, N)).astype(np.float32)
        a_st, b_st = stored(bits(Ai, "bf16"), ta), stored(bits(Bi, "bf16"), tb)
        c32 = run(mx, "bf16", ta, tb, a_st, b_st, M, N, K, "f32")
        assert np.array_equal(c32, (Ai.astype(np.int64) @ Bi.astype(np.int64)).astype(np.float64))


def test_large_sampled(mx):
    # the bench shape, sampled outputs against the oracle
    M = N = K = 2048
    rng = np.random.default_rng(9)
    A = bits(rng.standard_normal((M, K)), "bf16")
    B = bits(rng.standard_normal((N, K)), "bf16")     # stored [N][K]: NT
    c32 = run(mx, "bf16", 0, 1, A, B, M, N, K, "f32")
    ms, ns = rng.integers(0, M, 2000), rng.integers(0, N, 2000)
    Av = oracle.dense_values("bf16", A, (M, K))
    Bv = oracle.dense_values("bf16", B, (N, K))
    ref = np.einsum("ik,ik->i", Av[ms], Bv[ns])
    S = np.einsum("ik,ik->i", np.abs(Av[ms]), np.abs(Bv[ns]))
    assert np.all(np.abs(c32[ms, ns] - ref) <= (K / 16 + 16) * 2.0 ** -24 * S)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("shape", [(4096, 3072, 264), (2048, 3072, 520), (1000, 1000, 72)],
                         ids=["256x256tile", "128x256tile", "128x128tile"])
def test_tile_layouts_sampled(mx, dtype, ta, tb, shape):
    # every layout runs on the tile kernel (an operand stored [K][M] or
    # [K][N] with slots of K rows, read transposed), on the 256 x 256,
    # 128 x 256 or 128 x 128 tile by the number of output tiles; K not a
    # multiple of the 64-deep super-stage; sampled outputs plus the last row
    # and column against the oracle
    M, N, K = shape
    rng = np.random.default_rng(M + N + K + 2 * ta + tb)
    A = bits(rng.standard_normal((M, K)), dtype)            # the logical [M][K] operand
    B = bits(rng.standard_normal((K, N)), dtype)            # the logical [K][N] operand
    a_st, b_st = stored(A, ta), stored(B, tb)
    print("dense tile", dtype, "NT"[ta] + "NT"[tb], shape, flush=True)
    c32 = run(mx, dtype, ta, tb, a_st, b_st, M, N, K, "f32")
    ms = np.concatenate([rng.integers(0, M, 3000), np.full(64, M - 1), rng.integers(0, M, 64)])
    ns = np.concatenate([rng.integers(0, N, 3000), rng.integers(0, N, 64), np.full(64, N - 1)])
    Av = oracle.dense_values(dtype, A, (M, K))
    Bv = oracle.dense_values(dtype, B, (K, N))
    ref = np.einsum("ik,ki->i", Av[ms], Bv[:, ns])
    S = np.einsum("ik,ki->i", np.abs(Av[ms]), np.abs(Bv[:, ns]))
    tol = (K / 16 + 16) * 2.0 ** -24 * S + 2.0 ** -126 * K
    assert np.all(np.abs(c32[ms, ns] - ref) <= tol)
    for out, rnd in (("bf16", oracle.round_bf16), ("f16", oracle.round_f16)):
        b16 = run(mx, dtype, ta, tb, a_st, b_st, M, N, K, out)
        assert np.array_equal(b16, rnd(c32)), "%s %s != RNE(f32)" % (shape, out)


def test_wide_k_major_operand_fallback(mx):
    # B stored [K][N] with 2^25 columns and K = 8: the tile kernel's 32-bit
    # offsets could wrap, so the transposing kernel runs it (sampled outputs,
    # the last columns included, exact: small integers)
    M, N, K = 8, 1 << 25, 8
    rng = np.random.default_rng(17)
    Ai = rng.integers(-4, 5, (M, K)).astype(np.float32)
    Bi = rng.integers(-4, 5, (K, N), dtype=np.int8)
    A = bits(Ai, "bf16")
    B = (Bi.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # small integers: exact in BF16
    print("dense fallback NN", (M, N, K), flush=True)
    c32 = run(mx, "bf16", 0, 0, A, B, M, N, K, "f32")
    ns = np.concatenate([rng.integers(0, N, 4000), np.arange(N - 64, N)])
    ref = Ai.astype(np.int64) @ Bi[:, ns].astype(np.int64)
    assert np.array_equal(c32[:, ns], ref.astype(np.float64))
