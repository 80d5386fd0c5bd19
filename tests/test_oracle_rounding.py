"""Pins for the oracle's direct double -> bf16 / fp16 rounding (no GPU):
exact rational nearest-even on random doubles (ties, subnormals, overflow)
and torch's float32 -> bfloat16 / float16 casts on float32 inputs."""
from fractions import Fraction
import math

import numpy as np
import torch

import oracle


def _grid_value(bits: int, mbits: int, ebits: int) -> Fraction:
    bias = (1 << (ebits - 1)) - 1
    s = (bits >> (mbits + ebits)) & 1
    e = (bits >> mbits) & ((1 << ebits) - 1)
    m = bits & ((1 << mbits) - 1)
    if e == 0:
        v = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return -v if s else v


def _nearest_even(x: float, mbits: int, ebits: int) -> int:
    """Brute force over the positive finite grid: nearest, ties to even bits."""
    bias = (1 << (ebits - 1)) - 1
    X = Fraction(abs(x))
    nfin = ((1 << ebits) - 1) << mbits      # number of finite non-negative encodings
    # binary search on the monotone grid
    lo, hi = 0, nfin - 1
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if _grid_value(mid, mbits, ebits) <= X:
            lo = mid
        else:
            hi = mid - 1
    cands = [lo, lo + 1]
    maxv = _grid_value(nfin - 1, mbits, ebits)
    # overflow: anything at or beyond max + half an ulp rounds to infinity
    half_ulp = Fraction(2) ** ((1 << ebits) - 2 - bias - mbits - 1)
    sign = (1 << (mbits + ebits)) if math.copysign(1.0, x) < 0 else 0
    if X >= maxv + half_ulp:
        return sign | nfin
    best = None
    for c in cands:
        if c >= nfin:
            continue
        d = abs(_grid_value(c, mbits, ebits) - X)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return sign | best[1]


def _random_doubles(rng, n, lo_exp, hi_exp):
    m = rng.uniform(1, 2, n)
    e = rng.integers(lo_exp, hi_exp, n)
    s = rng.choice([-1.0, 1.0], n)
    return s * np.ldexp(m, e)


def test_bf16_against_rational_nearest_even():
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        _random_doubles(rng, 3000, -140, 129),
        # exact ties and near-ties at several binades
        np.ldexp(1.0 + (2 * rng.integers(0, 128, 200) + 1) / 256.0, rng.integers(-126, 127, 200)),
        np.ldexp(1.0 + (2 * rng.integers(0, 128, 200) + 1) / 256.0, rng.integers(-126, 127, 200)) * (1 + 2.0 ** -40),
        [2.0 ** -133, 1.5 * 2.0 ** -134, 2.0 ** -134, 3 * 2.0 ** -135, (2 - 2.0 ** -8) * 2.0 ** 127,
         (2 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -30), 2.0 ** 128, 1e300, -1e300, 0.0, -0.0],
    ])
    got = oracle.round_bf16(xs)
    for x, g in zip(xs, got):
        assert int(g) == _nearest_even(float(x), 7, 8), (x, hex(int(g)))


def test_f16_against_rational_nearest_even():
    rng = np.random.default_rng(2)
    xs = np.concatenate([
        _random_doubles(rng, 3000, -27, 17),
        np.ldexp(1.0 + (2 * rng.integers(0, 1024, 200) + 1) / 2048.0, rng.integers(-14, 16, 200)),
        [65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26, 0.0, -0.0],
    ])
    got = oracle.round_f16(xs)
    for x, g in zip(xs, got):
        assert int(g) == _nearest_even(float(x), 10, 5), (x, hex(int(g)))


def test_bf16_and_f16_match_torch_on_float32_inputs():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    got = oracle.round_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    g16 = oracle.round_f16(f.astype(np.float64))
    r16 = torch.from_numpy(f.copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(g16, r16)


def test_nan_and_inf():
    x = np.array([np.nan, np.inf, -np.inf])
    assert list(oracle.round_bf16(x)) == [0x7FC0, 0x7F80, 0xFF80]
    assert list(oracle.round_f16(x)) == [0x7E00, 0x7C00, 0xFC00]
