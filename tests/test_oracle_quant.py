"""Pins for the oracle's MX quantizer (oracle.quantize), none of which re-types
its formula: the E2M1 rounding table written out from the round-to-nearest-
even rule, torch's own float8_e4m3fn cast (a library RNE conversion), exact
round trips from random codes and scales, the scale choice in closed form,
power-of-two scaling invariance and the NaN / zero special cases.

Rule being pinned (OCP MX v1.0 conversion; the pages name only the
BlockWise1x32 E8M0 scales, "PyTorch 接上 FlyDSL", 5ulink.com, 支持边界):
scale code = floor(log2 amax) - emax + 127 clamped to [0, 254] (emax 2 for
E2M1, 8 for E4M3), elements to the nearest code, ties to even, saturating.
"""
import numpy as np
import pytest
import torch

import oracle

E2M1_POS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fp4_codes(codes, K):
    lo = codes & 0xF
    hi = codes >> 4
    out = np.empty((codes.shape[0], K), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def test_e2m1_rounding_table():
    # a block whose amax is 6 has scale code 127 (scale 1): elements round in place
    cases = [  # value, expected magnitude code (ties go to the even code)
        (0.0, 0), (0.24, 0), (0.25, 0), (0.26, 1), (0.5, 1), (0.74, 1), (0.75, 2), (1.0, 2),
        (1.25, 2), (1.26, 3), (1.5, 3), (1.75, 4), (2.0, 4), (2.25, 4), (2.5, 4), (2.75, 5),
        (3.0, 5), (3.5, 6), (4.0, 6), (4.5, 6), (5.0, 6), (5.5, 7), (6.0, 7),
    ]
    vals = [v for v, _ in cases]
    for sign in (1.0, -1.0):
        for i in range(0, len(vals), 31):
            chunk = vals[i:i + 31]
            x = np.zeros(32, np.float32)
            x[0] = 6.0
            x[1:1 + len(chunk)] = sign * np.array(chunk, np.float32)
            codes, scales = oracle.quantize("fp4", bf16_bits(x), 1, 32)
            assert scales[0, 0] == 127
            got = fp4_codes(codes, 32)[0, 1:1 + len(chunk)]
            want = [c | (8 if sign < 0 else 0) for _, c in cases[i:i + 31]]
            assert list(got) == want


def test_e4m3_elements_match_torch_cast():
    rng = np.random.default_rng(11)
    rows = 64
    x = rng.uniform(-448, 448, size=(rows, 32)).astype(np.float32)
    x *= rng.choice([1.0, 1 / 64, 1 / 4096], size=(rows, 32)).astype(np.float32)   # reach subnormal E4M3
    x[:, 0] = rng.uniform(256, 448, size=rows)    # amax in [256, 512): scale code 127
    xb = bf16_bits(x)
    codes, scales = oracle.quantize("fp8", xb, rows, 32)
    assert np.all(scales == 127)
    xf = torch.tensor(xb.view(np.int16)).view(torch.bfloat16).float()
    ref = xf.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_round_trip_exact(fmt):
    # codes whose block holds a code of the top binade decode to values whose
    # quantization must give back the same codes and scale
    rng = np.random.default_rng(5 if fmt == "fp4" else 6)
    rows = 200
    if fmt == "fp4":
        mags = np.array(E2M1_POS)
        top = [6, 7]                       # 4, 6: amax in [4, 8)
        sbit = 8
        q = rng.integers(0, 8, size=(rows, 32))
    else:
        mags = np.array([0.0] + [float(v) for v in
                                 torch.arange(1, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float()])
        top = list(range(0x78, 0x7F))      # 256 .. 448: amax in [256, 512)
        sbit = 128
        q = rng.integers(0, 127, size=(rows, 32))
    q[:, rng.integers(0, 32)] = rng.choice(top, size=rows)
    sign = rng.integers(0, 2, size=(rows, 32))
    s = rng.integers(100, 150, size=rows)
    x = np.where(sign == 1, -1.0, 1.0) * mags[q] * np.ldexp(1.0, (s - 127))[:, None]
    xb = bf16_bits(x)
    assert np.array_equal(torch.tensor(xb.view(np.int16)).view(torch.bfloat16).double().numpy(), x)   # exact in bf16
    codes, scales = oracle.quantize(fmt, xb, rows, 32)
    want = q | (sign * sbit)
    got = fp4_codes(codes, 32) if fmt == "fp4" else codes
    assert np.array_equal(scales[:, 0], s)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt,emax", [("fp4", 2), ("fp8", 8)])
def test_scale_choice_closed_form(fmt, emax):
    # amax = 2^e * (1 + f): scale code e - emax + 127, clamped to [0, 254]
    for bits, e in ((0x3F80, 0), (0x3FFF, 0), (0x4000, 1), (0x7F7F, 127), (0x0080, -126),
                    (0x0001, -133), (0x0040, -127), (0x3E00, -3)):
        x = np.zeros(32, np.uint16)
        x[17] = bits
        _, scales = oracle.quantize(fmt, x, 1, 32)
        assert scales[0, 0] == min(max(e - emax + 127, 0), 254), hex(bits)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_power_of_two_invariance(fmt):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    c0, s0 = oracle.quantize(fmt, bf16_bits(x), 32, 64)
    for k in (-9, 3, 20):
        c1, s1 = oracle.quantize(fmt, bf16_bits(np.ldexp(x, k)), 32, 64)
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1.astype(int), s0.astype(int) + k)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_special_blocks(fmt):
    x = np.zeros((4, 32), np.uint16)
    x[0, 3] = 0x7FC0              # NaN
    x[1, 5] = 0xFF80              # -inf
    x[1, 6] = 0x3F80
    x[2, :] = 0x8000              # all -0: scale 0, sign kept
    x[3, :] = 0x3F80              # all ones
    codes, scales = oracle.quantize(fmt, x, 4, 32)
    assert list(scales[:, 0]) == [255, 255, 0, 127 - (2 if fmt == "fp4" else 8)]
    el = fp4_codes(codes, 32) if fmt == "fp4" else codes
    assert np.all(el[:2] == 0)
    assert np.all(el[2] == (8 if fmt == "fp4" else 0x80))
    # 1.0 at scale 2^-emax: 4 (E2M1 code 6) or 256 (E4M3 code 0x78)
    assert np.all(el[3] == (6 if fmt == "fp4" else 0x78))
