"""Pins for the oracle's element and scale decoding (no GPU).

E4M3 and E8M0 are checked code by code against torch's float8 casts; E2M1
against the E4M3 bit mapping decoded by torch and against the eight
magnitudes the OCP MX v1.0 specification lists for FP4 E2M1.
"""
import math

import numpy as np
import pytest

import oracle
from tests import refdecode


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    nan = np.isnan(a)
    assert np.array_equal(nan, np.isnan(b))
    assert np.array_equal(a[~nan], b[~nan])
    # signed zeros too
    assert np.array_equal(np.signbit(a[~nan]), np.signbit(b[~nan]))


def test_e4m3_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    got = oracle.decode("fp8", codes, 1, 256)[0]
    _same(got, refdecode.e4m3(np.arange(256)))
    # the spec's landmarks: max finite 448, NaN only at S.1111.111, min subnormal 2^-9
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.isnan(got).sum() == 2
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e8m0_all_codes_match_torch_cast():
    got = oracle.decode_scale(np.arange(256, dtype=np.uint8))
    _same(got, refdecode.e8m0(np.arange(256)))
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127
    assert np.isnan(got[255])


def test_e2m1_all_codes():
    # one byte per pair of codes: element 2i in the low nibble, 2i+1 in the high nibble
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).reshape(1, 8)
    got = oracle.decode("fp4", packed, 1, 16)[0]
    _same(got, refdecode.e2m1(codes))
    # OCP MX v1.0 lists the FP4 (E2M1) magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
    assert list(got[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(got[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert math.copysign(1.0, got[8]) == -1.0


def test_fp4_nibble_order():
    # byte 0x52: element 0 = code 2 (1.0) from the low nibble, element 1 = code 5 (3.0)
    packed = np.array([[0x52] * 16], dtype=np.uint8)
    got = oracle.decode("fp4", packed, 1, 32)[0]
    assert got[0] == 1.0 and got[1] == 3.0
    assert np.array_equal(got[0::2], np.full(16, 1.0)) and np.array_equal(got[1::2], np.full(16, 3.0))


def test_decode_random_rows_match_reference():
    rng = np.random.default_rng(0)
    for fmt in ("fp4", "fp8"):
        rows, K = 7, 256
        packed = rng.integers(0, 256, size=(rows, K // 2 if fmt == "fp4" else K), dtype=np.uint8)
        _same(oracle.decode(fmt, packed, rows, K), refdecode.values(fmt, packed, rows, K))
