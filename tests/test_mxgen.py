"""Checks of the seeded input generator (no GPU).  The generator is input
preparation, not the GEMM; these tests pin its encoders against torch's
float8 cast and the E2M1 tie rules, and its scale choice against the OCP
MX v1.0 rule floor(log2(amax)) - emax."""
import numpy as np
import pytest
import torch

import mxgen
from tests import refdecode


def test_e4m3_encoder_matches_torch_cast():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000) * 100, rng.uniform(-448, 448, 50000),
                        np.ldexp(rng.uniform(1, 2, 20000), rng.integers(-12, 9, 20000)),
                        np.array([0.0, 448.0, -448.0, 464.0, 2.0 ** -10, 3 * 2.0 ** -11, 17.0, 19.0])])
    v = np.clip(v.astype(np.float32), -448, 448).astype(np.float64)
    got = mxgen._encode_e4m3(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # +-0 may differ only in the sign of zero
    same = (got == ref) | ((got & 0x7F) == 0) & ((ref & 0x7F) == 0)
    assert same.all()


def test_e2m1_encoder_ties_and_saturation():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, 7.9, 100.0, -0.25, -5.0, 0.26, 0.24])
    got = refdecode.e2m1(mxgen._encode_e2m1(v))
    assert list(got) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 6.0, -0.0, -4.0, 0.5, 0.0]


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_quantize_roundtrip_of_representable_values(fmt):
    # values that are exactly code * 2^(X-127) with the block amax at the top binade come back unchanged
    a, s = mxgen.random_codes(4, fmt, 16, 256, 110, 140)
    codes = refdecode.unpack(fmt, a, 16, 256)
    vals = refdecode.values(fmt, a, 16, 256)
    top = 6.0 if fmt == "fp4" else 448.0
    codes[:, ::32] = 0x7 if fmt == "fp4" else 0x7E    # force each block's amax to the largest code
    vals[:, ::32] = top
    x = vals * np.repeat(refdecode.e8m0(s), 32, axis=1)
    qa, qs = mxgen.quantize(x.astype(np.float32), fmt)
    assert np.array_equal(qs, s)
    assert np.array_equal(refdecode.values(fmt, qa, 16, 256), vals)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_scale_choice_places_amax_in_top_binade(fmt):
    x = mxgen.normal_bf16(1, (64, 512))
    a, s = mxgen.quantize(x, fmt)
    amax = np.abs(x.astype(np.float64)).reshape(64, 16, 32).max(2)
    scaled = amax / refdecode.e8m0(s)
    lo = 4.0 if fmt == "fp4" else 256.0
    assert np.all((scaled >= lo) & (scaled < 2 * lo))
    # every element is a nearest grid value of x / scale (brute force over all finite codes)
    y = x.astype(np.float64) / np.repeat(refdecode.e8m0(s), 32, axis=1)
    v = refdecode.values(fmt, a, 64, 512)
    grid = refdecode.e2m1(np.arange(16)) if fmt == "fp4" else refdecode.e4m3(np.arange(256))
    grid = grid[np.isfinite(grid)]
    best = np.min(np.abs(y.reshape(-1, 1) - grid.reshape(1, -1)), axis=1).reshape(y.shape)
    assert np.array_equal(np.abs(v - y), best)


def test_zero_block_gets_code_zero():
    x = np.zeros((2, 64), np.float32)
    x[1, 40] = 1.0
    a, s = mxgen.quantize(x, "fp8")
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and s[1, 1] == 127 - 8


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(2).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(mxgen.round_to_bf16(x), ref)


def test_pack_unpack_fp4():
    c = np.random.default_rng(3).integers(0, 16, size=(5, 64), dtype=np.uint8)
    p = mxgen.pack_fp4(c)
    assert p.shape == (5, 32) and p[0, 0] == (c[0, 0] | (c[0, 1] << 4))
    assert np.array_equal(mxgen.unpack_fp4(p), c)


def test_named_case_small_and_seeded():
    c1 = mxgen.case("c1_fp4_32x256x256")
    c1b = mxgen.case("c1_fp4_32x256x256")
    assert c1.a.shape == (32, 128) and c1.b.shape == (256, 128) and c1.sa.shape == (32, 8)
    assert np.array_equal(c1.a, c1b.a) and np.array_equal(c1.sb, c1b.sb)


def test_scale_shift_perturbation_count():
    s = np.full((100, 40), 120, np.uint8)
    t = mxgen._shift_blocks(s, 0.01, 8, 7)
    d = t.astype(int) - s.astype(int)
    assert (d != 0).sum() == 40 and set(np.unique(d[d != 0])) <= {-8, 8}


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_generator_encoder_agrees_with_oracle_quantizer(fmt):
    # the generator's numpy encoder (input synthesis) and the oracle's C
    # quantizer are written independently; on finite bf16 data they must give
    # the same MX codes, so every GEMM input is what the quantization rule makes
    import oracle
    x = mxgen.normal_bf16(41, (96, 512), sigma=3.0)
    x[5, :64] *= np.float32(1e-30)
    x[9, 32:64] = 0.0
    x = mxgen.round_to_bf16(x)
    codes, scales = mxgen.quantize(x, fmt)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    oc, os_ = oracle.quantize(fmt, bits, 96, 512)
    assert np.array_equal(scales, os_)
    assert np.array_equal(codes, oc)
