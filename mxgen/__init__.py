"""Seeded synthetic inputs for the NT MX block-scaled GEMM.

This module is shared by the GPU tests, the oracle tests, the benchmark and
the smoke check.  It produces packed operand bytes and E8M0 scale bytes and
nothing else: it holds none of the GEMM's arithmetic (no decoding of packed
operands back to values, no products, no sums over K).  Both the GPU path
and the oracle consume exactly the bytes made here.

Recipe (one reading per step; the pages fix only "one E8M0 scale per 32
values" and that measurement starts from already-quantized inputs):
  1. draw float32 N(0, sigma^2) from numpy's PCG64 with a fixed seed;
  2. optional outlier columns are multiplied before rounding;
  3. round to bf16 (round-to-nearest-even);
  4. per block of 32 consecutive K values: amax = max |x|; the shared scale
     exponent is floor(log2(amax)) - emax, with emax = 2 for E2M1 and 8 for
     E4M3 (OCP MX v1.0 scale choice), stored as an E8M0 code clamped to
     [0, 254]; an all-zero block gets code 0;
  5. each value divided by its block scale is rounded to the nearest element
     code (ties to even mantissa), saturating at +-6 (E2M1) / +-448 (E4M3);
  6. FP4 codes are packed two per byte, even k in the low nibble.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

EMAX = {"fp4": 2, "fp8": 8}
ELEM_MAX = {"fp4": 6.0, "fp8": 448.0}


# --------------------------------------------------------------------------- bf16

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (ties to even).
    Inputs are finite (normal draws); NaN/Inf are not produced here."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs: u <= 0xFF7FFFFF, so u + 0x8000 cannot wrap in uint32
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.view(np.float32)


def normal_bf16(seed: int, shape: Tuple[int, int], sigma: float = 1.0,
                outlier_rows: Optional[np.ndarray] = None, outlier_mult: float = 1.0) -> np.ndarray:
    """Seeded N(0, sigma^2) draw rounded to bf16, as float32 [rows, K]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if outlier_rows is not None and len(outlier_rows):
        x[outlier_rows] *= np.float32(outlier_mult)
    return round_to_bf16(x)


# ----------------------------------------------------------------- quantization

def _block_scale_codes(xb: np.ndarray, fmt: str) -> np.ndarray:
    """xb: [rows, nblk, 32] float64 -> E8M0 codes [rows, nblk] (uint8)."""
    amax = np.max(np.abs(xb), axis=2)
    _, ex = np.frexp(amax)                      # amax = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1 - EMAX[fmt]     # floor(log2(amax)) - emax
    code = np.clip(e + 127, 0, 254)
    code[amax == 0] = 0
    return code.astype(np.uint8)


def _encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (ties to even mantissa, saturating at 6)."""
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, 0)               # binade, 0 covers the subnormal step
    q = np.ldexp(1.0, e - 1)                                 # 1 mantissa bit
    r = np.minimum(np.rint(a / q) * q, 6.0)
    # encode r in {0, .5, 1, 1.5, 2, 3, 4, 6}
    _, er = np.frexp(np.where(r > 0, r, 1.0))
    er = er.astype(np.int64) - 1
    mant = np.where(r >= 1.0, np.rint(r / np.ldexp(1.0, er - 1)) - 2, 0).astype(np.int64)
    expf = np.where(r >= 1.0, er + 1, 0)
    code = np.where(r >= 1.0, (expf << 1) | mant, np.where(r == 0.5, 1, 0))
    sign = np.signbit(v).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


def _encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 (OCP "FN") code, ties to even mantissa, saturating at 448."""
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    q = np.ldexp(1.0, e - 3)                                 # 3 mantissa bits
    r = np.minimum(np.rint(a / q) * q, 448.0)
    sub = r < 2.0 ** -6
    _, er = np.frexp(np.where(r > 0, r, 1.0))
    er = er.astype(np.int64) - 1
    mant_n = np.rint(r / np.ldexp(1.0, er - 3)).astype(np.int64) - 8
    code_n = ((er + 7) << 3) | mant_n
    code_s = np.rint(r / 2.0 ** -9).astype(np.int64)
    code = np.where(sub, code_s, code_n)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """[rows, K] nibble codes -> [rows, K/2] bytes, even k in the low nibble."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_fp4 (a byte shuffle; no values are formed)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def quantize(x: np.ndarray, fmt: str, chunk_rows: int = 2048) -> Tuple[np.ndarray, np.ndarray]:
    """x: [rows, K] float32 (bf16-valued) -> (packed codes, E8M0 scales [rows, K/32])."""
    rows, K = x.shape
    assert K % 32 == 0
    nblk = K // 32
    codes = np.empty((rows, K // 2 if fmt == "fp4" else K), dtype=np.uint8)
    scales = np.empty((rows, nblk), dtype=np.uint8)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        xb = x[r0:r1].astype(np.float64).reshape(r1 - r0, nblk, 32)
        sc = _block_scale_codes(xb, fmt)
        v = np.ldexp(xb, -(sc.astype(np.int64)[..., None] - 127)).reshape(r1 - r0, K)
        if fmt == "fp4":
            codes[r0:r1] = pack_fp4(_encode_e2m1(v))
        else:
            codes[r0:r1] = _encode_e4m3(v)
        scales[r0:r1] = sc
    return codes, scales


# ------------------------------------------------------------------ test inputs

def random_codes(seed: int, fmt: str, rows: int, K: int, scale_lo: int = 120, scale_hi: int = 134,
                 allow_nan: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Uniformly random packed codes and scale codes in [scale_lo, scale_hi].
    E4M3 NaN codes (0x7F, 0xFF) are excluded unless allow_nan."""
    rng = np.random.default_rng(seed)
    if fmt == "fp4":
        codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    else:
        codes = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
        if not allow_nan:
            nan = (codes & 0x7F) == 0x7F
            codes[nan] ^= 0x01
    scales = rng.integers(scale_lo, scale_hi + 1, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales


@dataclasses.dataclass
class Case:
    name: str
    fmt: str
    M: int
    N: int
    K: int
    a: np.ndarray        # packed A [M][K/2 or K]
    b: np.ndarray        # packed B [N][K/2 or K]
    sa: np.ndarray       # [M][K/32]
    sb: np.ndarray       # [N][K/32]
    recipe: str

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def algorithmic_bytes(self, out_bytes: int = 2) -> float:
        e = 0.5 if self.fmt == "fp4" else 1.0
        return (self.M + self.N) * self.K * e + (self.M + self.N) * self.K / 32 + self.M * self.N * out_bytes


def _shift_blocks(scales: np.ndarray, frac: float, shift: int, seed: int) -> np.ndarray:
    """Move round(frac * #blocks) scale codes, chosen without replacement,
    by +-shift (fair coin per block).  Raises if a code would leave [0, 254]."""
    rng = np.random.default_rng(seed)
    flat = scales.reshape(-1).astype(np.int64)
    n = int(round(frac * flat.size))
    idx = rng.choice(flat.size, size=n, replace=False)
    sgn = np.where(rng.integers(0, 2, size=n) == 1, 1, -1)
    flat[idx] += sgn * shift
    if flat.min() < 0 or flat.max() > 254:
        raise ValueError("scale shift left the E8M0 range")
    return flat.astype(np.uint8).reshape(scales.shape)


def make_case(name: str, fmt: str, M: int, N: int, K: int, case_id: int,
              sigma_a: float = 1.0, sigma_b: float = 1.0, outlier_frac: float = 0.0,
              outlier_mult: float = 1.0, shift_frac: float = 0.0, shift: int = 0) -> Case:
    """Seeded recipe: seed = 1000*case_id + {A: 1, B: 2, scale shift: 3, outliers: 4}."""
    xa = normal_bf16(1000 * case_id + 1, (M, K), sigma_a)
    out_rows = None
    if outlier_frac > 0:
        rng = np.random.default_rng(1000 * case_id + 4)
        out_rows = np.sort(rng.choice(N, size=int(round(outlier_frac * N)), replace=False))
    xb = normal_bf16(1000 * case_id + 2, (N, K), sigma_b, out_rows, outlier_mult)
    a, sa = quantize(xa, fmt)
    del xa
    b, sb = quantize(xb, fmt)
    del xb
    recipe = "A~N(0,%g) B~N(0,%g)" % (sigma_a, sigma_b)
    if shift_frac > 0:
        sa = _shift_blocks(sa, shift_frac, shift, 1000 * case_id + 3)
        sb = _shift_blocks(sb, shift_frac, shift, 1000 * case_id + 5)
        recipe += ", %g%% of scale blocks shifted by +-%d" % (100 * shift_frac, shift)
    if out_rows is not None:
        recipe += ", %d outlier columns of B x%g" % (len(out_rows), outlier_mult)
    return Case(name, fmt, M, N, K, a, b, sa, sb, recipe)


# Named workloads.  The pages plot 17 MXFP8 and 17 MXFP4 NT shapes without
# listing them; the one they name is 32x14336x4096 (the MXFP4 peak).  These
# stand in for that suite: decode-width GEMMs at the projection widths of the
# models the pages serve (8B / 32B / 70B-class MLPs), a 70B-style MLP
# up-projection at 256 concurrent tokens, and one compute-bound square.
NAMED = {
    "c1_fp4_32x256x256": dict(fmt="fp4", M=32, N=256, K=256, case_id=1),
    "c2_fp4_32x14336x4096": dict(fmt="fp4", M=32, N=14336, K=4096, case_id=2, shift_frac=0.01, shift=8),
    "c3_fp8_64x4096x4096": dict(fmt="fp8", M=64, N=4096, K=4096, case_id=3),
    "c4a_fp8_256x28672x8192": dict(fmt="fp8", M=256, N=28672, K=8192, case_id=4, sigma_b=0.02,
                                    outlier_frac=0.001, outlier_mult=20.0),
    "c4b_fp4_256x28672x8192": dict(fmt="fp4", M=256, N=28672, K=8192, case_id=5, sigma_b=0.02,
                                    outlier_frac=0.001, outlier_mult=20.0),
    "c5_fp4_8192x8192x8192": dict(fmt="fp4", M=8192, N=8192, K=8192, case_id=6),
}
SWEEP_M = (1, 8, 32, 128, 512, 2048)
SWEEP_NK = ((4096, 4096), (14336, 4096), (4096, 14336), (25600, 5120))
for _i, _m in enumerate(SWEEP_M):
    for _j, (_n, _k) in enumerate(SWEEP_NK):
        NAMED["sw_fp4_%dx%dx%d" % (_m, _n, _k)] = dict(fmt="fp4", M=_m, N=_n, K=_k, case_id=100 + 10 * _i + _j)


def case(name: str) -> Case:
    spec = dict(NAMED[name])
    return make_case(name, **spec)


def case_shape(name: str) -> Tuple[str, int, int, int]:
    s = NAMED[name]
    return s["fmt"], s["M"], s["N"], s["K"]


# ------------------------------------------------------------ grouped inputs

@dataclasses.dataclass
class GroupedCase:
    name: str
    fmt: str
    G: int
    M: int               # rows of A over all groups
    N: int
    K: int
    sizes: np.ndarray    # rows per group (int64 [G]); zeros are empty groups
    offs: np.ndarray     # cumulative ends (int32 [G]), as the grouped entry points take them
    a: np.ndarray        # packed A [M][K/2 or K]
    b: np.ndarray        # packed B [G*N][K/2 or K] (group-major)
    sa: np.ndarray       # [M][K/32]
    sb: np.ndarray       # [G*N][K/32]
    recipe: str

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def algorithmic_bytes(self, out_bytes: int = 2) -> float:
        """A, the B operands (and scales) of the non-empty groups, C."""
        e = 0.5 if self.fmt == "fp4" else 1.0
        used = int(np.count_nonzero(self.sizes))
        return (self.M + used * self.N) * self.K * (e + 1.0 / 32) + self.M * self.N * out_bytes


def grouped_sizes(seed: int, G: int, M: int, n_empty: int, skew: float = 0.8) -> np.ndarray:
    """Rows per group for an unbalanced mixture-of-experts routing: n_empty
    groups get no rows; the others draw M rows multinomially with weights
    1/(rank+1)^skew over a seeded random ranking."""
    rng = np.random.default_rng(seed)
    live = np.sort(rng.choice(G, size=G - n_empty, replace=False))
    w = 1.0 / (rng.permutation(len(live)) + 1.0) ** skew
    sizes = np.zeros(G, dtype=np.int64)
    sizes[live] = rng.multinomial(M, w / w.sum())
    return sizes


def make_grouped_case(name: str, fmt: str, G: int, M: int, N: int, K: int, case_id: int,
                      n_empty: int = 0, sigma_b: float = 1.0) -> GroupedCase:
    """Seeded recipe: seed = 1000*case_id + {A: 1, B: 2, group sizes: 6}."""
    sizes = grouped_sizes(1000 * case_id + 6, G, M, n_empty)
    xa = normal_bf16(1000 * case_id + 1, (M, K))
    a, sa = quantize(xa, fmt)
    del xa
    xb = normal_bf16(1000 * case_id + 2, (G * N, K), sigma_b)
    b, sb = quantize(xb, fmt)
    del xb
    recipe = ("A~N(0,1) B~N(0,%g), %d groups, %d empty, rows per group %s"
              % (sigma_b, G, n_empty, ",".join(str(int(s)) for s in sizes)))
    offs = np.cumsum(sizes).astype(np.int32)
    return GroupedCase(name, fmt, G, M, N, K, sizes, offs, a, b, sa, sb, recipe)


# Grouped workloads.  The pages run 24 unlisted grouped-GEMM cases, five of
# them with unbalanced experts including empty ones; these stand in for
# them at the MXFP8 precision of the roadmap's grouped kernel: a prefill
# batch over 8 experts (8192 routed rows, one expert empty) and a decode
# step over 32 experts (256 routed rows, 5 experts empty).
GROUPED = {
    "g1_fp8_8x8192x4096x4096": dict(fmt="fp8", G=8, M=8192, N=4096, K=4096, case_id=201, n_empty=1),
    "g2_fp8_32x256x2048x2048": dict(fmt="fp8", G=32, M=256, N=2048, K=2048, case_id=202, n_empty=5),
}


def grouped_case(name: str) -> GroupedCase:
    return make_grouped_case(name, **GROUPED[name])
