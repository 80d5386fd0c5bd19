"""Independent element decoders used only to pin the oracle.

They go through torch's own float8 casts (a library routine), never through
the oracle's tables:
  * E4M3 codes -> torch.float8_e4m3fn -> float32;
  * E8M0 codes -> torch.float8_e8m0fnu -> float32;
  * E2M1 codes are mapped bit-wise onto the E4M3 code of the same value
    (sign bit moves to bit 7, the 2-bit exponent is re-biased from 1 to 7,
    the mantissa bit moves to the top of the 3-bit mantissa; the one
    subnormal, 0.5, is the normal E4M3 2^-1) and then decoded by torch.
"""
import numpy as np
import torch

_E4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
with np.errstate(invalid="ignore"):
    _E8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float32).numpy().astype(np.float64)


def e2m1_to_e4m3_code(c: int) -> int:
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    if e == 0:
        mag = 0x30 if m else 0x00          # 0.5 = 2^-1 -> exponent field 6, or zero
    else:
        mag = ((e - 1 + 7) << 3) | (m << 2)
    return (s << 7) | mag


_E2 = np.array([_E4[e2m1_to_e4m3_code(c)] for c in range(16)])


def e4m3(codes):
    return _E4[np.asarray(codes, dtype=np.uint8)]


def e8m0(codes):
    return _E8[np.asarray(codes, dtype=np.uint8)]


def e2m1(codes):
    return _E2[np.asarray(codes, dtype=np.uint8)]


def unpack(fmt, packed, rows, K):
    p = np.asarray(packed, dtype=np.uint8).reshape(rows, -1)
    if fmt == "fp8":
        return p.copy()
    out = np.empty((rows, K), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def values(fmt, packed, rows, K):
    codes = unpack(fmt, packed, rows, K)
    return e2m1(codes) if fmt == "fp4" else e4m3(codes)
