"""CPU oracle for the NT MX block-scaled GEMM (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library and its Python binding never import it,
and it never imports them: the two share no code, tables or helpers.

The arithmetic lives in ``mx_oracle.c`` (plain C, double precision, OpenMP
over output elements); this module only builds and loads it and marshals
numpy arrays.  What is computed (see ``mx_oracle.c`` for the citations):

    C[m,n] = sum_kb 2^(sa[m,kb]-127) 2^(sb[n,kb]-127) sum_j dec(A[m,32kb+j]) dec(B[n,32kb+j])

with one E8M0 scale per 32 consecutive K values, A row-major and B
column-major ("PyTorch 接上 FlyDSL", support matrix row "MXFP 缩放 GEMM" and
the paragraph under it).

Pins (tests/test_oracle_*.py): E4M3 and E8M0 tables against torch's own
float8 casts; E2M1 against the E4M3 bit mapping; the GEMM against exact
rational brute force, float64 matmul of independently decoded operands and
int64 matmul of integer-valued inputs; scale and sign invariants; the
double->bf16/fp16 rounding against exact rational nearest-even and torch.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
_LIB = os.path.join(_HERE, "libmxoracle.so")

FMT = {"fp8": 0, "fp4": 1}

_lib = None


def build(force: bool = False) -> str:
    """Compile mx_oracle.c with gcc (-O2, OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.mx_oracle_decode.argtypes = [ctypes.c_int, P, I64, I64, P]
    lib.mx_oracle_decode_scale.argtypes = [P, I64, P]
    lib.mx_oracle_gemm.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, I64, P, P]
    lib.mx_oracle_gemm_at.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, I64, P, P, I64, P, P]
    lib.mx_oracle_round_bf16.argtypes = [P, I64, P]
    lib.mx_oracle_round_f16.argtypes = [P, I64, P]
    lib.mx_oracle_quantize.argtypes = [ctypes.c_int, P, I64, I64, P, P]
    for f in (lib.mx_oracle_decode, lib.mx_oracle_decode_scale, lib.mx_oracle_gemm,
              lib.mx_oracle_gemm_at, lib.mx_oracle_round_bf16, lib.mx_oracle_round_f16,
              lib.mx_oracle_quantize):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _u8(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.uint8)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _row_bytes(fmt: str, K: int) -> int:
    return K // 2 if fmt == "fp4" else K


def decode(fmt: str, packed, rows: int, K: int) -> np.ndarray:
    """Element values of a packed operand, shape [rows, K], float64."""
    lib = _load()
    p = _u8(packed)
    assert p.size == rows * _row_bytes(fmt, K)
    out = np.empty((rows, K), dtype=np.float64)
    rc = lib.mx_oracle_decode(FMT[fmt], _ptr(p), rows, K, _ptr(out))
    if rc:
        raise ValueError("mx_oracle_decode: %d" % rc)
    return out


def decode_scale(codes) -> np.ndarray:
    """E8M0 codes -> float64 powers of two (NaN for 0xFF)."""
    lib = _load()
    c = _u8(codes)
    out = np.empty(c.shape, dtype=np.float64)
    lib.mx_oracle_decode_scale(_ptr(c), c.size, _ptr(out))
    return out


def _check(fmt, a, b, sa, sb, M, N, K):
    a, b, sa, sb = _u8(a), _u8(b), _u8(sa), _u8(sb)
    rb = _row_bytes(fmt, K)
    if a.size != M * rb or b.size != N * rb or sa.size != M * (K // 32) or sb.size != N * (K // 32):
        raise ValueError("operand sizes do not match M=%d N=%d K=%d (%s)" % (M, N, K, fmt))
    return a, b, sa, sb


def gemm(fmt: str, a, b, sa, sb, M: int, N: int, K: int):
    """Full oracle GEMM.  Returns (c, s): float64 [M, N] each, where s is
    sum_k |a_k b_k| with the scales applied."""
    lib = _load()
    a, b, sa, sb = _check(fmt, a, b, sa, sb, M, N, K)
    c = np.empty((M, N), dtype=np.float64)
    s = np.empty((M, N), dtype=np.float64)
    rc = lib.mx_oracle_gemm(FMT[fmt], _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), M, N, K, _ptr(c), _ptr(s))
    if rc:
        raise ValueError("mx_oracle_gemm: %d" % rc)
    return c, s


def gemm_at(fmt: str, a, b, sa, sb, M: int, N: int, K: int, ms, ns):
    """Oracle values at the listed output positions (ms[i], ns[i])."""
    lib = _load()
    a, b, sa, sb = _check(fmt, a, b, sa, sb, M, N, K)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    assert ms.shape == ns.shape
    c = np.empty(ms.shape, dtype=np.float64)
    s = np.empty(ms.shape, dtype=np.float64)
    rc = lib.mx_oracle_gemm_at(FMT[fmt], _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), M, N, K,
                               _ptr(ms), _ptr(ns), ms.size, _ptr(c), _ptr(s))
    if rc:
        raise ValueError("mx_oracle_gemm_at: %d" % rc)
    return c, s


def group_rows(offs, groups: int, M: int):
    """Row ranges [start, end) of each group of a grouped product: group g
    ends at offs[g] (cumulative sizes, "PyTorch 接上 FlyDSL" support-matrix
    row "Grouped GEMM": groups of A may differ in length, empty groups are
    skipped), with the library's documented reading of arbitrary offs: the
    ends are made non-decreasing and clamped into [0, M]."""
    offs = np.asarray(offs, dtype=np.int64).reshape(groups)
    ranges = []
    end = 0
    for g in range(groups):
        start = end
        end = min(M, max(int(offs[g]), start))
        ranges.append((start, end))
    return ranges


def grouped_gemm(fmt: str, a, b, sa, sb, offs, groups: int, M: int, N: int, K: int):
    """Grouped product, group by group: rows [start_g, end_g) of A (and of its
    scales) times B[g] ([groups][N][K] operand, [groups][N][K/32] scales)
    with the plain oracle GEMM.  Returns (c, s, covered): float64 [M, N]
    values and sum |a_k b_k| (NaN in rows no group covers) and the bool
    [M] mask of covered rows."""
    rb = _row_bytes(fmt, K)
    a = _u8(a).reshape(M, rb) if M else _u8(a).reshape(0, rb)
    sa = _u8(sa).reshape(M, K // 32) if M else _u8(sa).reshape(0, K // 32)
    b = _u8(b).reshape(groups, N, rb)
    sb = _u8(sb).reshape(groups, N, K // 32)
    c = np.full((M, N), np.nan)
    s = np.full((M, N), np.nan)
    covered = np.zeros(M, dtype=bool)
    for g, (r0, r1) in enumerate(group_rows(offs, groups, M)):
        if r1 > r0:
            c[r0:r1], s[r0:r1] = gemm(fmt, a[r0:r1], b[g], sa[r0:r1], sb[g], r1 - r0, N, K)
            covered[r0:r1] = True
    return c, s, covered


def dense_values(dtype: str, bits, shape) -> np.ndarray:
    """BF16 or FP16 bit patterns (uint16) -> float64 values, exactly."""
    u = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).reshape(shape)
    if dtype == "bf16":
        return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return u.view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def dense_gemm(dtype: str, trans_a: int, trans_b: int, a_bits, b_bits, M: int, N: int, K: int):
    """Dense BF16 / FP16 product C = A B ("PyTorch 接上 FlyDSL", support-matrix
    row for torch.mm: FP16/BF16, static 2-D, NN / NT / TN / TT), in double.
    A is stored [M][K] (trans_a 0) or [K][M] (trans_a 1); B is stored [K][N]
    (trans_b 0) or [N][K] (trans_b 1).  Returns (c, s): float64 [M, N] and
    sum_k |a_mk b_kn|.  A float64 matmul is exact here only up to double
    rounding; products of BF16/FP16 values are exact in double and the sums
    carry a relative error below K * 2^-53, far inside any GPU tolerance."""
    A = dense_values(dtype, a_bits, (K, M) if trans_a else (M, K))
    B = dense_values(dtype, b_bits, (N, K) if trans_b else (K, N))
    A = A.T if trans_a else A
    B = B.T if trans_b else B
    return A @ B, np.abs(A) @ np.abs(B)


ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_TANH = 0, 1, 2, 3


def activation(act: int, x):
    """The epilogue activations in double precision, from their definitions:
    ReLU max(x, 0); SiLU x * sigmoid(x) = x / (1 + e^-x); GELU with the tanh
    form 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, dtype=np.float64)
    if act == ACT_NONE:
        return x.copy()
    if act == ACT_RELU:
        return np.where(x > 0, x, 0.0)
    with np.errstate(over="ignore"):
        if act == ACT_SILU:
            return x / (1.0 + np.exp(-x))
        if act == ACT_GELU_TANH:
            return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))
    raise ValueError("unknown activation %r" % act)


def epilogue(c, bias_bf16, act: int):
    """GEMM tail fusion (roadmap item "GEMM 尾部融合" of "PyTorch 接上 FlyDSL"):
    per-column bias (BF16 bit patterns [N], or None) added to the exact
    product, then the activation; double precision.  Returns (y, slope):
    y and |d act / d x| at the pre-activation value (used to carry the
    product's error bound through the activation)."""
    x = np.asarray(c, dtype=np.float64)
    if bias_bf16 is not None:
        b = (np.asarray(bias_bf16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
        x = x + b.astype(np.float64)[None, :]
    y = activation(act, x)
    if act == ACT_NONE:
        slope = np.ones_like(x)
    elif act == ACT_RELU:
        slope = (x > 0).astype(np.float64)
    else:
        # |act'| of SiLU and tanh-GELU stays below 1.13 everywhere
        slope = np.full_like(x, 1.13)
    return y, slope


def round_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), round-to-nearest-even, direct."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.mx_oracle_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


def round_f16(x) -> np.ndarray:
    """float64 -> fp16 bit patterns (uint16), round-to-nearest-even, direct."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.mx_oracle_round_f16(_ptr(x), x.size, _ptr(out))
    return out


def quantize(fmt: str, x_bf16, rows: int, K: int):
    """MX-quantize BF16 rows (uint16 bit patterns, [rows][K], K % 32 == 0) along K.

    Returns (codes, scales): codes [rows][K/2] (fp4, two per byte, even k low
    nibble) or [rows][K] (fp8) uint8, scales [rows][K/32] E8M0 uint8.  The
    rule (OCP MX v1.0 conversion; the pages only name BlockWise1x32 E8M0
    scales, "PyTorch 接上 FlyDSL", 5ulink.com, 支持边界): scale code =
    floor(log2 amax) - emax + 127 clamped to [0, 254] (emax 2 / 8, 0 for an
    all-zero block, 0xFF for a block holding NaN or Inf); elements rounded to
    the nearest code, ties to even, saturating; sign from the input.
    """
    x = np.ascontiguousarray(np.asarray(x_bf16, dtype=np.uint16).reshape(rows, K))
    codes = np.zeros((rows, K // 2 if fmt == "fp4" else K), dtype=np.uint8)
    scales = np.zeros((rows, K // 32), dtype=np.uint8)
    rc = _load().mx_oracle_quantize(FMT[fmt], _ptr(x), rows, K, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("mx_oracle_quantize: invalid arguments")
    return codes, scales
