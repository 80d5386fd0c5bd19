"""Python binding of the gfx950 NT MX block-scaled GEMM library (libmxgemm.so).

Argument marshalling only: every step of the product runs in the HIP
kernels of ``csrc/``.  PyTorch supplies device memory and the stream.  The
functions carry the C ABI's names (see ``include/mxgemm.h``):

    mx_scaled_mm_fp4(a, b, a_scale, b_scale, c, M, N, K, out_dtype=None, workspace="auto", stream=None)
    mx_scaled_mm_fp8(...)
    mx_scaled_mm_workspace_bytes(is_fp4, M, N, K)
    mx_scaled_mm_config(is_fp4, a, b, a_scale, b_scale, c, M, N, K, variant, splits=1,
                        workspace="auto", out_dtype=None, stream=None)
    mx_default_config(is_fp4, M, N, K, with_workspace=True) -> (variant, splits)
    mx_default_variant(is_fp4, M, N, K)

``a``/``b`` are contiguous 1-byte CUDA tensors holding packed codes
([M, K/2] / [N, K/2] for MXFP4, [M, K] / [N, K] for MXFP8), the scales are
[M, K/32] / [N, K/32] E8M0 bytes, ``c`` is a contiguous [M, N] tensor of
the output dtype.  A non-zero status raises MxGemmError (the caller's cue to
fall back to another implementation).  There is no CPU fallback: if the
library is missing, importing this package raises.

``scaled_mm`` is the convenience form that allocates C and returns it.
"""
from __future__ import annotations

import ctypes
import os

import torch  # load torch's HIP runtime first so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxgemm.so")

OUT_BF16, OUT_F16, OUT_F32 = 0, 1, 2
_OUT_OF_DTYPE = {torch.bfloat16: OUT_BF16, torch.float16: OUT_F16, torch.float32: OUT_F32}
_DTYPE_OF_OUT = {v: k for k, v in _OUT_OF_DTYPE.items()}

if not os.path.exists(LIB_PATH):
    raise ImportError("libmxgemm.so is not built (%s); run __graft_entry__.build() or "
                      "python block_scaled_precision_mm_amd/build.py" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_INT = ctypes.c_int
_lib.mx_scaled_mm_fp4.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _P, _SZ, _P]
_lib.mx_scaled_mm_fp8.argtypes = _lib.mx_scaled_mm_fp4.argtypes
_lib.mx_scaled_mm_config.argtypes = [_INT, _P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _INT, _INT, _P, _SZ, _P]
_lib.mx_scaled_mm_workspace_bytes.argtypes = [_INT, _I64, _I64, _I64]
_lib.mx_scaled_mm_workspace_bytes.restype = _SZ
_lib.mx_config_workspace_bytes.argtypes = [_INT, _INT, _I64, _I64]
_lib.mx_config_workspace_bytes.restype = _SZ
_lib.mx_default_config.argtypes = [_INT, _I64, _I64, _I64, _INT, ctypes.POINTER(_INT)]
_lib.mx_default_variant.argtypes = [_INT, _I64, _I64, _I64]
_lib.mx_scaled_mm_noalloc.argtypes = [_INT, _P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _P]
_lib.mx_noalloc_scratch_bytes.restype = _SZ
_lib.mx_variant_max_k.argtypes = [_INT, _INT]
_lib.mx_variant_max_k.restype = _I64
_lib.mx_status_string.argtypes = [_INT]
_lib.mx_status_string.restype = ctypes.c_char_p
_lib.mx_variant_name.argtypes = [_INT]
_lib.mx_variant_name.restype = ctypes.c_char_p
_lib.mx_quantize_bf16.argtypes = [_P, _P, _P, _I64, _I64, _INT, _P]
_lib.mx_grouped_mm_fp4.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _INT, _P]
_lib.mx_grouped_mm_fp8.argtypes = _lib.mx_grouped_mm_fp4.argtypes
_lib.mx_grouped_mm_config.argtypes = [_INT, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _INT, _INT, _P]
_lib.mx_grouped_variant_name.argtypes = [_INT]
_lib.mx_grouped_variant_name.restype = ctypes.c_char_p
_lib.mx_grouped_default_variant.argtypes = [_I64, _I64, _I64]
_lib.mx_scaled_mm_fused.argtypes = [_INT, _P, _P, _P, _P, _P, _INT, _P, _P, _I64, _I64, _I64, _INT, _INT, _P]
_lib.mx_fused_variant_name.argtypes = [_INT]
_lib.mx_fused_variant_name.restype = ctypes.c_char_p
_lib.mx_fused_default_variant.argtypes = [_INT, _I64, _I64, _I64]
_lib.mx_fused_variant_max_k.argtypes = [_INT, _INT]
_lib.mx_fused_variant_max_k.restype = _I64
_lib.mx_dense_gemm.argtypes = [_INT, _INT, _INT, _P, _P, _P, _I64, _I64, _I64, _INT, _P]
_lib.mx_empty_like.argtypes = [_INT, _I64, _I64, _I64, _P]
for _f in ("mx_scaled_mm_fp4", "mx_scaled_mm_fp8", "mx_scaled_mm_config", "mx_num_variants",
           "mx_default_config", "mx_scaled_mm_noalloc",
           "mx_last_hip_error", "mx_abi_version", "mx_default_variant", "mx_quantize_bf16",
           "mx_grouped_mm_fp4", "mx_grouped_mm_fp8", "mx_grouped_mm_config",
           "mx_grouped_num_variants", "mx_grouped_default_variant", "mx_scaled_mm_fused",
           "mx_fused_num_variants", "mx_fused_default_variant", "mx_dense_gemm", "mx_empty_like"):
    getattr(_lib, _f).restype = _INT

# every symbol include/mxgemm.h declares
EXPORTS = ("mx_scaled_mm_fp4", "mx_scaled_mm_fp8", "mx_scaled_mm_config", "mx_num_variants",
           "mx_scaled_mm_workspace_bytes", "mx_config_workspace_bytes", "mx_default_config",
           "mx_scaled_mm_noalloc", "mx_noalloc_scratch_bytes",
           "mx_variant_max_k", "mx_variant_name", "mx_default_variant", "mx_status_string",
           "mx_last_hip_error", "mx_abi_version", "mx_quantize_bf16",
           "mx_grouped_mm_fp4", "mx_grouped_mm_fp8", "mx_grouped_mm_config",
           "mx_grouped_num_variants", "mx_grouped_variant_name", "mx_grouped_default_variant",
           "mx_scaled_mm_fused", "mx_fused_num_variants", "mx_fused_variant_name",
           "mx_fused_default_variant", "mx_fused_variant_max_k", "mx_dense_gemm", "mx_empty_like")


class MxGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.mx_status_string(status).decode()
        if status == -8:
            msg += " (hipError %d)" % _lib.mx_last_hip_error()
        super().__init__("%s: %s (status %d)" % (where, msg, status))


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check_tensors(is_fp4, a, b, sa, sb, c, M, N, K):
    """Shape/contiguity checks on torch tensors (ints pass through as raw pointers)."""
    eb = K // 2 if is_fp4 else K
    for name, t, rows, cols in (("a", a, M, eb), ("b", b, N, eb), ("a_scale", sa, M, K // 32),
                                ("b_scale", sb, N, K // 32)):
        if isinstance(t, torch.Tensor):
            if not t.is_cuda or not t.is_contiguous() or t.element_size() != 1:
                raise ValueError("%s must be a contiguous 1-byte CUDA tensor" % name)
            if t.numel() != rows * cols:
                raise ValueError("%s has %d bytes, expected %d x %d" % (name, t.numel(), rows, cols))
    if isinstance(c, torch.Tensor):
        if not c.is_cuda or not c.is_contiguous() or c.numel() != M * N:
            raise ValueError("c must be a contiguous CUDA tensor with M*N elements")


def _out_code(c, out_dtype):
    if out_dtype is not None:
        return out_dtype
    if isinstance(c, torch.Tensor):
        return _OUT_OF_DTYPE[c.dtype]
    raise ValueError("out_dtype is required when c is a raw pointer")


_WORKSPACES = {}


def _workspace(ws, nbytes, stream_ptr):
    """(pointer, bytes) of the split-K workspace argument (see the module doc)."""
    if ws is None or nbytes == 0:
        return 0, 0
    if isinstance(ws, torch.Tensor):
        if not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA tensor")
        return ws.data_ptr(), ws.numel() * ws.element_size()
    if ws != "auto":
        raise ValueError("workspace must be a tensor, None or 'auto'")
    key = (torch.cuda.current_device(), stream_ptr)
    t = _WORKSPACES.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        _WORKSPACES[key] = t
    return t.data_ptr(), t.numel()


def mx_scaled_mm_workspace_bytes(is_fp4, M, N, K) -> int:
    return int(_lib.mx_scaled_mm_workspace_bytes(int(bool(is_fp4)), M, N, K))


def mx_config_workspace_bytes(variant, splits, M, N) -> int:
    return int(_lib.mx_config_workspace_bytes(variant, splits, M, N))


def _default(is_fp4, a, b, a_scale, b_scale, c, M, N, K, out_dtype, workspace, stream, fn, name):
    _check_tensors(is_fp4, a, b, a_scale, b_scale, c, M, N, K)
    st_ptr = _stream(stream)
    wp, wb = _workspace(workspace, mx_scaled_mm_workspace_bytes(is_fp4, M, N, K), st_ptr)
    st = fn(_ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale), _ptr(c), M, N, K, _out_code(c, out_dtype),
            wp, wb, st_ptr)
    if st:
        raise MxGemmError(st, name)


def mx_scaled_mm_fp4(a, b, a_scale, b_scale, c, M, N, K, out_dtype=None, workspace="auto",
                     stream=None) -> None:
    _default(True, a, b, a_scale, b_scale, c, M, N, K, out_dtype, workspace, stream,
             _lib.mx_scaled_mm_fp4, "mx_scaled_mm_fp4")


def mx_scaled_mm_fp8(a, b, a_scale, b_scale, c, M, N, K, out_dtype=None, workspace="auto",
                     stream=None) -> None:
    _default(False, a, b, a_scale, b_scale, c, M, N, K, out_dtype, workspace, stream,
             _lib.mx_scaled_mm_fp8, "mx_scaled_mm_fp8")


def mx_scaled_mm_config(is_fp4, a, b, a_scale, b_scale, c, M, N, K, variant, splits=1,
                        workspace="auto", out_dtype=None, stream=None) -> None:
    _check_tensors(bool(is_fp4), a, b, a_scale, b_scale, c, M, N, K)
    st_ptr = _stream(stream)
    wp, wb = _workspace(workspace, mx_config_workspace_bytes(variant, splits, M, N), st_ptr)
    st = _lib.mx_scaled_mm_config(int(bool(is_fp4)), _ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale),
                                  _ptr(c), M, N, K, _out_code(c, out_dtype), variant, splits, wp, wb, st_ptr)
    if st:
        raise MxGemmError(st, "mx_scaled_mm_config")


def mx_default_config(is_fp4, M, N, K, with_workspace=True):
    """(variant, K parts) of the default entry points for this shape."""
    sp = _INT(0)
    v = int(_lib.mx_default_config(int(bool(is_fp4)), M, N, K, int(bool(with_workspace)), ctypes.byref(sp)))
    if v < 0:
        raise MxGemmError(v, "mx_default_config")
    return v, int(sp.value)


def mx_default_variant(is_fp4, M, N, K) -> int:
    v = int(_lib.mx_default_variant(int(bool(is_fp4)), M, N, K))
    if v < 0:
        raise MxGemmError(v, "mx_default_variant")
    return v


def mx_num_variants() -> int:
    return int(_lib.mx_num_variants())


def mx_variant_max_k(variant, is_fp4) -> int:
    v = int(_lib.mx_variant_max_k(variant, int(bool(is_fp4))))
    if v < 0:
        raise MxGemmError(v, "mx_variant_max_k")
    return v


def variants_for(is_fp4, K):
    """Every variant that accepts this format and K."""
    return [v for v in range(mx_num_variants()) if K <= mx_variant_max_k(v, is_fp4)]


def mx_variant_name(variant) -> str | None:
    r = _lib.mx_variant_name(variant)
    return None if r is None else r.decode()


def mx_status_string(status) -> str:
    return _lib.mx_status_string(status).decode()


def mx_last_hip_error() -> int:
    return int(_lib.mx_last_hip_error())


def mx_abi_version() -> int:
    return int(_lib.mx_abi_version())


def mx_quantize_bf16(x, codes, scales, rows: int, K: int, is_fp4: bool, stream=None) -> None:
    """MX-quantize BF16 rows along K on the GPU (C ABI mx_quantize_bf16).

    x: bfloat16 [rows][K] (or a raw device pointer); codes: uint8 [rows][K/2]
    (E2M1, two per byte, even k low nibble) or [rows][K] (E4M3); scales:
    uint8 [rows][K/32] E8M0.  Argument marshalling only.
    """
    if isinstance(x, torch.Tensor):
        if not x.is_cuda or not x.is_contiguous() or x.element_size() != 2 or x.numel() != rows * K:
            raise ValueError("x must be a contiguous 2-byte CUDA tensor with rows*K elements")
    for name, t, n in (("codes", codes, rows * (K // 2 if is_fp4 else K)), ("scales", scales, rows * (K // 32))):
        if isinstance(t, torch.Tensor):
            if not t.is_cuda or not t.is_contiguous() or t.element_size() != 1 or t.numel() != n:
                raise ValueError("%s must be a contiguous 1-byte CUDA tensor of %d elements" % (name, n))
    rc = _lib.mx_quantize_bf16(_ptr(x), _ptr(codes), _ptr(scales), rows, K, 1 if is_fp4 else 0,
                               _stream(stream))
    if rc != 0:
        raise MxGemmError(rc, "mx_quantize_bf16")


def _check_grouped(is_fp4, a, b, sa, sb, c, offs, groups, M, N, K):
    eb = K // 2 if is_fp4 else K
    for name, t, n in (("a", a, M * eb), ("b", b, groups * N * eb), ("a_scale", sa, M * (K // 32)),
                       ("b_scale", sb, groups * N * (K // 32))):
        if isinstance(t, torch.Tensor):
            if not t.is_cuda or not t.is_contiguous() or t.element_size() != 1 or t.numel() != n:
                raise ValueError("%s must be a contiguous 1-byte CUDA tensor of %d bytes" % (name, n))
    if isinstance(c, torch.Tensor):
        if not c.is_cuda or not c.is_contiguous() or c.numel() != M * N:
            raise ValueError("c must be a contiguous CUDA tensor with M*N elements")
    if isinstance(offs, torch.Tensor):
        if not offs.is_cuda or offs.dtype != torch.int32 or not offs.is_contiguous() or offs.numel() != groups:
            raise ValueError("offs must be a contiguous int32 CUDA tensor of `groups` elements")


def mx_grouped_mm_fp4(a, b, a_scale, b_scale, c, offs, groups, M, N, K, out_dtype=None,
                      stream=None) -> None:
    """Grouped MXFP4 product (C ABI mx_grouped_mm_fp4): rows [offs[g-1], offs[g])
    of a times b[g] (b is [groups][N][K/2]); offs is an int32 device tensor."""
    _check_grouped(True, a, b, a_scale, b_scale, c, offs, groups, M, N, K)
    st = _lib.mx_grouped_mm_fp4(_ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale), _ptr(c), _ptr(offs),
                                groups, M, N, K, _out_code(c, out_dtype), _stream(stream))
    if st:
        raise MxGemmError(st, "mx_grouped_mm_fp4")


def mx_grouped_mm_fp8(a, b, a_scale, b_scale, c, offs, groups, M, N, K, out_dtype=None,
                      stream=None) -> None:
    """Grouped MXFP8 product (C ABI mx_grouped_mm_fp8); b is [groups][N][K]."""
    _check_grouped(False, a, b, a_scale, b_scale, c, offs, groups, M, N, K)
    st = _lib.mx_grouped_mm_fp8(_ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale), _ptr(c), _ptr(offs),
                                groups, M, N, K, _out_code(c, out_dtype), _stream(stream))
    if st:
        raise MxGemmError(st, "mx_grouped_mm_fp8")


def mx_grouped_mm_config(is_fp4, a, b, a_scale, b_scale, c, offs, groups, M, N, K, variant,
                         out_dtype=None, stream=None) -> None:
    _check_grouped(bool(is_fp4), a, b, a_scale, b_scale, c, offs, groups, M, N, K)
    st = _lib.mx_grouped_mm_config(int(bool(is_fp4)), _ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale),
                                   _ptr(c), _ptr(offs), groups, M, N, K, _out_code(c, out_dtype),
                                   variant, _stream(stream))
    if st:
        raise MxGemmError(st, "mx_grouped_mm_config")


def mx_grouped_num_variants() -> int:
    return _lib.mx_grouped_num_variants()


def mx_grouped_variant_name(variant) -> str | None:
    n = _lib.mx_grouped_variant_name(variant)
    return n.decode() if n is not None else None


def mx_grouped_default_variant(groups, M, N) -> int:
    return _lib.mx_grouped_default_variant(groups, M, N)


OUT_BF16, OUT_F16, OUT_F32, OUT_MXFP8, OUT_MXFP4 = 0, 1, 2, 3, 4
ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_TANH = 0, 1, 2, 3


def mx_scaled_mm_fused(is_fp4, a, b, a_scale, b_scale, bias, act, c, c_scale, M, N, K,
                       out_kind=None, variant=-1, stream=None) -> None:
    """MX GEMM with a fused epilogue (C ABI mx_scaled_mm_fused):
    y = act(A B^T + bias) into c (BF16/FP16/FP32, the dtype of c unless
    out_kind is given) or, with out_kind OUT_MXFP8 / OUT_MXFP4, MX codes into
    c (uint8 [M][N] or [M][N/2]) and E8M0 codes into c_scale (uint8 [M][N/32]).
    bias: bfloat16 [N] tensor or None.  Argument marshalling only."""
    _check_tensors(bool(is_fp4), a, b, a_scale, b_scale, None, M, N, K)
    if out_kind is None:
        out_kind = _out_code(c, None)
    if isinstance(bias, torch.Tensor):
        if not bias.is_cuda or bias.dtype != torch.bfloat16 or not bias.is_contiguous() or bias.numel() != N:
            raise ValueError("bias must be a contiguous bfloat16 CUDA tensor of N elements")
    if isinstance(c, torch.Tensor):
        n = M * N if out_kind in (OUT_BF16, OUT_F16, OUT_F32, OUT_MXFP8) else M * N // 2
        if not c.is_cuda or not c.is_contiguous() or c.numel() != n:
            raise ValueError("c must be a contiguous CUDA tensor of %d elements" % n)
    st = _lib.mx_scaled_mm_fused(int(bool(is_fp4)), _ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale),
                                 _ptr(bias), act, _ptr(c), _ptr(c_scale), M, N, K, out_kind, variant,
                                 _stream(stream))
    if st:
        raise MxGemmError(st, "mx_scaled_mm_fused")


def mx_fused_num_variants() -> int:
    return _lib.mx_fused_num_variants()


def mx_fused_default_variant(is_fp4, M, N, K) -> int:
    return _lib.mx_fused_default_variant(int(bool(is_fp4)), M, N, K)


def mx_fused_variant_max_k(variant, is_fp4) -> int:
    v = _lib.mx_fused_variant_max_k(variant, int(bool(is_fp4)))
    if v < 0:
        raise MxGemmError(v, "mx_fused_variant_max_k")
    return v


def mx_fused_variant_name(variant) -> str | None:
    n = _lib.mx_fused_variant_name(variant)
    return n.decode() if n is not None else None


def mx_dense_gemm(a, b, c, M, N, K, trans_a=0, trans_b=0, dtype=None, out_dtype=None,
                  stream=None) -> None:
    """Dense BF16 / FP16 product C = A B (C ABI mx_dense_gemm): a stored
    [M][K] (trans_a 0) or [K][M] (1), b stored [K][N] (trans_b 0) or [N][K]
    (1); dtype 0 BF16 / 1 FP16 (default: from a's torch dtype)."""
    if dtype is None:
        if not isinstance(a, torch.Tensor):
            raise ValueError("dtype is required when a is a raw pointer")
        dtype = {torch.bfloat16: 0, torch.float16: 1}[a.dtype]
    for name, t, n in (("a", a, M * K), ("b", b, N * K), ("c", c, M * N)):
        if isinstance(t, torch.Tensor):
            if not t.is_cuda or not t.is_contiguous() or t.numel() != n:
                raise ValueError("%s must be a contiguous CUDA tensor of %d elements" % (name, n))
    st = _lib.mx_dense_gemm(dtype, trans_a, trans_b, _ptr(a), _ptr(b), _ptr(c), M, N, K,
                            _out_code(c, out_dtype), _stream(stream))
    if st:
        raise MxGemmError(st, "mx_dense_gemm")


# ------------------------------------------------------------- convenience
_FMT_OF_DTYPE = {}
for _name, _fmt in (("float4_e2m1fn_x2", "fp4"), ("float8_e4m3fn", "fp8")):
    if hasattr(torch, _name):
        _FMT_OF_DTYPE[getattr(torch, _name)] = _fmt


def _nk_storage(t):
    """A 2-D operand given as stored [rows][cols] (contiguous), or as the
    column-major [cols][rows] view of that storage (what F.scaled_mm takes as
    its second operand): the contiguous [rows][cols] tensor."""
    if t.dim() != 2:
        raise ValueError("operands must be 2-D")
    if t.is_contiguous():
        return t
    if t.t().is_contiguous():
        return t.t()
    raise ValueError("operand must be contiguous or the transpose of a contiguous tensor")


def scaled_mm_shapes(a, b, a_scale, b_scale, fmt=None):
    """(fmt, M, N, K, a, b, a_scale, b_scale) of a scaled_mm call with 2-D
    operands: a [M][K/2] (E2M1 pairs) or [M][K] (E4M3) bytes, row-major; b
    [N][K/2] / [N][K] bytes, or its column-major [K/2][N] / [K][N] view; the
    scales [M][K/32] and [N][K/32] (or that one's transpose view).  fmt
    'fp4' / 'fp8', or None to take it from a's dtype."""
    if fmt is None:
        fmt = _FMT_OF_DTYPE.get(a.dtype)
        if fmt is None:
            raise ValueError("fmt is required unless a is float4_e2m1fn_x2 or float8_e4m3fn")
    if fmt not in ("fp4", "fp8"):
        raise ValueError("fmt must be 'fp4' or 'fp8'")
    a, b = _nk_storage(a), _nk_storage(b)
    a_scale, b_scale = _nk_storage(a_scale), _nk_storage(b_scale)
    M, kb = a.shape
    N = b.shape[0]
    K = kb * 2 if fmt == "fp4" else kb
    if b.shape[1] != kb:
        raise ValueError("a and b disagree on K")
    if tuple(a_scale.shape) != (M, K // 32) or tuple(b_scale.shape) != (N, K // 32):
        raise ValueError("scales must be [M][K/32] and [N][K/32]")
    return fmt, int(M), int(N), int(K), a, b, a_scale, b_scale


def scaled_mm(a, b, a_scale, b_scale, fmt=None, M=None, N=None, K=None,
              out_dtype=torch.bfloat16, workspace="auto", stream=None) -> torch.Tensor:
    """C = MX scaled GEMM of packed operands; returns a new [M, N] tensor.

    With M, N and K given, the operands are any 1-byte CUDA tensors (or raw
    pointers) laid out as mx_scaled_mm_fp4 / mx_scaled_mm_fp8 take them and
    fmt ('fp4' or 'fp8') is required.  Without them, the operands are 2-D
    tensors whose shapes give the sizes (scaled_mm_shapes): torch's
    float4_e2m1fn_x2 / float8_e4m3fn codes and float8_e8m0fnu scales, or
    uint8 with fmt, B either stored [N][K] or as F.scaled_mm's column-major
    [K][N] view of that storage."""
    if M is None or N is None or K is None:
        fmt, M, N, K, a, b, a_scale, b_scale = scaled_mm_shapes(a, b, a_scale, b_scale, fmt)
    elif fmt not in ("fp4", "fp8"):
        raise ValueError("fmt must be 'fp4' or 'fp8'")
    dev = a.device if isinstance(a, torch.Tensor) else torch.device("cuda")
    c = torch.empty((M, N), dtype=out_dtype, device=dev)
    fn = mx_scaled_mm_fp4 if fmt == "fp4" else mx_scaled_mm_fp8
    fn(a, b, a_scale, b_scale, c, M, N, K, workspace=workspace, stream=stream)
    return c


def mx_empty_like(is_fp4, M, N, K, stream=None) -> None:
    """Enqueue an empty kernel on the grid the default product would use for
    this shape (C ABI mx_empty_like; measurement of the launch cost)."""
    st = _lib.mx_empty_like(int(bool(is_fp4)), M, N, K, _stream(stream))
    if st:
        raise MxGemmError(st, "mx_empty_like")


def mx_scaled_mm_noalloc(is_fp4, a, b, a_scale, b_scale, c, M, N, K, out_dtype=None, stream=None) -> None:
    """The default product with the library's built-in split-K scratch
    (C ABI mx_scaled_mm_noalloc): no workspace argument and no allocation.
    Calls that may overlap on one GPU race on that scratch."""
    _check_tensors(bool(is_fp4), a, b, a_scale, b_scale, c, M, N, K)
    st = _lib.mx_scaled_mm_noalloc(int(bool(is_fp4)), _ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale),
                                   _ptr(c), M, N, K, _out_code(c, out_dtype), _stream(stream))
    if st:
        raise MxGemmError(st, "mx_scaled_mm_noalloc")


def mx_noalloc_scratch_bytes() -> int:
    return int(_lib.mx_noalloc_scratch_bytes())
