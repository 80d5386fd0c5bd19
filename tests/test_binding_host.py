"""Host-only checks of the Python binding's argument marshalling (no GPU):
scaled_mm's reading of 2-D operands (sizes, format from torch's MX dtypes,
B stored [N][K] or given as the column-major [K][N] view that F.scaled_mm
takes), on CPU tensors that never reach the library."""
from __future__ import annotations

import pytest
import torch

import block_scaled_precision_mm_amd as mx


def _ops(fmt, M, N, K, dtypes=True):
    kb = K // 2 if fmt == "fp4" else K
    code = {"fp4": torch.float4_e2m1fn_x2, "fp8": torch.float8_e4m3fn}[fmt] if dtypes else torch.uint8
    scale = torch.float8_e8m0fnu if dtypes else torch.uint8
    a = torch.zeros((M, kb), dtype=torch.uint8).view(code)
    b = torch.zeros((N, kb), dtype=torch.uint8).view(code)
    sa = torch.zeros((M, K // 32), dtype=torch.uint8).view(scale)
    sb = torch.zeros((N, K // 32), dtype=torch.uint8).view(scale)
    return a, b, sa, sb


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_sizes_and_format_from_dtypes(fmt):
    a, b, sa, sb = _ops(fmt, 48, 200, 512)
    f, M, N, K, a2, b2, sa2, sb2 = mx.scaled_mm_shapes(a, b, sa, sb)
    assert (f, M, N, K) == (fmt, 48, 200, 512)
    assert a2 is a and b2 is b and sa2 is sa and sb2 is sb


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_column_major_b_view(fmt):
    # F.scaled_mm's second operand: K x N column-major, i.e. the transpose
    # view of the [N][K] storage; the binding hands the library that storage
    a, b, sa, sb = _ops(fmt, 8, 64, 256)
    f, M, N, K, _, b2, _, sb2 = mx.scaled_mm_shapes(a, b.t(), sa, sb.t())
    assert (M, N, K) == (8, 64, 256)
    assert b2.is_contiguous() and b2.data_ptr() == b.data_ptr() and tuple(b2.shape) == tuple(b.shape)
    assert sb2.data_ptr() == sb.data_ptr() and tuple(sb2.shape) == tuple(sb.shape)


def test_uint8_operands_need_fmt():
    a, b, sa, sb = _ops("fp8", 4, 32, 128, dtypes=False)
    with pytest.raises(ValueError):
        mx.scaled_mm_shapes(a, b, sa, sb)
    assert mx.scaled_mm_shapes(a, b, sa, sb, fmt="fp8")[:4] == ("fp8", 4, 32, 128)
    # the same bytes read as E2M1 pairs hold twice the K
    a4, b4 = a[:, :64].contiguous(), b[:, :64].contiguous()
    assert mx.scaled_mm_shapes(a4, b4, sa, sb, fmt="fp4")[:4] == ("fp4", 4, 32, 128)


def test_inconsistent_shapes_rejected():
    a, b, sa, sb = _ops("fp4", 8, 64, 256)
    with pytest.raises(ValueError):                      # K disagrees
        mx.scaled_mm_shapes(a, b[:, :64].contiguous(), sa, sb)
    with pytest.raises(ValueError):                      # scale columns not K/32
        mx.scaled_mm_shapes(a, b, sa[:, :4].contiguous(), sb)
    with pytest.raises(ValueError):                      # neither layout
        mx.scaled_mm_shapes(a, b[::2], sa, sb)
    with pytest.raises(ValueError):
        mx.scaled_mm_shapes(a, b, sa, sb, fmt="fp6")
