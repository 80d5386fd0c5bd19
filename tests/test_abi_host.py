"""Host-only checks of the C ABI library (no GPU needed).

The library must load and export every function include/mxgemm.h
declares, and every invalid argument must be rejected with its status code
before any HIP call (so these run on a machine without a GPU).
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxgemm.h")
LIB = os.path.join(ROOT, "block_scaled_precision_mm_amd", "libmxgemm.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "mxbuild", os.path.join(ROOT, "block_scaled_precision_mm_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    L = ctypes.CDLL(LIB)
    P, I64, INT, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.mx_scaled_mm_fp4.argtypes = [P, P, P, P, P, I64, I64, I64, INT, P, SZ, P]
    L.mx_scaled_mm_fp8.argtypes = L.mx_scaled_mm_fp4.argtypes
    L.mx_scaled_mm_config.argtypes = [INT, P, P, P, P, P, I64, I64, I64, INT, INT, INT, P, SZ, P]
    L.mx_scaled_mm_workspace_bytes.argtypes = [INT, I64, I64, I64]
    L.mx_scaled_mm_workspace_bytes.restype = SZ
    L.mx_config_workspace_bytes.argtypes = [INT, INT, I64, I64]
    L.mx_config_workspace_bytes.restype = SZ
    L.mx_default_config.argtypes = [INT, I64, I64, I64, INT, ctypes.POINTER(INT)]
    L.mx_status_string.restype = ctypes.c_char_p
    L.mx_variant_name.restype = ctypes.c_char_p
    L.mx_default_variant.argtypes = [INT, I64, I64, I64]
    L.mx_variant_max_k.argtypes = [INT, INT]
    L.mx_variant_max_k.restype = I64
    L.mx_quantize_bf16.argtypes = [P, P, P, I64, I64, INT, P]
    L.mx_grouped_mm_fp4.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, INT, P]
    L.mx_grouped_mm_fp8.argtypes = L.mx_grouped_mm_fp4.argtypes
    L.mx_grouped_mm_config.argtypes = [INT, P, P, P, P, P, P, I64, I64, I64, I64, INT, INT, P]
    L.mx_grouped_variant_name.restype = ctypes.c_char_p
    L.mx_grouped_default_variant.argtypes = [I64, I64, I64]
    L.mx_scaled_mm_fused.argtypes = [INT, P, P, P, P, P, INT, P, P, I64, I64, I64, INT, INT, P]
    L.mx_fused_variant_name.restype = ctypes.c_char_p
    return L


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("mx_scaled_mm_fp4", "mx_scaled_mm_fp8", "mx_scaled_mm_config",
                     "mx_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.mx_abi_version() == 8
    assert lib.mx_num_variants() >= 1
    for v in range(lib.mx_num_variants()):
        assert lib.mx_variant_name(v)
    assert lib.mx_variant_name(lib.mx_num_variants()) is None


def test_binding_names_match_header():
    import importlib
    import sys
    sys.path.insert(0, ROOT)
    pkg = importlib.import_module("block_scaled_precision_mm_amd")
    for name in declared_functions():
        assert name in pkg.EXPORTS and hasattr(pkg, name), name


A = 0x10000   # fake but aligned device addresses: validation never dereferences them


@pytest.mark.parametrize("fn", ["mx_scaled_mm_fp4", "mx_scaled_mm_fp8"])
@pytest.mark.parametrize("args,status", [
    ((0, A, A, A, A, 8, 8, 128, 0), -1),          # null a
    ((A, A, A, 0, A, 8, 8, 128, 0), -1),          # null b_scale
    ((A, A, A, A, 0, 8, 8, 128, 0), -1),          # null c
    ((A, A, A, A, A, 0, 8, 128, 0), -2),          # M = 0
    ((A, A, A, A, A, 8, -1, 128, 0), -2),         # N < 0
    ((A, A, A, A, A, 8, 8, 0, 0), -2),            # K = 0
    ((A, A, A, A, A, 8, 8, 96, 0), -3),           # K % 128 != 0
    ((A, A, A, A, A, 8, 8, 200, 0), -3),
    ((A + 8, A, A, A, A, 8, 8, 128, 0), -4),      # a not 16-byte aligned
    ((A, A, A, A, A + 4, 8, 8, 128, 0), -4),      # c not 16-byte aligned
    ((A, A, A + 2, A, A, 8, 8, 128, 0), -4),      # scale not 4-byte aligned
    ((A, A, A, A, A, 8, 8, 128, 3), -5),          # bad out dtype
    ((A, A, A, A, A, 8, 8, 128, -1), -5),
    ((A, A, A, A, A, 1 << 40, 8, 128, 0), -2),    # M beyond the kernels' index range
    ((A, A, A, A, A, 8, 1 << 31, 128, 0), -2),    # N beyond the kernels' index range
    ((A, A, A, A, A, 8, 8, (1 << 22) + 128, 0), -2),  # K beyond the per-workgroup buffer range
])
def test_invalid_arguments_rejected_before_any_hip_call(lib, fn, args, status):
    rc = getattr(lib, fn)(*args, None, 0, None)
    assert rc == status, (rc, lib.mx_status_string(rc))


@pytest.mark.parametrize("args,status", [
    ((0, A, A, 4, 64, 1), -1),              # null x
    ((A, 0, A, 4, 64, 0), -1),              # null codes
    ((A, A, 0, 4, 64, 1), -1),              # null scales
    ((A, A, A, 0, 64, 1), -2),              # rows = 0
    ((A, A, A, 4, 0, 1), -2),               # K = 0
    ((A, A, A, 1 << 30, 1 << 12, 1), -2),   # rows * K beyond 2^40
    ((A, A, A, 4, 48, 1), -3),              # K % 32 != 0
    ((A + 2, A, A, 4, 64, 1), -4),          # x not 16-byte aligned
    ((A, A + 8, A, 4, 64, 0), -4),          # codes not 16-byte aligned
])
def test_quantize_invalid_arguments(lib, args, status):
    rc = lib.mx_quantize_bf16(*args, None)
    assert rc == status, (rc, lib.mx_status_string(rc))


@pytest.mark.parametrize("fn", ["mx_grouped_mm_fp4", "mx_grouped_mm_fp8"])
@pytest.mark.parametrize("args,status", [
    ((A, A, A, A, A, 0, 4, 64, 8, 128, 0), -1),          # null offs
    ((0, A, A, A, A, A, 4, 64, 8, 128, 0), -1),          # null a
    ((A, A, A, A, A, A, 0, 64, 8, 128, 0), -2),          # no groups
    ((A, A, A, A, A, A, (1 << 16) + 1, 64, 8, 128, 0), -2),   # too many groups
    ((A, A, A, A, A, A, 4, -1, 8, 128, 0), -2),          # M < 0
    ((A, A, A, A, A, A, 4, 64, 0, 128, 0), -2),          # N = 0
    ((A, A, A, A, A, A, 4, 64, 8, 96, 0), -3),           # K % 128
    ((A, A, A, A, A, A, 4, 0, 8, 96, 0), -3),            # M = 0 is still checked
    ((A, A, A, A, A, A + 2, 4, 64, 8, 128, 0), -4),      # offs not 4-byte aligned
    ((A, A, A, A, A + 8, A, 4, 64, 8, 128, 0), -4),      # c not 16-byte aligned
    ((A, A, A, A, A, A, 4, 64, 8, 128, 7), -5),          # bad out dtype
    ((A, A, A, A, A, A, 1 << 16, 64, (1 << 31) - 1, 1 << 22, 0), -2),   # groups*N*K beyond int64
    ((A, A, A, A, A, A, 1 << 16, (1 << 31) - 1, 1 << 16, 128, 0), -2),   # worst-case grid too large
])
def test_grouped_invalid_arguments(lib, fn, args, status):
    rc = getattr(lib, fn)(*args, None)
    assert rc == status, (rc, lib.mx_status_string(rc))


def test_grouped_configs(lib):
    n = lib.mx_grouped_num_variants()
    assert n >= 1
    for v in range(n):
        assert lib.mx_grouped_variant_name(v)
    assert lib.mx_grouped_variant_name(n) is None
    ok = (A, A, A, A, A, A, 4, 64, 64, 512, 0)
    assert lib.mx_grouped_mm_config(1, *ok, -1, None) == -9
    assert lib.mx_grouped_mm_config(0, *ok, n, None) == -9
    # argument errors take precedence over the variant check
    assert lib.mx_grouped_mm_config(1, A, A, A, A, A, 0, 4, 64, 64, 512, 0, 99, None) == -1
    # M = 0 with valid arguments enqueues nothing (no HIP call, so it passes here)
    assert lib.mx_grouped_mm_fp8(A, A, A, A, A, A, 4, 0, 64, 512, 0, None) == 0
    assert lib.mx_grouped_mm_fp8(0, A, 0, A, 0, A, 4, 0, 64, 512, 0, None) == 0
    assert lib.mx_grouped_mm_fp8(0, 0, 0, A, 0, A, 4, 0, 64, 512, 0, None) == -1
    for shape in ((8, 8192, 4096), (32, 256, 2048), (64, 1, 7168), (1, 100000, 128)):
        assert 0 <= lib.mx_grouped_default_variant(*shape) < n
    assert lib.mx_grouped_default_variant(0, 8, 8) == -2


@pytest.mark.parametrize("args,status", [
    ((1, 0, A, A, A, 0, 0, A, 0, 8, 64, 128, 0, -1), -1),     # null a
    ((1, A, A, A, A, 0, 0, A, 0, 8, 64, 96, 0, -1), -3),      # K % 128
    ((1, A, A, A, A, 0, 0, A, 0, 8, 64, 128, 5, -1), -5),     # unknown out kind
    ((1, A, A, A, A, 0, 0, A, 0, 8, 64, 128, -1, -1), -5),
    ((1, A, A, A, A, 0, 4, A, 0, 8, 64, 128, 0, -1), -9),     # unknown activation
    ((1, A, A, A, A, A + 1, 0, A, 0, 8, 64, 128, 0, -1), -4), # odd bias address
    ((1, A, A, A, A, 0, 0, A, 0, 8, 64, 128, 3, -1), -1),     # MX output without c_scale
    ((0, A, A, A, A, 0, 0, A, A, 8, 48, 128, 4, -1), -2),     # MX output, N % 32
    ((0, A, A, A, A, 0, 0, A, A, 8, 64, 128, 0, 99), -9),     # unknown variant
    ((0, A, A, A, A, A, 0, A, A, 8, (1 << 30) + 32, 128, 0, -1), -2),   # bias beyond 2^30 columns
])
def test_fused_invalid_arguments(lib, args, status):
    rc = lib.mx_scaled_mm_fused(*args, None)
    assert rc == status, (rc, lib.mx_status_string(rc))
    n = lib.mx_fused_num_variants()
    assert n >= 1 and lib.mx_fused_variant_name(n) is None and lib.mx_fused_variant_name(0)
    lib.mx_fused_default_variant.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    lib.mx_fused_variant_max_k.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.mx_fused_variant_max_k.restype = ctypes.c_int64
    for is_fp4 in (0, 1):
        for shape in ((1, 4096, 4096), (32, 14336, 4096), (32, 14336, 8192), (64, 64, 128),
                      (256, 28672, 8192), (8192, 8192, 8192)):
            v = lib.mx_fused_default_variant(is_fp4, *shape)
            assert 0 <= v < n
            # the default always accepts the K it was picked for
            assert shape[2] <= lib.mx_fused_variant_max_k(v, is_fp4)
    # wide N at 17-64 rows (outside the E2M1 decode widths): the 64 x 64 four-slot tile
    assert lib.mx_fused_variant_name(lib.mx_fused_default_variant(0, 32, 14336, 4096)) == b"ftile_64x64_r4"
    assert lib.mx_fused_variant_name(lib.mx_fused_default_variant(1, 32, 14336, 4096)) == b"fdecode_32x64_k2"
    assert lib.mx_fused_variant_name(lib.mx_fused_default_variant(0, 32, 4096, 4096)) == b"fstream_2x4_k8"
    assert lib.mx_fused_default_variant(1, 0, 8, 128) == -2
    assert lib.mx_fused_default_variant(1, 8, 8, 0) == -2
    assert lib.mx_fused_variant_max_k(n, 1) == -9
    # a fused variant with a K limit rejects a larger K before touching memory
    for v in range(n):
        km = lib.mx_fused_variant_max_k(v, 1)
        if km < (1 << 22):
            rc = lib.mx_scaled_mm_fused(1, A, A, A, A, 0, 0, A, A, 32, 64, km + 128, 0, v, None)
            assert rc == -9, (v, rc)


@pytest.mark.parametrize("args,status", [
    ((0, 0, 0, 0, A, A, 8, 8, 8, 0), -1),          # null a
    ((2, 0, 0, A, A, A, 8, 8, 8, 0), -5),          # unknown dtype
    ((0, 0, 0, A, A, A, 8, 8, 8, 3), -5),          # unknown out dtype
    ((0, 2, 0, A, A, A, 8, 8, 8, 0), -9),          # trans flag
    ((0, 0, 0, A, A, A, 0, 8, 8, 0), -2),          # M = 0
    ((0, 0, 0, A, A, A, 8, 8, 12, 0), -2),         # a [M][K] rows not 16-byte aligned
    ((0, 1, 0, A, A, A, 12, 8, 8, 0), -2),         # a [K][M] rows not 16-byte aligned
    ((0, 0, 0, A, A, A, 8, 12, 8, 0), -2),         # b [K][N] rows not 16-byte aligned
    ((0, 0, 1, A, A, A, 8, 8, 12, 0), -2),         # b [N][K] (and a) rows
    ((0, 0, 0, A + 2, A, A, 8, 8, 8, 0), -4),      # a not 16-byte aligned
    ((0, 0, 0, A, A, A, 1 << 16, 8, 1 << 14, 0), -2),   # operand beyond 2^30 elements
])
def test_dense_invalid_arguments(lib, args, status):
    lib.mx_dense_gemm.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_void_p]
    rc = lib.mx_dense_gemm(*args, None)
    assert rc == status, (rc, lib.mx_status_string(rc))


def test_invalid_configs(lib):
    ok = (A, A, A, A, A, 64, 64, 512, 0)
    assert lib.mx_scaled_mm_config(1, *ok, -1, 1, None, 0, None) == -9
    assert lib.mx_scaled_mm_config(1, *ok, lib.mx_num_variants(), 1, None, 0, None) == -9
    # a variant that keeps A resident in LDS rejects K beyond its capacity
    for v in range(lib.mx_num_variants()):
        for is4 in (0, 1):
            kmax = lib.mx_variant_max_k(v, is4)
            assert kmax >= 512 and kmax % 128 == 0
            if kmax < (1 << 22):
                args = (A, A, A, A, A, 64, 64, kmax + 128, 0)
                assert lib.mx_scaled_mm_config(is4, *args, v, 1, None, 0, None) == -9
    assert lib.mx_variant_max_k(-1, 1) == -9
    assert lib.mx_variant_max_k(lib.mx_num_variants(), 0) == -9
    # argument errors take precedence over the variant check
    assert lib.mx_scaled_mm_config(1, A, A, A, A, A, 64, 64, 500, 0, 0, 1, None, 0, None) == -3
    assert lib.mx_scaled_mm_config(0, 0, A, A, A, A, 64, 64, 512, 0, 0, 1, None, 0, None) == -1


def _variant(lib, name):
    return next(v for v in range(lib.mx_num_variants()) if lib.mx_variant_name(v).decode() == name)


def test_split_k_configs(lib):
    """Split-K across workgroups: K-part counts, workspace size and errors,
    all decided on the host before any HIP call."""
    tile = _variant(lib, "tile_128x128")
    nosplit = _variant(lib, "decode_32x64_k2")
    M, N, K = 512, 4096, 4096
    args = (A, A, A, A, A, M, N, K, 0)
    # workspace: the fixed region of 16384 counters, then 128 x 2 partial
    # tiles of 128 x 128 FP32
    need = lib.mx_config_workspace_bytes(tile, 2, M, N)
    assert need == 16384 * 4 + 128 * 2 * 128 * 128 * 4
    # split-K only on launches of at most 16384 tiles
    assert lib.mx_config_workspace_bytes(tile, 2, 128 * 128, 128 * 129) == 0
    assert lib.mx_scaled_mm_config(1, A, A, A, A, A, 128 * 128, 128 * 129, K, 0, tile, 2, A, 1 << 40, None) == -9
    assert lib.mx_config_workspace_bytes(tile, 1, M, N) == 0
    assert lib.mx_config_workspace_bytes(tile, 0, M, N) == 0
    assert lib.mx_config_workspace_bytes(-1, 2, M, N) == 0
    # splits > 1 needs a large enough workspace
    assert lib.mx_scaled_mm_config(1, *args, tile, 2, None, 0, None) == -6
    assert lib.mx_scaled_mm_config(1, *args, tile, 2, A, need - 1, None) == -6
    # ... 16-byte aligned
    assert lib.mx_scaled_mm_config(1, *args, tile, 2, A + 8, need, None) == -4
    # part counts out of range: at least 512 K per part, at most 64 parts
    assert lib.mx_scaled_mm_config(1, *args, tile, 0, A, need, None) == -9
    assert lib.mx_scaled_mm_config(1, *args, tile, 9, A, 1 << 40, None) == -9      # 4096 / 512 = 8
    assert lib.mx_scaled_mm_config(1, A, A, A, A, A, M, N, 1 << 16, 0, tile, 65, A, 1 << 40, None) == -9
    # a kernel without split-K rejects splits > 1
    assert lib.mx_scaled_mm_config(1, *args, nosplit, 2, A, 1 << 40, None) == -9
    # the decode kernels (A tile of the whole K in LDS) take no split-K
    dec = _variant(lib, "decode_32x64")
    assert lib.mx_scaled_mm_config(1, A, A, A, A, A, 32, 14336, 4096, 0, dec, 2, A, 1 << 40, None) == -9
    assert lib.mx_config_workspace_bytes(dec, 2, 32, 14336) == 0
    assert lib.mx_scaled_mm_fp4(*args, A + 4, 1 << 30, None) == -4
    # (valid configurations, which get as far as the device check, are
    # exercised by tests/sanitize/abi_driver.c against a build without
    # device code, so that no kernel can ever start on fake pointers)


def test_default_config(lib):
    sp = ctypes.c_int(0)
    for shape in ((1, 4096, 4096), (32, 14336, 4096), (64, 4096, 4096), (512, 4096, 4096),
                  (256, 28672, 8192), (8192, 8192, 8192)):
        for is4 in (0, 1):
            for with_ws in (0, 1):
                v = lib.mx_default_config(is4, *shape, with_ws, ctypes.byref(sp))
                assert 0 <= v < lib.mx_num_variants()
                assert 1 <= sp.value <= 64
                if not with_ws:
                    assert sp.value == 1
            v = lib.mx_default_config(is4, *shape, 1, ctypes.byref(sp))
            need = lib.mx_scaled_mm_workspace_bytes(is4, *shape)
            assert need == lib.mx_config_workspace_bytes(v, sp.value, shape[0], shape[1])
            assert (need > 0) == (sp.value > 1)
            assert lib.mx_default_variant(is4, *shape) == v
    assert lib.mx_default_config(1, 8, 8, 100, 1, None) == -3
    assert lib.mx_scaled_mm_workspace_bytes(1, 8, 8, 100) == 0


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10):
        assert lib.mx_status_string(s) != b"unknown status"
    assert b"128" in lib.mx_status_string(-3)
    assert lib.mx_status_string(-1234) == b"unknown status"


def test_default_variant(lib):
    n = lib.mx_num_variants()
    for shape in ((1, 4096, 4096), (32, 14336, 4096), (64, 4096, 4096), (256, 28672, 8192),
                  (8192, 8192, 8192), (7, 3, 128)):
        for is4 in (0, 1):
            v = lib.mx_default_variant(is4, *shape)
            assert 0 <= v < n, (shape, v)
    assert lib.mx_default_variant(1, 8, 8, 100) == -3
    assert lib.mx_default_variant(1, 0, 8, 128) == -2


# The default choice shape by shape, as decided by the measured sweeps on
# MI355X (the host half of the path: validate, pick, launch).
DEFAULTS = [
    # (is_fp4, M, N, K, variant)
    (1, 32, 14336, 4096, "decode_32x64"),
    (1, 16, 14336, 4096, "decode_16x64"),
    (1, 8, 14336, 4096, "decode_16x64"),
    (1, 1, 14336, 4096, "stream_1x1_k4"),
    (1, 8, 4096, 14336, "stream_1x1_k16"),
    (1, 1, 4096, 14336, "stream_1x1_k16"),
    (1, 1, 14336, 8192, "tile_64x64_r4"),      # long K on wide N: the 64 x 64 tile
    (1, 16, 14336, 10240, "tile_64x64_r4"),
    (1, 32, 14336, 8192, "tile_64x64_r4"),     # K past the decode kernel's LDS-resident A tile
    (1, 32, 25600, 5120, "decode_32x64_k2_long"),
    (1, 16, 14336, 8192, "decode_16x64_k2_long"),
    (1, 128, 4096, 5120, "decode_32x64_k2_long"),
    (0, 32, 14336, 4096, "tile_64x64_r4"),     # E4M3 17-32 rows on wide N: the 64 x 64 tile
    (0, 16, 14336, 8192, "tile_64x64_r4"),     # E4M3 1-16 rows on wide N at K >= 8192
    (0, 8, 14336, 4096, "stream_1x2_k4"),
    (1, 32, 4096, 4096, "stream_2x1_k4"),
    (1, 32, 256, 256, "stream_2x1_k1"),      # one wave per K up to 256 bytes per row
    (1, 8, 256, 1024, "stream_1x1_k1"),      # 1-16 rows: one wave up to K = 1024
    (0, 16, 4096, 512, "stream_1x1_k1"),
    (1, 1, 4096, 2048, "stream_1x1_k2"),     # two up to 2048 (E2M1) / 4096 (E4M3)
    (0, 8, 4096, 4096, "stream_1x1_k2"),
    (1, 8, 4096, 4096, "stream_1x1_k4"),
    (0, 24, 1024, 256, "stream_2x1_k1"),
    (1, 32, 1024, 2048, "stream_2x1_k2"),    # two up to 1024
    (0, 32, 4096, 1024, "stream_2x1_k2"),
    (0, 32, 1024, 2048, "stream_2x1_k4"),
    (0, 64, 4096, 4096, "stream_2x2_k4"),
    (1, 64, 14336, 4096, "tile_64x64_r4"),
    (0, 48, 28672, 4096, "tile_64x64_r4"),
    (1, 128, 4096, 4096, "decode_32x64_k2"),   # narrow N: too few tiles for the tile kernels
    (1, 128, 4096, 14336, "stream_4x2_k8"),      # whole K (with a workspace: 64 x 64 tiles, 2 parts)
    (0, 128, 4096, 4096, "stream_4x2_k8"),
    (1, 256, 4096, 4096, "tile_64x64_r4"),
    (1, 256, 4096, 1024, "tile_64x64_r4"),
    (1, 512, 4096, 4096, "tile_64x64_r4"),       # <= 128 tiles of 128 x 128, K <= 4096
    (0, 512, 2048, 2048, "tile_64x64_r4"),
    (1, 640, 4096, 4096, "tile_128x128_r4"),     # 160 tiles
    (1, 512, 4096, 8192, "tile_128x128_r4"),     # long K: 128 x 128 in two parts with a workspace
    (1, 128, 14336, 4096, "tile_64x64_r4"),      # 112 tiles of 128 x 128
    (1, 128, 25600, 5120, "tile_128x128_r4"),  # no half-empty 256-row tiles; four slots over a long K
    (1, 333, 517, 1152, "tile_64x64_r4"),      # few tiles
    (1, 1100, 2048, 1152, "tile_128x128"),     # > 128 tiles, short K: two slots
    (1, 256, 28672, 8192, "tile_128x256"),
    (0, 256, 28672, 8192, "tile_128x256"),
    (1, 8192, 8192, 8192, "tile_256x256"),
    (1, 512, 25600, 5120, "tile_256x256"),
    (1, 512, 14336, 4096, "tile_128x256"),
]


@pytest.mark.parametrize("is4,M,N,K,name", DEFAULTS, ids=lambda x: str(x))
def test_default_variant_choice(lib, is4, M, N, K, name):
    lib.mx_variant_max_k.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.mx_variant_max_k.restype = ctypes.c_int64
    # without a workspace (with one, split-K may take over: see SPLIT_DEFAULTS)
    sp = ctypes.c_int(0)
    v = lib.mx_default_config(is4, M, N, K, 0, ctypes.byref(sp))
    assert lib.mx_variant_name(v).decode() == name
    assert sp.value == 1
    assert K <= lib.mx_variant_max_k(v, is4)


# With a workspace: split-K across workgroups where it measured faster on
# MI355X (few output tiles over a long K), the whole-K choice elsewhere.
SPLIT_DEFAULTS = [
    # (is_fp4, M, N, K, variant, K parts)
    (1, 512, 4096, 14336, "tile_128x128_r4", 2),
    (1, 512, 4096, 4096, "tile_64x64_r4", 1),
    (1, 128, 4096, 14336, "tile_64x64_r4", 2),
    (0, 128, 4096, 4096, "tile_64x64_r4", 2),
    (0, 128, 4096, 8192, "tile_64x64_r4", 2),
    (1, 32, 4096, 14336, "stream_2x4_k8", 4),
    (1, 32, 4096, 4096, "stream_2x1_k4", 1),
    (1, 32, 14336, 4096, "decode_32x64", 1),
    (0, 64, 4096, 4096, "stream_2x2_k4", 1),
    (1, 256, 28672, 8192, "tile_128x256", 1),
    (1, 8192, 8192, 8192, "tile_256x256", 1),
    (1, 2048, 4096, 14336, "tile_128x256", 1),
]


@pytest.mark.parametrize("is4,M,N,K,name,parts", SPLIT_DEFAULTS, ids=lambda x: str(x))
def test_default_config_with_workspace(lib, is4, M, N, K, name, parts):
    sp = ctypes.c_int(0)
    v = lib.mx_default_config(is4, M, N, K, 1, ctypes.byref(sp))
    assert lib.mx_variant_name(v).decode() == name
    assert sp.value == parts
    assert (lib.mx_scaled_mm_workspace_bytes(is4, M, N, K) > 0) == (parts > 1)


def test_noalloc_argument_checks(lib):
    """The allocation-free entry point validates like the others, before
    any HIP call."""
    P, I64, INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.mx_scaled_mm_noalloc.argtypes = [INT, P, P, P, P, P, I64, I64, I64, INT, P]
    lib.mx_noalloc_scratch_bytes.restype = ctypes.c_size_t
    assert lib.mx_scaled_mm_noalloc(1, A, A, A, A, 0, 8, 8, 128, 0, None) == -1
    assert lib.mx_scaled_mm_noalloc(0, A, A, A, A, A, 8, 8, 100, 0, None) == -3
    assert lib.mx_scaled_mm_noalloc(1, A + 8, A, A, A, A, 8, 8, 128, 0, None) == -4
    assert lib.mx_scaled_mm_noalloc(1, A, A, A, A, A, 8, 8, 128, 9, None) == -5
    # its scratch holds the largest default split-K workspace
    assert lib.mx_noalloc_scratch_bytes() >= lib.mx_scaled_mm_workspace_bytes(1, 512, 4096, 14336) > 0
    assert b"scratch" in lib.mx_status_string(-10)


# The environment overrides of the default path (MXG_CONFIG / MXG_LOG) are
# read once per process, so each setting runs in a child process.  Only
# calls that fail before the device check are made (no GPU is needed, and
# no kernel could start on the fake pointers).
_ENV_PROBE = r"""
import ctypes, json, sys
L = ctypes.CDLL(sys.argv[1])
I64, INT, P, SZ = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
L.mx_default_config.argtypes = [INT, I64, I64, I64, INT, ctypes.POINTER(INT)]
L.mx_scaled_mm_workspace_bytes.argtypes = [INT, I64, I64, I64]
L.mx_scaled_mm_workspace_bytes.restype = SZ
L.mx_config_workspace_bytes.argtypes = [INT, INT, I64, I64]
L.mx_config_workspace_bytes.restype = SZ
L.mx_variant_name.restype = ctypes.c_char_p
L.mx_scaled_mm_fp4.argtypes = [P] * 5 + [I64] * 3 + [INT, P, SZ, P]
sp = INT(0)
out = {}
v = L.mx_default_config(1, 128, 4096, 14336, 1, ctypes.byref(sp))
out["ws"] = [v, sp.value, L.mx_variant_name(v).decode() if v >= 0 else None]
v2 = L.mx_default_config(1, 128, 4096, 14336, 0, ctypes.byref(sp))
out["nows"] = [v2, sp.value]
out["ws_bytes"] = [L.mx_scaled_mm_workspace_bytes(1, 128, 4096, 14336),
                   L.mx_config_workspace_bytes(v, 2, 128, 4096) if v >= 0 else -1]
out["long_k"] = L.mx_default_config(1, 32, 14336, 65536, 1, ctypes.byref(sp))
A = 1 << 20
if sys.argv[2] == "call":
    out["call"] = L.mx_scaled_mm_fp4(A, A, A, A, A, 128, 4096, 14336, 0, None, 0, None)
print(json.dumps(out))
"""


def _env_probe(value, call):
    import json
    import subprocess
    import sys
    env = {k: v for k, v in os.environ.items() if not k.startswith("MXG_")}
    env["MXG_CONFIG"] = value
    r = subprocess.run([sys.executable, "-c", _ENV_PROBE, LIB, "call" if call else "nocall"],
                       env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_env_config_override(lib):
    # a valid override: reported by mx_default_config, sized by
    # mx_scaled_mm_workspace_bytes, and a call short of workspace refused
    out = _env_probe("tile_64x64_r4:2", call=True)
    assert out["ws"][2] == "tile_64x64_r4" and out["ws"][1] == 2
    assert out["nows"] == [out["ws"][0], 1]
    assert out["ws_bytes"][0] == out["ws_bytes"][1] > 0
    assert out["long_k"] == out["ws"][0]           # the 64x64 tile takes any K
    assert out["call"] == -6                       # MXG_ERR_WORKSPACE
    # a variant whose K limit the shape exceeds: MXG_ERR_CONFIG for that shape
    out = _env_probe("decode_32x64", call=False)
    assert out["ws"][0] == -9 and out["long_k"] == -9
    # names no variant / no part count: every call MXG_ERR_CONFIG
    for bad in ("no_such_variant", "tile_128x128:x", "tile_128x128:0", "tile_128x128:65"):
        out = _env_probe(bad, call=True)
        assert out["ws"][0] == -9 and out["nows"][0] == -9 and out["call"] == -9, bad
