"""GPU test of the allocation-free entry point (mx_scaled_mm_noalloc).

Through the C ABI: two calls in a row, the second with a smaller input,
each compared bit for bit with the existing entry point mx_scaled_mm_fp4 /
mx_scaled_mm_fp8 given its own workspace (the same configuration, hence
the same bits) and against the oracle on sampled outputs.  The shapes
include the default split-K configurations (two K parts on the 128 x 128
tile, four on the 32 x 64 stream tile), which use the built-in scratch,
and a whole-K one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mxgen
import oracle
from tests import mxcheck

pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _inputs(fmt, M, N, K, seed):
    a, sa = mxgen.quantize(mxgen.normal_bf16(seed, (M, K)), fmt)
    b, sb = mxgen.quantize(mxgen.normal_bf16(seed + 1, (N, K)), fmt)
    return a, b, sa, sb


def _check(mx, fmt, M, N, K, seed):
    a, b, sa, sb = _inputs(fmt, M, N, K, seed)
    ops = (dev(a), dev(b), dev(sa), dev(sb))
    is4 = fmt == "fp4"
    v, parts = mx.mx_default_config(is4, M, N, K)
    print("noalloc", fmt, M, N, K, mx.mx_variant_name(v), "parts", parts, flush=True)
    for out in (torch.float32, torch.bfloat16):
        got = torch.empty((M, N), dtype=out, device="cuda")
        mx.mx_scaled_mm_noalloc(is4, *ops, got, M, N, K)
        ws = torch.zeros(max(mx.mx_scaled_mm_workspace_bytes(is4, M, N, K), 1), dtype=torch.uint8, device="cuda")
        ref = torch.empty((M, N), dtype=out, device="cuda")
        (mx.mx_scaled_mm_fp4 if is4 else mx.mx_scaled_mm_fp8)(*ops, ref, M, N, K, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16 if out == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if out == torch.bfloat16 else torch.int32)), \
            "noalloc differs from mx_scaled_mm (%s %dx%dx%d %s)" % (fmt, M, N, K, out)
        if out == torch.float32:
            rng = np.random.default_rng(seed)
            ms = np.concatenate([rng.integers(0, M, 2000), [0, M - 1]])
            ns = np.concatenate([rng.integers(0, N, 2000), [N - 1, 0]])
            cref, S = oracle.gemm_at(fmt, a, b, sa, sb, M, N, K, ms, ns)
            mxcheck.check_f32(got.cpu().numpy().astype(np.float64)[ms, ns], cref, S, K, None,
                              "noalloc %s %dx%dx%d" % (fmt, M, N, K))


def test_noalloc_matches_the_workspace_entry_point_twice_smaller_second():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_scaled_precision_mm_amd as mx
    # first the largest default split configuration, then smaller inputs
    _check(mx, "fp4", 512, 4096, 14336, seed=61)      # two K parts, 16.1 MiB of scratch
    _check(mx, "fp4", 32, 4096, 14336, seed=62)       # four K parts, smaller
    _check(mx, "fp4", 20, 1000, 12288, seed=63)       # four K parts, smaller still
    _check(mx, "fp8", 48, 300, 1024, seed=64)         # whole K (no scratch)


def test_noalloc_rejects_nothing_it_should_run():
    import block_scaled_precision_mm_amd as mx
    assert mx.mx_noalloc_scratch_bytes() >= mx.mx_scaled_mm_workspace_bytes(True, 512, 4096, 14336)
