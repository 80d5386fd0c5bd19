"""GPU parity of the grouped (mixture-of-experts) MX GEMM through the C ABI
(mx_grouped_mm_fp4/fp8, mx_grouped_mm_config) against the oracle's grouped
product.  Same tolerance as the plain GEMM; rows no group covers must keep
their previous contents."""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import mxgen
import oracle
from tests import mxcheck

pytestmark = pytest.mark.gpu

OUT = {"f32": torch.float32, "bf16": torch.bfloat16}
SENTINEL = 12345.0


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_scaled_precision_mm_amd as mx
    return mx


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_grouped(mx, fmt, a, b, sa, sb, offs, G, M, N, K, out="f32", variant=None):
    c = torch.full((max(M, 1), N), SENTINEL, dtype=OUT[out], device="cuda")[:M]
    args = (dev(a), dev(b), dev(sa), dev(sb), c, dev(np.asarray(offs, np.int32)), G, M, N, K)
    if variant is None:
        (mx.mx_grouped_mm_fp4 if fmt == "fp4" else mx.mx_grouped_mm_fp8)(*args)
    else:
        mx.mx_grouped_mm_config(fmt == "fp4", *args, variant)
    torch.cuda.synchronize()
    if out == "f32":
        return c.cpu().numpy().astype(np.float64)
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


def inputs(fmt, sizes, N, K, seed):
    G, M = len(sizes), int(sum(sizes))
    xa = mxgen.normal_bf16(seed, (max(M, 1), K))[:M]
    xb = mxgen.normal_bf16(seed + 1, (G * N, K))
    a, sa = mxgen.quantize(xa, fmt)
    b, sb = mxgen.quantize(xb, fmt)
    return a, b, sa, sb, np.cumsum(sizes).astype(np.int32), G, M


def check(mx, fmt, a, b, sa, sb, offs, G, M, N, K, variant=None, what=""):
    cref, S, cov = oracle.grouped_gemm(fmt, a, b, sa, sb, offs, G, M, N, K)
    c32 = run_grouped(mx, fmt, a, b, sa, sb, offs, G, M, N, K, "f32", variant)
    assert np.all(c32[~cov] == SENTINEL), what + ": a row outside every group was written"
    # MXFP8: elements outside the strict bound must meet it around the E4M3
    # instruction's own value (tests/mxcheck.py), group by group
    model = None
    if fmt == "fp8" and cov.any():
        rows = np.flatnonzero(cov)
        gm = mxcheck.GroupedE4M3RunModel(a, b, sa, sb, offs, G, M, N, K)
        model = lambda ms, ns: gm(rows[ms], ns)
    if cov.any():
        mxcheck.check_f32(c32[cov], cref[cov], S[cov], K, model, what)
    bits = run_grouped(mx, fmt, a, b, sa, sb, offs, G, M, N, K, "bf16", variant)
    if cov.any():
        mxcheck.check_rounded(bits[cov], cref[cov], S[cov], K, "bf16", model, what + " bf16")
        assert np.array_equal(bits[cov], oracle.round_bf16(c32[cov])), what + " bf16 != RNE(f32)"
    sent = np.uint16(torch.tensor([SENTINEL], dtype=torch.bfloat16).view(torch.int16).item() & 0xFFFF)
    assert np.all(bits[~cov] == sent), what + ": bf16 row outside every group was written"


# ragged groups with empty ones, against every tile size: a group of one row,
# groups spanning several M tiles with ragged tails, empty groups at the
# start, in the middle and at the end
SIZES = [[0, 5, 17, 0, 33, 1, 70, 0], [300, 0, 257, 64], [1], [0, 0, 9]]


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("si", range(len(SIZES)))
def test_ragged_groups_every_variant(mx, fmt, si):
    sizes = SIZES[si]
    N, K = 200, 384
    a, b, sa, sb, offs, G, M = inputs(fmt, sizes, N, K, seed=400 + si)
    print("grouped", fmt, sizes, N, K, flush=True)
    for v in range(mx.mx_grouped_num_variants()):
        check(mx, fmt, a, b, sa, sb, offs, G, M, N, K, v,
              "%s sizes=%s %s" % (fmt, sizes, mx.mx_grouped_variant_name(v)))


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_default_variant_and_random_codes(mx, fmt):
    # every element code, scales over 2^+-14, 13 groups (two chunks of the
    # lookup need not be exercised: 64 groups per chunk) -- plus 70 groups,
    # which does cross a chunk
    for G in (13, 70):
        rng = np.random.default_rng(G)
        sizes = rng.integers(0, 12, G)
        sizes[rng.integers(0, G, 3)] = 0
        M, N, K = int(sizes.sum()), 72, 256
        a, sa = mxgen.random_codes(500 + G, fmt, M, K, 113, 141)
        b, sb = mxgen.random_codes(600 + G, fmt, G * N, K, 113, 141)
        offs = np.cumsum(sizes).astype(np.int32)
        print("grouped random", fmt, G, M, flush=True)
        check(mx, fmt, a, b, sa, sb, offs, G, M, N, K, None, "%s random codes G=%d" % (fmt, G))


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_irregular_offsets(mx, fmt):
    # decreasing entries, negative entries, ends past M and rows past the
    # last end: the documented clamping, the same in the oracle
    N, K, M = 64, 256, 90
    G = 6
    a, sa = mxgen.random_codes(71, fmt, M, K)
    b, sb = mxgen.random_codes(72, fmt, G * N, K)
    for offs in ([10, 4, 40, -3, 70, 80], [-1, 0, 30, 200, 5, 1000], [0, 0, 0, 0, 0, 0]):
        offs = np.array(offs, np.int32)
        print("grouped offs", fmt, list(offs), flush=True)
        for v in range(mx.mx_grouped_num_variants()):
            check(mx, fmt, a, b, sa, sb, offs, G, M, N, K, v, "%s offs=%s v%d" % (fmt, list(offs), v))


def test_zero_rows_is_a_noop(mx):
    c = torch.full((1, 8), SENTINEL, device="cuda")
    one = torch.zeros(64, dtype=torch.uint8, device="cuda")
    offs = torch.zeros(2, dtype=torch.int32, device="cuda")
    mx.mx_grouped_mm_fp4(one[:0], torch.zeros(2 * 8 * 64, dtype=torch.uint8, device="cuda"), one[:0],
                         torch.zeros(2 * 8 * 4, dtype=torch.uint8, device="cuda"), c[:0], offs, 2, 0, 8, 128)
    torch.cuda.synchronize()
    assert torch.all(c == SENTINEL)


@functools.lru_cache(maxsize=1)
def _gcase(name):
    return mxgen.grouped_case(name)


@pytest.mark.parametrize("name", list(mxgen.GROUPED))
def test_grouped_workload_sampled_oracle(mx, name):
    cs = _gcase(name)
    print("grouped workload", name, cs.recipe, flush=True)
    rng = np.random.default_rng(len(name))
    ms = np.concatenate([rng.integers(0, cs.M, 3000), cs.offs[cs.sizes > 0] - 1, [0]])
    ns = np.concatenate([rng.integers(0, cs.N, 3000), np.zeros(int((cs.sizes > 0).sum()), np.int64), [cs.N - 1]])
    cref = np.empty(ms.size)
    S = np.empty(ms.size)
    bg = cs.b.reshape(cs.G, cs.N, -1)
    sbg = cs.sb.reshape(cs.G, cs.N, -1)
    for g, (r0, r1) in enumerate(oracle.group_rows(cs.offs, cs.G, cs.M)):
        sel = (ms >= r0) & (ms < r1)
        if sel.any():
            cref[sel], S[sel] = oracle.gemm_at(cs.fmt, cs.a[r0:r1], bg[g], cs.sa[r0:r1], sbg[g],
                                               r1 - r0, cs.N, cs.K, ms[sel] - r0, ns[sel])
    da, db, dsa, dsb, doffs = dev(cs.a), dev(cs.b), dev(cs.sa), dev(cs.sb), dev(cs.offs)
    fn = mx.mx_grouped_mm_fp4 if cs.fmt == "fp4" else mx.mx_grouped_mm_fp8
    c = torch.empty((cs.M, cs.N), dtype=torch.float32, device="cuda")
    fn(da, db, dsa, dsb, c, doffs, cs.G, cs.M, cs.N, cs.K)
    cb = torch.empty((cs.M, cs.N), dtype=torch.bfloat16, device="cuda")
    fn(da, db, dsa, dsb, cb, doffs, cs.G, cs.M, cs.N, cs.K)
    torch.cuda.synchronize()
    c32 = c.cpu().numpy().astype(np.float64)
    bits = cb.view(torch.int16).cpu().numpy().view(np.uint16)
    # quantized N(0,1) inputs: the strict bound, no hardware term
    relmax, _ = mxcheck.check_f32(c32[ms, ns], cref, S, cs.K, None, name)
    mxcheck.check_rounded(bits[ms, ns], cref, S, cs.K, "bf16", None, name)
    assert np.array_equal(bits, oracle.round_bf16(c32))
    print(name, "max err/S %.3e" % relmax, flush=True)
