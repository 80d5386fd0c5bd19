"""GPU parity of the fused-epilogue MX GEMM (mx_scaled_mm_fused, through the
C ABI) against the oracle's product + epilogue reference.

* FP32 output: |y_gpu - y_ref| <= slope * (1e-5 S + tiny) + activation error
  (8 FP32 ulps of |x| + |y|), slope = |act'| bound (1 for none, 1.13 for
  SiLU / tanh-GELU); this is the product's pre-rounding bound carried
  through the activation.
* BF16 / FP16 output: bit-exact RNE of the same variant's FP32 output.
* MX output: bit-exact equal to the oracle's quantizer (oracle.quantize,
  pinned on its own in test_oracle_quant.py) applied to the same variant's
  BF16 output -- the documented definition -- and to mx_quantize_bf16 of
  it; every dequantized element within the MX format's worst rounding /
  saturation step of its block (2 * 2^(s-127) for E2M1, 64 * 2^(s-127) for E4M3) plus the FP32
  bound of y_ref.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mxgen
import oracle
from tests import mxcheck, refdecode

pytestmark = pytest.mark.gpu

ACTS = [0, 1, 2, 3]


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_scaled_precision_mm_amd as mx
    return mx


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def inputs(fmt, M, N, K, seed):
    a, sa = mxgen.quantize(mxgen.normal_bf16(seed, (M, K)), fmt)
    b, sb = mxgen.quantize(mxgen.normal_bf16(seed + 1, (N, K)), fmt)
    bias = torch.tensor(np.random.default_rng(seed + 2).standard_normal(N) * 8, dtype=torch.float32).to(torch.bfloat16)
    return a, b, sa, sb, bias


def fused(mx, fmt, ops, bias, act, M, N, K, out_kind, variant):
    a, b, sa, sb = ops
    if out_kind <= 2:
        dt = {0: torch.bfloat16, 1: torch.float16, 2: torch.float32}[out_kind]
        c = torch.empty((M, N), dtype=dt, device="cuda")
        cs = None
    else:
        c = torch.empty(M * (N if out_kind == 3 else N // 2), dtype=torch.uint8, device="cuda")
        cs = torch.empty(M * (N // 32), dtype=torch.uint8, device="cuda")
    mx.mx_scaled_mm_fused(fmt == "fp4", a, b, sa, sb, bias, act, c, cs, M, N, K, out_kind, variant)
    torch.cuda.synchronize()
    return c, cs


def check_case(mx, fmt, M, N, K, act, with_bias, variant, seed):
    a, b, sa, sb, bias = inputs(fmt, M, N, K, seed)
    bias_bits = bias.view(torch.int16).numpy().view(np.uint16) if with_bias else None
    what = "%s %dx%dx%d act=%d bias=%d v=%s" % (fmt, M, N, K, act, with_bias, mx.mx_fused_variant_name(variant))
    print("fused", what, flush=True)
    cref, S = oracle.gemm(fmt, a, b, sa, sb, M, N, K)
    yref, slope = oracle.epilogue(cref, bias_bits, act)
    ops = (dev(a), dev(b), dev(sa), dev(sb))
    dbias = bias.cuda() if with_bias else None
    # FP32 output against the reference
    c32, _ = fused(mx, fmt, ops, dbias, act, M, N, K, 2, variant)
    y32 = c32.cpu().numpy().astype(np.float64)
    xpre = cref + (bias.double().numpy()[None, :] if with_bias else 0.0)
    tol = slope * mxcheck.pre_tolerance(S, K) + 8 * 2.0 ** -24 * (np.abs(xpre) + np.abs(yref)) + 1e-37
    err = np.abs(y32 - yref)
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d elements over the bound, worst err %g tol %g" % (
        what, bad.sum(), err[bad].max(), tol[bad][np.argmax(err[bad])])
    # BF16 / FP16 output: RNE of the FP32 output, bit for bit
    for kind, rnd in ((0, oracle.round_bf16), (1, oracle.round_f16)):
        c16, _ = fused(mx, fmt, ops, dbias, act, M, N, K, kind, variant)
        bits = c16.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(bits, rnd(y32)), what + " 16-bit output != RNE(FP32 output)"
    if N % 32:
        return
    cb, _ = fused(mx, fmt, ops, dbias, act, M, N, K, 0, variant)
    for kind, qf in ((3, "fp8"), (4, "fp4")):
        codes, scales = fused(mx, fmt, ops, dbias, act, M, N, K, kind, variant)
        qc = torch.empty_like(codes)
        qs = torch.empty_like(scales)
        mx.mx_quantize_bf16(cb, qc, qs, M, N, qf == "fp4")
        torch.cuda.synchronize()
        assert torch.equal(codes, qc) and torch.equal(scales, qs), what + " MX output != quantize(BF16 output)"
        # and the oracle's quantizer of the same BF16 output, bit for bit
        cb_bits = cb.view(torch.int16).cpu().numpy().view(np.uint16)
        oc, osc = oracle.quantize(qf, cb_bits, M, N)
        assert np.array_equal(codes.cpu().numpy().reshape(oc.shape), oc), what + " MX codes != oracle.quantize"
        assert np.array_equal(scales.cpu().numpy().reshape(osc.shape), osc), what + " MX scales != oracle.quantize"
        # dequantized output against the reference
        vals = refdecode.values(qf, codes.cpu().numpy().reshape(M, -1), M, N)
        sc = scales.cpu().numpy().reshape(M, N // 32).astype(np.int64)
        step = np.ldexp(2.0 if qf == "fp4" else 64.0, sc - 127)
        deq = vals * np.repeat(np.ldexp(1.0, sc - 127), 32, axis=1)
        qtol = np.repeat(step, 32, axis=1) + tol + np.abs(yref) * 2.0 ** -8
        qerr = np.abs(deq - yref)
        assert np.all(qerr <= qtol), "%s %s: dequantized output off by %g" % (what, qf, (qerr - qtol).max())


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("act", ACTS)
def test_every_variant_small(mx, fmt, act):
    # ragged M against every tile; N a multiple of 32 (MX output) but not of
    # the wider tiles; K several stages
    for v in range(mx.mx_fused_num_variants()):
        assert 512 <= mx.mx_fused_variant_max_k(v, fmt == "fp4")
        check_case(mx, fmt, 70, 96, 512, act, True, v, seed=11 + act)
    check_case(mx, fmt, 5, 160, 256, act, False, 0, seed=21 + act)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_ragged_n_default(mx, fmt):
    # N not a multiple of 32 (16-bit / FP32 outputs only), default choice
    for M in (3, 40, 300):
        check_case(mx, fmt, M, 200, 384, 2, True, -1, seed=31 + M)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_larger_default(mx, fmt):
    check_case(mx, fmt, 512, 1024, 1024, 3, True, -1, seed=41)
    check_case(mx, fmt, 32, 2048, 2048, 2, True, -1, seed=42)
    # decode widths on wide N: the whole-row decode variants for E2M1
    check_case(mx, fmt, 24, 8192, 1024, 1, True, -1, seed=43)
    check_case(mx, fmt, 9, 8192, 640, 3, False, -1, seed=44)
