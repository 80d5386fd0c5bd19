"""GPU parity of the MX quantizer (mx_quantize_bf16, through the C ABI)
against the oracle's quantizer: integer output, so bit-exact."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_mm_amd as m
    return m


def gpu_quantize(mx, xbits, rows, K, fmt):
    x = torch.from_numpy(np.ascontiguousarray(xbits).view(np.int16)).cuda()
    codes = torch.empty(rows * (K // 2 if fmt == "fp4" else K), dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows * (K // 32), dtype=torch.uint8, device="cuda")
    mx.mx_quantize_bf16(x, codes, scales, rows, K, fmt == "fp4")
    torch.cuda.synchronize()
    return codes.cpu().numpy().reshape(rows, -1), scales.cpu().numpy().reshape(rows, -1)


def check(mx, xbits, rows, K, fmt, what):
    print("quantize", what, fmt, rows, K, flush=True)
    gc, gs = gpu_quantize(mx, xbits, rows, K, fmt)
    oc, os_ = oracle.quantize(fmt, xbits, rows, K)
    assert np.array_equal(gs, os_), "%s %s: scale codes differ at %s" % (what, fmt, np.argwhere(gs != os_)[:5])
    assert np.array_equal(gc, oc), "%s %s: element codes differ at %s" % (what, fmt, np.argwhere(gc != oc)[:5])


def bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (17, 4096), (130, 160), (257, 2048)],
                         ids=lambda s: "%dx%d" % s)
@pytest.mark.parametrize("sigma", [1.0, 1e-36, 1e30])
def test_random_normal(mx, fmt, shape, sigma):
    rows, K = shape
    rng = np.random.default_rng(rows * 7 + K)
    x = (rng.standard_normal((rows, K)) * sigma).astype(np.float32)
    check(mx, bf16_bits(x), rows, K, fmt, "normal sigma=%g" % sigma)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_every_bf16_pattern(mx, fmt):
    # all 65536 bit patterns, 31 per block next to a block maximum that sets
    # the scale (so each pattern is rounded at several scales), plus blocks
    # of the raw patterns themselves (NaN / Inf / subnormal / zero blocks)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rows_raw = pats.reshape(-1, 32)
    blocks = []
    for lead in (0x3F80, 0x4780, 0x3200, 0x0001):   # 1.0, 65536, 2^-27, smallest subnormal
        body = pats.reshape(-1, 31) if pats.size % 31 == 0 else np.resize(pats, (pats.size // 31 + 1) * 31).reshape(-1, 31)
        lead_col = np.full((body.shape[0], 1), lead, np.uint16)
        blocks.append(np.concatenate([lead_col, body], axis=1))
    allb = np.concatenate([rows_raw] + blocks, axis=0)
    rows = allb.shape[0] // 64 * 64
    x = allb[:rows].reshape(rows // 64, 64 * 32)
    check(mx, x, x.shape[0], x.shape[1], fmt, "all bf16 patterns")


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_ties_and_special_values(mx, fmt):
    vals = [0.0, -0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -5.0, 448.0, 440.0, 464.0,
            2.0 ** -6, 2.0 ** -9, 1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9, 7.5 * 2.0 ** -9, 1e-40, 3e38]
    x = np.zeros((8, 64), np.float32)
    x[0, :len(vals)] = vals
    with np.errstate(over="ignore"):
        x[1, :len(vals)] = np.array(vals) * 64      # 3e38 * 64 overflows: an Inf block
    x[2, :len(vals)] = -np.array(vals)
    x[3, 5] = np.inf
    x[4, 40] = np.nan
    x[5, :] = -0.0
    x[6, 33] = -np.inf
    x[7, :] = 6.0
    check(mx, bf16_bits(x), 8, 64, fmt, "ties and specials")


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_quantize_then_gemm(mx, fmt):
    # the quantizer's output feeds the GEMM unchanged (same layout): quantize
    # A and B on the GPU, multiply on the GPU, compare with the oracle GEMM of
    # the same codes
    from tests import mxcheck
    M, N, K = 40, 72, 512
    rng = np.random.default_rng(3)
    xa = bf16_bits(rng.standard_normal((M, K)))
    xb = bf16_bits(rng.standard_normal((N, K)))
    ca, sa = gpu_quantize(mx, xa, M, K, fmt)
    cb, sb = gpu_quantize(mx, xb, N, K, fmt)
    oa, osa = oracle.quantize(fmt, xa, M, K)
    assert np.array_equal(ca, oa) and np.array_equal(sa, osa)
    cref, S = oracle.gemm(fmt, ca, cb, sa, sb, M, N, K)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    fn = mx.mx_scaled_mm_fp4 if fmt == "fp4" else mx.mx_scaled_mm_fp8
    fn(dev(ca), dev(cb), dev(sa), dev(sb), c, M, N, K)
    torch.cuda.synchronize()
    mxcheck.check_f32(c.cpu().numpy().astype(np.float64), cref, S, K, None, "quantize+gemm " + fmt)
