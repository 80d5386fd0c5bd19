"""This library's default MX product beside ATen's on the same operands.

    rocprofv3 --kernel-trace --output-format csv -d DIR -o t -- \\
        python3 -m block_scaled_precision_mm_amd.vs_aten > LOG
    python -m block_scaled_precision_mm_amd.profsum vs-aten DIR LOG

For every shape, ATen's MX scaled GEMM (torch.nn.functional.scaled_mm with
BlockWise1x32 E8M0 scales on both operands, no swizzle, BF16 output) and
mx_scaled_mm_fp4 / mx_scaled_mm_fp8 (the default configuration, with its
split-K workspace) run the same calls on the same operands: R rotated sets
of at least 1 GiB in all, so that both stream from HBM.  Each phase is
bracketed by launches of the library's empty kernel, so that the kernel
trace gives each side's device time per call without host overhead.  The
pages report their kernels' speedup over ATen; this measures the same ratio
for these kernels on one MI355X.

Operands: BF16 N(0,1) rows quantized on the GPU by mx_quantize_bf16 (the
same codes feed both sides).  Before timing, one call of each is compared:
`max_diff_over_max` = max |c_aten - c_lib| / max |c_lib| (summation order
only: at most one BF16 unit in the last place of the largest output).
ATen takes M and N multiples of 32 only, and A scales padded to whole
groups of 16 (MXFP4) or 32 (MXFP8) rows (the padding rows are not read);
the shapes it rejects are listed with its message.
"""
from __future__ import annotations

import json
import math
import sys

import torch
import torch.nn.functional as F

import block_scaled_precision_mm_amd as mx

# the MXFP4 sweep shapes (M x (N, K)), the headline configurations, and the
# same sweep in MXFP8
SWEEP = [(M, N, K) for M in (1, 8, 32, 128, 512, 2048)
         for N, K in ((4096, 4096), (14336, 4096), (4096, 14336), (25600, 5120))]
PLAN = ([("fp4", s) for s in [(32, 256, 256), (32, 14336, 4096), (256, 28672, 8192), (8192, 8192, 8192)]]
        + [("fp8", s) for s in [(64, 4096, 4096), (256, 28672, 8192)]]
        + [("fp4", s) for s in SWEEP] + [("fp8", s) for s in SWEEP])


def _operands(fmt, M, N, K, gen, dev):
    kb = K // 2 if fmt == "fp4" else K
    code = torch.float4_e2m1fn_x2 if fmt == "fp4" else torch.float8_e4m3fn

    def quantized(rows):
        x = torch.randn((rows, K), device=dev, generator=gen).to(torch.bfloat16)
        codes = torch.empty((rows, kb), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev)
        mx.mx_quantize_bf16(x, codes, scales, rows, K, fmt == "fp4")
        return codes.view(code), scales.view(torch.float8_e8m0fnu)

    a, sa = quantized(M)
    b, sb = quantized(N)
    grp = 16 if fmt == "fp4" else 32   # ATen's row padding of the A scales
    mp = (M + grp - 1) // grp * grp
    sa_aten = sa
    if mp != M:
        pad = torch.full((mp - M, K // 32), 127, dtype=torch.uint8, device=dev)
        sa_aten = torch.cat([sa.view(torch.uint8), pad]).view(torch.float8_e8m0fnu)
    return a, b, sa, sb, sa_aten


def _marker():
    mx.mx_empty_like(1, 64, 64, 128)


def run(plan=PLAN):
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20251203)
    for fmt, (M, N, K) in plan:
        kb = K // 2 if fmt == "fp4" else K
        set_bytes = (M + N) * (kb + K // 32) + 2 * M * N
        R = max(1, min(64, math.ceil((1 << 30) / set_bytes)))
        sets = [_operands(fmt, M, N, K, gen, dev) for _ in range(R)]
        outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
        ws_bytes = mx.mx_scaled_mm_workspace_bytes(fmt == "fp4", M, N, K)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        fn = mx.mx_scaled_mm_fp4 if fmt == "fp4" else mx.mx_scaled_mm_fp8
        calls = max(2 * R, 50 if M * N * K >= 2 ** 36 else 200)

        def aten(i):
            a, b, _, sb, sa = sets[i % R]
            return F.scaled_mm(a, b.t(), sa, F.ScalingType.BlockWise1x32, sb, F.ScalingType.BlockWise1x32,
                               swizzle_a=F.SwizzleType.NO_SWIZZLE, swizzle_b=F.SwizzleType.NO_SWIZZLE,
                               output_dtype=torch.bfloat16)

        def lib(i):
            a, b, sa, sb, _ = sets[i % R]
            fn(a, b, sa, sb, outs[i % R], M, N, K, workspace=ws if ws_bytes else None)

        rec = {"fmt": fmt, "M": M, "N": N, "K": K}
        try:
            ca = aten(0)
            torch.cuda.synchronize()
        except Exception as e:   # a shape ATen does not take
            rec["aten_error"] = str(e).splitlines()[0][:200]
            print(json.dumps(rec), flush=True)
            del sets, outs, ws
            continue
        lib(0)
        torch.cuda.synchronize()
        x, y = ca.float(), outs[0].float()
        rec["max_diff_over_max"] = ((x - y).abs().max() / y.abs().max()).item()
        rec.update(R=R, calls=calls)
        del ca, x, y
        for f in (aten, lib):
            for i in range(R + 5):
                f(i)
            torch.cuda.synchronize()
            _marker()
            for i in range(calls):
                f(i)
            _marker()
            torch.cuda.synchronize()
        print(json.dumps(rec), flush=True)
        del sets, outs, ws
        torch.cuda.empty_cache()


if __name__ == "__main__":
    run()
    print("done", flush=True)
    sys.exit(0)
