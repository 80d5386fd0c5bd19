// mx_epilogue.hpp -- fused GEMM epilogue: per-column bias, activation and
// optional MX re-quantization of the output, applied to the FP32
// accumulators before they leave the kernel (the roadmap's "GEMM 尾部融合",
// GEMM tail fusion, "PyTorch 接上 FlyDSL", 5ulink.com, closing paragraph).
//
//   y[m][n] = act(acc[m][n] + bias[n])
//
// bias: BF16 [N] or absent; act: none, ReLU, SiLU x / (1 + e^-x), or GELU
// in its tanh form 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), all in
// FP32 (hardware exp2 and reciprocal; see epilogue_value).  The output is y rounded to BF16 / FP16, y in FP32, or -- the MX
// kinds -- y rounded to BF16 and then MX-quantized along N exactly as
// mx_quantize_bf16 does it (so the output is the next GEMM's A operand,
// K' = N): one E8M0 code per 32 consecutive columns from the block amax,
// elements rounded to nearest even, saturating.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_common.hpp"
#include "mx_quant.hpp"

namespace mxg {

enum { ACT_NONE = 0, ACT_RELU = 1, ACT_SILU = 2, ACT_GELU_TANH = 3 };

__device__ __forceinline__ float bf16_to_float(uint16_t h)
{
    return __uint_as_float((unsigned)h << 16);
}

// e^-t as 2^(-t log2 e) on the hardware exp2 (v_exp_f32, about 1 ulp; the
// rounding of the product adds a relative error of about |t| ulps, which
// the activations below scale back down)
__device__ __forceinline__ float exp_neg(float t)
{
    return __builtin_amdgcn_exp2f(-1.4426950408889634f * t);
}

// The activations with the hardware exp2 and reciprocal (v_rcp_f32, 1 ulp):
// a handful of instructions per element, so that the epilogue of a 4-wave
// tile stays short next to its main loop.  Written from the definitions:
//   SiLU(x) = x * 1 / (1 + e^-x)
//   GELU(x) = 0.5 x (1 + tanh u) = x * 1 / (1 + e^-2u),  u = sqrt(2/pi) (x + 0.044715 x^3)
// (1 + tanh u = 2 / (1 + e^-2u)).  For x -> -inf both reach -0 through
// e^-t -> inf and rcp(inf) = 0; NaN stays NaN.
// Branch-free (act is uniform; the selects cost less than control flow in
// an unrolled epilogue, where branches around every element made the
// register allocator spill the 256-accumulator tile).
__device__ __forceinline__ float epilogue_value(float x, int act)
{
    const float relu = x > 0.f ? x : 0.f;
    // SiLU: x * sigmoid(x); tanh-GELU: x * sigmoid(2u)
    const float t = act == ACT_SILU ? x : 1.5957691216057308f * (x + 0.044715f * x * x * x);
    const float gated = x * __builtin_amdgcn_rcpf(1.f + exp_neg(t));
    return act == ACT_NONE ? x : (act == ACT_RELU ? relu : gated);
}

// Bias and activation on four consecutive columns n .. n+3.  The bias is
// read through a buffer over [bias, bias + N) (empty when there is none):
// columns past N, and every column without a bias, read 0 with no branch.
__device__ __forceinline__ v4f epilogue4(v4f v, const GemmArgs &p, int n)
{
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bias, p.bias ? 2 * p.N : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned off = (unsigned)(n + i) * 2u;
        const float b = bf16_to_float(__builtin_amdgcn_raw_buffer_load_b16(rb, off, 0, 0));
        v[i] = epilogue_value(v[i] + b, p.act);
    }
    return v;
}

// Two FP32 values -> two BF16 (round to nearest even) in one dword, low first.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi)
{
    return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)lo) |
           ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)hi) << 16);
}

// E8M0 code of a block from its largest BF16 magnitude (sign cleared), as
// the quantizer chooses it: 0xFF for NaN / Inf, else the biased exponent
// field minus emax, clamped at 0.
template <int F>
__device__ __forceinline__ unsigned block_scale_code(unsigned amax)
{
    constexpr int EMAX = F == FMT_FP4 ? 2 : 8;
    return amax >= 0x7F80u ? 255u : (unsigned)max((int)(amax >> 7) - EMAX, 0);
}

// Codes of the BF16 pairs in w (n pairs) at scale code s; a NaN / Inf block
// gets all-zero codes.  E2M1: one byte per pair; E4M3: two bytes per pair.
template <int F, int NP>
__device__ __forceinline__ void mx_codes(const unsigned (&w)[NP], unsigned s, unsigned (&out)[F == FMT_FP4 ? (NP + 3) / 4 : (NP + 1) / 2])
{
    const float sc = __uint_as_float(s << 23);
    if constexpr (F == FMT_FP4) {
#pragma unroll
        for (int d = 0; d < (NP + 3) / 4; ++d) {
            unsigned v = 0;
            if (0 < NP - 4 * d)
                v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, as_bf16x2(w[4 * d]), sc, 0);
            if (1 < NP - 4 * d)
                v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, as_bf16x2(w[4 * d + 1]), sc, 1);
            if (2 < NP - 4 * d)
                v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, as_bf16x2(w[4 * d + 2]), sc, 2);
            if (3 < NP - 4 * d)
                v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, as_bf16x2(w[4 * d + 3]), sc, 3);
            out[d] = s == 255u ? 0u : v;
        }
    } else {
#pragma unroll
        for (int d = 0; d < (NP + 1) / 2; ++d) {
            s16x2v o = {0, 0};
            o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, as_bf16x2(w[2 * d]), sc, false);
            if (2 * d + 1 < NP)
                o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, as_bf16x2(w[2 * d + 1]), sc, true);
            out[d] = s == 255u ? 0u : e4m3_saturate(__builtin_bit_cast(unsigned, o));
        }
    }
}

// Largest BF16 magnitude of the pairs in w.
template <int NP>
__device__ __forceinline__ unsigned amax_pairs(const unsigned (&w)[NP])
{
    unsigned m = 0;
#pragma unroll
    for (int i = 0; i < NP; ++i)
        m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    return m;
}

}  // namespace mxg
