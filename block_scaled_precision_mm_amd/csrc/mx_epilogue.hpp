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

// Output of a workgroup tile reduced in LDS (the decode-width kernels).
// Thread tid of nthr takes the groups of four consecutive columns q = tid,
// tid + nthr, ... of a ROWS x 4*CG tile, in row-major group order (row =
// q / CG, column group c4 = q % CG), whose FP32 values quad(row, c4)
// returns; with EPI it applies bias and activation, then writes output kind
// OUT at C[m0 + row][n0 + 4*c4 ..]:
//   * BF16 / FP16 / FP32: one bounds-checked store per group;
//   * MX kinds: the eight consecutive groups of a row's 32-column block
//     share its amax over three lane exchanges.  N % 32 == 0 and CG % 8 == 0,
//     so a block lies wholly inside or outside C; nthr and ROWS * CG are
//     multiples of 64, so whole waves take part in the exchanges.
template <int OUT, int EPI, int ROWS, int CG, class Quad>
__device__ __forceinline__ void store_reduced_tile(const GemmArgs &p, int m0, int n0, int tid, int nthr,
                                                   Quad &&quad)
{
    constexpr int NQ = ROWS * CG;
    if constexpr (OUT == OUT_MX8 || OUT == OUT_MX4) {
        static_assert(CG % 8 == 0 && NQ % 64 == 0, "MX output needs whole 32-column blocks and whole waves");
        constexpr int QF = OUT == OUT_MX4 ? FMT_FP4 : FMT_FP8;
        const int wave0 = tid & ~63;
        for (int q0 = 0; q0 < NQ; q0 += nthr) {
            if (q0 + wave0 >= NQ)          // NQ is a multiple of 64: wave-uniform
                break;
            const int q = q0 + tid;
            const int row = q / CG, c4 = q % CG;
            const int m = m0 + row, n = n0 + 4 * c4;
            const v4f sum = epilogue4(quad(row, c4), p, n);
            const unsigned w2[2] = {pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
            unsigned amax = amax_pairs(w2);
            amax = max(amax, (unsigned)__shfl_xor((int)amax, 1, 64));
            amax = max(amax, (unsigned)__shfl_xor((int)amax, 2, 64));
            amax = max(amax, (unsigned)__shfl_xor((int)amax, 4, 64));
            const unsigned sc = block_scale_code<QF>(amax);
            unsigned code[1];
            mx_codes<QF, 2>(w2, sc, code);
            if (m < p.M && n < p.N) {
                uint8_t *c8 = static_cast<uint8_t *>(p.c);
                if constexpr (QF == FMT_FP4)
                    *reinterpret_cast<uint16_t *>(c8 + (size_t)m * (p.N / 2) + n / 2) = (uint16_t)code[0];
                else
                    *reinterpret_cast<unsigned *>(c8 + (size_t)m * p.N + n) = code[0];
                if ((c4 & 7) == 0)
                    p.c_scale[(size_t)m * (p.N / 32) + n / 32] = (uint8_t)sc;
            }
        }
    } else {
        const bool vec_ok = (p.N & 3) == 0;
        for (int q = tid; q < NQ; q += nthr) {
            const int row = q / CG, c4 = q % CG;
            const int m = m0 + row, n = n0 + 4 * c4;
            v4f sum = quad(row, c4);
            if constexpr (EPI)
                sum = epilogue4(sum, p, n);
            if (m < p.M && n < p.N)
                store4<OUT>(p.c, p.N, m, n, sum, vec_ok && n + 3 < p.N);
        }
    }
}

}  // namespace mxg
