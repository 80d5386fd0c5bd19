// mx_quant.hpp -- MX quantization of BF16 rows along K, gfx950: the step
// before the GEMM ("PyTorch 接上 FlyDSL", 5ulink.com: the support-matrix
// paragraph names BlockWise1x32 E8M0 scales; activations are quantized
// before every MX GEMM in A4W4/A8W8 serving).
//
// Per block of 32 consecutive K values of a row (OCP MX v1.0 conversion):
// scale code s = floor(log2 amax) - emax + 127 clamped to [0, 254]
// (emax 2 for E2M1, 8 for E4M3; 0 for an all-zero block; 0xFF for a block
// holding a NaN or an infinity, whose element codes are then 0); each
// element |x| / 2^(s-127) rounded to the nearest code, ties to even,
// saturating at the largest finite code; the sign bit copied from x.
//
// Bound: HBM.  Per element: 2 bytes read, 0.5 (E2M1) or 1 (E4M3) byte of
// code and 1/32 byte of scale written.  Each 16-byte load instruction of a
// wave reads 1 KB contiguous (lane l: bytes 1024j + 16l of the wave's 4 KB
// tile), so the four lanes 4q..4q+3 hold one 32-value block and combine
// their maxima with two DPP quad permutations; code stores are contiguous
// per instruction too.  The input is read once, so its loads are marked
// nontemporal: on MI355X (8192 x 8192 BF16) that took E2M1 from 31.0 to
// 26.6-27.1 us (6.3 TB/s) and E4M3 from 36.5 to 34.5 us, where a plain
// kernel streaming the same bytes (16 B read, 4 B written per lane) takes
// 29.2 us; more tiles in flight per wave (2 or 4) and other grid sizes were
// slower or equal.
//
// The rounding is done by gfx950's scaled conversions
// (v_cvt_scalef32_pk_fp4_bf16 / v_cvt_scalef32_pk_fp8_bf16: two BF16 values
// to two codes).  Checked on MI355X over every BF16 pattern at scale
// exponents 0, 1, 100, 126, 127, 128, 130 and 254: they divide by 2^(e-127), e being only the exponent
// field of the f32 scale operand (so E8M0 code s passes as the bits s << 23,
// s = 0 included), and round to nearest even exactly, subnormal inputs
// included; E2M1 saturates at 6, but E4M3 turns every overflow into the NaN
// code 0x7F, which is mapped back to 0x7E (448) here.  An ALU version of
// the same rounding (midpoint counting, mantissa rounding on the float
// bits) ran at 43-58% of the HBM roofline, bound by its ~20 VALU
// operations per element; the conversion needs half an instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_common.hpp"

namespace mxg {

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short s16x2v __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));

// two BF16 values packed in a dword, as the conversions take them (by value:
// clang's __builtin_bit_cast of a vector-element lvalue reads element 0)
__device__ __forceinline__ bf16x2v as_bf16x2(unsigned v)
{
    return __builtin_bit_cast(bf16x2v, v);
}

// max over the 4 lanes of a quad (DPP quad permutations 1,0,3,2 and 2,3,0,1)
__device__ __forceinline__ unsigned quad_max(unsigned v)
{
    v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
    return v;
}

// largest BF16 magnitude (bits, sign cleared) among the 8 values of w
__device__ __forceinline__ unsigned amax8(const u4v &w)
{
    u16x2v m = __builtin_bit_cast(u16x2v, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int d = 1; d < 4; ++d)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2v, w[d] & 0x7FFF7FFFu));
    return max((unsigned)m[0], (unsigned)m[1]);
}

// E4M3 bytes whose magnitude is the NaN code 0x7F (an overflow of the
// conversion) become 0x7E, the largest finite code, sign kept
__device__ __forceinline__ unsigned e4m3_saturate(unsigned d)
{
    const unsigned t = d & 0x7F7F7F7Fu;
    return d - (((t + 0x01010101u) & 0x80808080u) >> 7);
}

template <int F>
__global__ __launch_bounds__(256)
void mx_quantize(const uint16_t *x, uint8_t *codes, uint8_t *scales, long long nblocks)
{
    constexpr int EMAX = F == FMT_FP4 ? 2 : 8;
    const int lane = threadIdx.x & 63;
    const long long wave0 = (long long)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    const long long nwaves = (long long)gridDim.x * (blockDim.x / 64);
    const long long ntiles = (nblocks + 63) / 64;        // 64 blocks (4 KB of input) per wave tile
    for (long long tile = wave0; tile < ntiles; tile += nwaves) {
        u4v w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const long long b = tile * 64 + 16 * j + (lane >> 2);    // this lane's block
            w[j] = u4v{0u, 0u, 0u, 0u};
            if (b < nblocks)
                w[j] = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(x + tile * 2048 + 512 * j + 8 * lane));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const long long b = tile * 64 + 16 * j + (lane >> 2);
            // block amax; NaN and Inf patterns are the magnitudes >= 0x7F80
            const unsigned amax = quad_max(amax8(w[j]));
            const bool special = amax >= 0x7F80u;
            // floor(log2 amax) - emax + 127 clamped at 0: the biased exponent
            // field minus emax (a subnormal or zero amax gives 0; the top,
            // 254 - emax, stays below 255)
            const unsigned s = special ? 255u : (unsigned)max((int)(amax >> 7) - EMAX, 0);
            const float sc = __uint_as_float(s << 23);
            if (b < nblocks) {
                if constexpr (F == FMT_FP4) {
                    unsigned d = 0;
                    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, as_bf16x2(w[j][0]), sc, 0);
                    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, as_bf16x2(w[j][1]), sc, 1);
                    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, as_bf16x2(w[j][2]), sc, 2);
                    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, as_bf16x2(w[j][3]), sc, 3);
                    *reinterpret_cast<unsigned *>(codes + tile * 1024 + 256 * j + 4 * lane) = special ? 0u : d;
                } else {
                    u2v d;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        s16x2v o = {0, 0};
                        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, as_bf16x2(w[j][2 * h]), sc, false);
                        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, as_bf16x2(w[j][2 * h + 1]), sc, true);
                        d[h] = special ? 0u : e4m3_saturate(__builtin_bit_cast(unsigned, o));
                    }
                    *reinterpret_cast<u2v *>(codes + tile * 2048 + 512 * j + 8 * lane) = d;
                }
                if ((lane & 3) == 0)
                    scales[b] = (uint8_t)s;
            }
        }
    }
}

}  // namespace mxg
