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
// per instruction too.  Rounding works on the float bits (E4M3) or by
// comparison with the midpoints (E2M1), not by search.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_common.hpp"

namespace mxg {

// floor(log2 m) for a finite non-zero BF16 magnitude m (sign cleared)
__device__ __forceinline__ int bf16_floor_log2(unsigned mag)
{
    const unsigned e = mag >> 7;
    if (e)
        return (int)e - 127;
    return (31 - __builtin_clz(mag)) - 133;   // subnormal: mantissa * 2^-133
}

// E2M1 magnitude code of v >= 0: the count of midpoints v has passed (a
// midpoint that ties goes to the even code: 0.25 -> 0, 0.75 -> 1.0,
// 1.25 -> 1.0, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4); beyond 6 saturates
__device__ __forceinline__ unsigned e2m1_code(float v)
{
    return (unsigned)(v > 0.25f) + (unsigned)(v >= 0.75f) + (unsigned)(v > 1.25f) +
           (unsigned)(v >= 1.75f) + (unsigned)(v > 2.5f) + (unsigned)(v >= 3.5f) +
           (unsigned)(v > 5.0f);
}

// E4M3 (OCP "FN") magnitude code of finite v >= 0, nearest even, saturating
// at 448 (0x7E; 0x7F is NaN)
__device__ __forceinline__ unsigned e4m3_code(float v)
{
    if (v >= 448.0f)
        return 0x7E;
    if (v < 0.015625f)                                   // below 2^-6: steps of 2^-9
        return (unsigned)__builtin_rintf(v * 512.0f);    // 8 = the smallest normal code
    unsigned b = __float_as_uint(v);
    b += 0x7FFFFu + ((b >> 20) & 1u);                   // keep 3 mantissa bits, ties to even
    return (b >> 20) - ((127u - 7u) << 3);               // rebias the exponent 127 -> 7
}

// max / or over the 4 lanes of a quad (DPP quad permutations 1,0,3,2 and 2,3,0,1)
__device__ __forceinline__ unsigned quad_max(unsigned v)
{
    v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
    return v;
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
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const long long b = tile * 64 + 16 * j + (lane >> 2);   // this lane's block
            const bool live = b < nblocks;
            const long long eoff = tile * 2048 + 512 * j + 8 * lane;  // first of its 8 elements
            u4v w = {0u, 0u, 0u, 0u};
            if (live)
                w = *reinterpret_cast<const u4v *>(x + eoff);
            unsigned amax = 0, special = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const unsigned mag = (w[e / 2] >> (16 * (e % 2))) & 0x7FFFu;
                special |= mag >= 0x7F80u;                     // Inf or NaN
                amax = max(amax, mag);
            }
            amax = quad_max(amax);
            special = quad_max(special);
            unsigned s;
            if (special)
                s = 255;
            else if (amax == 0)
                s = 0;
            else
                s = (unsigned)min(max(bf16_floor_log2(amax) - EMAX + 127, 0), 254);
            unsigned q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const unsigned h = (w[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
                const float v = __builtin_ldexpf(__uint_as_float((h & 0x7FFFu) << 16), 127 - (int)s);
                const unsigned mag = special ? 0u : (F == FMT_FP4 ? e2m1_code(v) : e4m3_code(v));
                q[e] = mag | (special ? 0u : (h >> 15) << (F == FMT_FP4 ? 3 : 7));
            }
            if (live) {
                if constexpr (F == FMT_FP4) {
                    unsigned d = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        d |= q[e] << (4 * e);
                    *reinterpret_cast<unsigned *>(codes + tile * 1024 + 256 * j + 4 * lane) = d;
                } else {
                    u2v d;
                    d.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
                    d.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
                    *reinterpret_cast<u2v *>(codes + tile * 2048 + 512 * j + 8 * lane) = d;
                }
                if ((lane & 3) == 0)
                    scales[b] = (uint8_t)s;
            }
        }
    }
}

}  // namespace mxg
