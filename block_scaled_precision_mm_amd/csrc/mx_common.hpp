// mx_common.hpp -- pieces shared by the gfx950 NT MX block-scaled GEMM
// kernels: operand formats, the scaled-MFMA wrapper, buffer resources and
// the output conversion.
//
// The operation ("PyTorch 接上 FlyDSL", 5ulink.com, support-matrix row
// "MXFP 缩放 GEMM" and the paragraph under it): C = A * B^T over packed
// MXFP4 (E2M1) or MXFP8 (E4M3) operands, A row-major and B column-major (so
// both are K-contiguous rows), one E8M0 scale per 32 consecutive K values,
// FP32 accumulation, BF16/FP16 output.
//
// The instruction.  v_mfma_scale_f32_16x16x128_f8f6f4 multiplies a 16x128
// tile by a 128x16 tile into a 16x16 FP32 accumulator, decoding the packed
// elements and applying one E8M0 scale per 32-element block on the way.
// Its lane layout on gfx950 (lane l = 16*g + r, r = l & 15, g = l >> 4;
// the 128 K values of one instruction are one "step"):
//   * each lane supplies row r of its operand tile;
//   * FP4: the lane's 16 bytes are K [32g, 32g+32) of the step -- exactly
//     one MX block;
//   * FP8: the lane's 32 bytes are K [16g, 16g+16) followed by
//     K [64+16g, 64+16g+16) of the step;
//   * the scale operand of lane 16*b + r is the E8M0 code of block b
//     (K [32b, 32b+32)) of row r, taken from the byte of the lane's 32-bit
//     scale register that the instruction's scale op_sel names (byte 0
//     here: each lane shifts its row's step dword by 8*g).
//   * accumulator: lane (r, g) holds D[4g + i][r], i = 0..3.
// The kernels pass B rows as the instruction's first operand and A rows as
// the second, so lane (r, g) of an accumulator tile holds
//   C[m0 + r][n0 + 4g + i], i = 0..3
// -- four consecutive output columns of one row, one 8-byte store in BF16.
//
// Operand bytes of one row (FP4 two codes per byte, even k in the low
// nibble; FP8 one code per byte) are read straight from global memory in the
// instruction's layout: in one load the four lanes of a row read 64
// contiguous bytes.  Scale bytes of a row are contiguous too: the 4 codes of
// one step form one dword, the 16 codes of four steps one 16-byte load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));

enum { FMT_FP8 = 0, FMT_FP4 = 1 };
// Unscaled 16-bit operands (the dense product on the tile kernel)
enum { FMT_BF16 = 2, FMT_F16 = 3 };
// Output kinds.  OUT_MX8 / OUT_MX4 (fused epilogue only): the BF16-rounded
// result MX-quantized along N (E4M3 / E2M1 codes + one E8M0 per 32 columns).
enum { OUT_BF16 = 0, OUT_F16 = 1, OUT_F32 = 2, OUT_MX8 = 3, OUT_MX4 = 4 };

template <int F> struct FmtTraits;
template <> struct FmtTraits<FMT_FP8> {
    static constexpr int step_bytes = 128;  // bytes of one 128-deep K step per row
    static constexpr int nvec = 2;          // 16-byte pieces per lane per step
    static constexpr int mfma_code = 0;     // instruction format code for E4M3
    static constexpr bool scaled = true;    // E8M0 codes per 32 K values
};
template <> struct FmtTraits<FMT_FP4> {
    static constexpr int step_bytes = 64;
    static constexpr int nvec = 1;
    static constexpr int mfma_code = 4;     // instruction format code for E2M1
    static constexpr bool scaled = true;
};
template <> struct FmtTraits<FMT_BF16> {
    static constexpr int step_bytes = 256;
    static constexpr int nvec = 1;
    static constexpr bool scaled = false;
};
template <> struct FmtTraits<FMT_F16> {
    static constexpr int step_bytes = 256;
    static constexpr int nvec = 1;
    static constexpr bool scaled = false;
};

// Kernel arguments shared by every kernel family.
struct GemmArgs {
    const uint8_t *a, *b, *sa, *sb;
    void *c;
    int M, N;
    int nsteps;           // 128-K steps this workgroup multiplies over: K / 128, or its K part's
    unsigned row_bytes;   // row stride of the packed operands: K/2 (FP4) or K (FP8) bytes
    unsigned srow_bytes;  // row stride of the scales: K/32 bytes
    unsigned kbytes;      // packed bytes per row in this workgroup's K range (row_bytes without split-K)
    // split-K across workgroups (mx_splitk.hpp): number of K parts
    // (gridDim.z), FP32 partial tiles and per-tile arrival counters
    int splits;
    float *ws;
    unsigned *flags;
    // grouped products only (mx_group.hpp): end offset of each group's rows
    // of A and C, and the group count; B and its scales hold one [N][K]
    // operand per group
    const int *offs;
    int groups;
    // fused epilogue only (mx_epilogue.hpp): per-column BF16 bias or null,
    // activation code, and the E8M0 scale output of the MX output kinds
    const uint16_t *bias;
    int act;
    uint8_t *c_scale;
};

// Cache-policy bits of a buffer load on gfx950: 2 = non-temporal (stream).
enum { CPOL_NONE = 0, CPOL_NT = 2 };

// An offset no valid buffer range reaches: a load from it returns zeros and
// issues no memory traffic (ranges are limited to < 2^31 bytes on the host).
constexpr unsigned kOutOfRange = 0x80000000u;

// Raw buffer over [base, base + bytes).  Word 3 = 0x00020000 is the plain
// 32-bit-format descriptor of the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <int CPOL>
__device__ __forceinline__ u4v load16(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL);
}

__device__ __forceinline__ unsigned load4(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// One step's fragment of one 16-row operand tile: the lane's packed bytes.
template <int F>
struct StepFrag {
    u4v d[FmtTraits<F>::nvec];
};

// Load lane (r, g)'s bytes of step `step` from a row that starts at byte
// `row_off` of the buffer.
template <int F, int CPOL>
__device__ __forceinline__ void load_step(StepFrag<F> &f, __amdgpu_buffer_rsrc_t r,
                                          unsigned row_off, int step, int g)
{
    const unsigned off = row_off + (unsigned)step * FmtTraits<F>::step_bytes + 16u * g;
#pragma unroll
    for (int v = 0; v < FmtTraits<F>::nvec; ++v)
        f.d[v] = load16<CPOL>(r, off + 64u * v);
}

// acc += B_tile(step) x A_tile(step)^T with the E8M0 codes in byte 0 of
// sb / sa (lane g already shifted its row's step dword by 8*g).
template <int F>
__device__ __forceinline__ v4f mfma(const StepFrag<F> &fb, unsigned sb, const StepFrag<F> &fa,
                                    unsigned sa, v4f acc)
{
    v8i x, y;
    if constexpr (F == FMT_FP4) {
        x = v8i{(int)fb.d[0].x, (int)fb.d[0].y, (int)fb.d[0].z, (int)fb.d[0].w, 0, 0, 0, 0};
        y = v8i{(int)fa.d[0].x, (int)fa.d[0].y, (int)fa.d[0].z, (int)fa.d[0].w, 0, 0, 0, 0};
    } else {
        x = v8i{(int)fb.d[0].x, (int)fb.d[0].y, (int)fb.d[0].z, (int)fb.d[0].w,
                (int)fb.d[1].x, (int)fb.d[1].y, (int)fb.d[1].z, (int)fb.d[1].w};
        y = v8i{(int)fa.d[0].x, (int)fa.d[0].y, (int)fa.d[0].z, (int)fa.d[0].w,
                (int)fa.d[1].x, (int)fa.d[1].y, (int)fa.d[1].z, (int)fa.d[1].w};
    }
    constexpr int c = FmtTraits<F>::mfma_code;
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc, c, c, 0, (int)sb, 0,
                                                            (int)sa);
}

// Store 4 consecutive columns n..n+3 of row m: one vector store when `full`
// (n+3 < N and N % 4 == 0, so the address is aligned), else element-wise
// with bounds checks.  BF16/FP16 conversion rounds to nearest even.
template <int OUT>
__device__ __forceinline__ void store4(void *c, int N, int m, int n, v4f v, bool full)
{
    if constexpr (OUT == OUT_F32) {
        float *p = reinterpret_cast<float *>(c) + (size_t)m * N + n;
        if (full) {
            *reinterpret_cast<v4f *>(p) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < N) p[i] = v[i];
        }
    } else {
        unsigned short h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (OUT == OUT_BF16)
                h[i] = __builtin_bit_cast(unsigned short, (__bf16)v[i]);
            else
                h[i] = __builtin_bit_cast(unsigned short, (_Float16)v[i]);
        }
        unsigned short *p = reinterpret_cast<unsigned short *>(c) + (size_t)m * N + n;
        if (full) {
            u2v w;
            w.x = (unsigned)h[0] | ((unsigned)h[1] << 16);
            w.y = (unsigned)h[2] | ((unsigned)h[3] << 16);
            *reinterpret_cast<u2v *>(p) = w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < N) p[i] = h[i];
        }
    }
}

}  // namespace mxg
