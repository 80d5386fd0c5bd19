// mx_dense.hpp -- dense BF16 / FP16 GEMM in the four storage layouts, gfx950
// (the torch.mm row of the support matrix of "PyTorch 接上 FlyDSL",
// 5ulink.com: FP16/BF16 inputs, static 2-D shapes, NN / NT / TN / TT).
//
//   C[M][N] = A[M][K] * B[K][N],  FP32 accumulation, BF16 / FP16 / FP32 out
//
// A is stored [M][K] (TA = 0) or [K][M] (TA = 1); B is stored [K][N]
// (TB = 0) or [N][K] (TB = 1).  "NT" -- both operands K-contiguous -- is the
// MFMA's own layout; in the others one or both operands are contiguous
// along M or N and are transposed on their way into LDS.  The library
// runs every layout on the tile kernel instead (mx_tile.hpp, 16-bit
// operands, an operand contiguous along M or N kept in K rows and read with
// transposing LDS reads: 8192^3 in 913-925 us against 1452-2241 here); this
// kernel is the fallback where an operand stored [K][M] / [K][N] is too
// large for the tile kernel's 32-bit offsets.
//
// Instruction.  v_mfma_f32_32x32x16_{bf16,f16}: lane l = 32g + r supplies
// row r of its 32-row operand block with the 8 K values [8g, 8g+8) of the
// 16-deep step; accumulator register 4v+e holds D[8v + 4g + e][r] of
// D = X * Y^T.  B rows are passed as X and A rows as Y, so lane (r, g)
// holds C[m0 + r][n0 + 8v + 4g + e]: runs of four consecutive columns.
//
// Workgroup.  128 x 128 output tile, four waves in 2 x 2 with 64 x 64 each
// (2 x 2 blocks of 32 x 32); 32 K values per stage.  LDS holds both tiles
// K-contiguous ([row][32] + 8 elements of padding, 80-byte rows), double
// buffered; each stage's global loads are issued before the current
// stage's MFMAs and stored to the other buffer after them, one barrier
// per stage.
//   * a K-contiguous operand: four lanes per row read its 64 bytes (16-byte
//     loads) and store them as they are;
//   * an M- or N-contiguous operand: sixteen lanes per K row read its 256
//     bytes; a 4 x 4 transpose of dwords across the four K rows a wave holds
//     (lane swaps between its 16-lane rows) leaves each lane two columns at
//     four consecutive K values, stored as two 8-byte writes into the
//     K-contiguous rows (the transposition).
// Loads go through buffer resources over the whole operand: rows past M /
// N and steps past K read as zeros, so tails need no branches.  Operand
// rows must be 16-byte aligned (the contiguous dimension a multiple of 8)
// and each operand below 2 GiB; the host checks both.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_common.hpp"

namespace mxg {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum { DENSE_BF16 = 0, DENSE_F16 = 1 };

struct DenseArgs {
    const uint16_t *a, *b;
    void *c;
    int M, N, K;
};

template <int T>
__device__ __forceinline__ v16f dense_mfma(const u4v &x, const u4v &y, v16f acc)
{
    if constexpr (T == DENSE_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, x),
                                                       __builtin_bit_cast(bf16x8v, y), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8v, x),
                                                      __builtin_bit_cast(f16x8v, y), acc, 0, 0, 0);
}

struct DenseTile {
    static constexpr int BM = 128, BN = 128, BK = 32;
    static constexpr int LDK = BK + 8;                  // LDS row stride in elements (80 bytes)
    static constexpr int TILE = BM * LDK;               // elements of one operand tile
};

// One operand's tile for stage kt: R rows (the M or N index) x 32 K.
// KC: the operand is K-contiguous in memory (row stride ld = K); else it is
// contiguous along rows (K-row stride ld = rows).  Two 16-byte loads per
// thread either way.
template <bool KC>
struct DenseLoader {
    __amdgpu_buffer_rsrc_t rs;
    int ld, rows, K;
    int r0;          // first row of the tile

    __device__ __forceinline__ void load(u4v (&v)[2], int kt) const
    {
        const int t = threadIdx.x;
        const int k0 = kt * DenseTile::BK;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            unsigned off = kOutOfRange;
            if constexpr (KC) {
                const int row = r0 + t / 4 + 64 * j, k = k0 + 8 * (t % 4);
                if (row < rows && k < K)
                    off = ((unsigned)row * (unsigned)ld + (unsigned)k) * 2u;
            } else {
                const int k = k0 + t / 16 + 16 * j, col = r0 + 8 * (t % 16);
                if (k < K && col < rows)
                    off = ((unsigned)k * (unsigned)ld + (unsigned)col) * 2u;
            }
            v[j] = load16<CPOL_NONE>(rs, off);
        }
    }

    __device__ __forceinline__ void store(uint16_t *s, const u4v (&v)[2]) const
    {
        const int t = threadIdx.x;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (KC) {
                *reinterpret_cast<u4v *>(s + (t / 4 + 64 * j) * DenseTile::LDK + 8 * (t % 4)) = v[j];
            } else {
                // The four 16-lane rows of a wave hold four consecutive K
                // rows (t / 16) of the same 128 columns, lane p of a row
                // columns 8p .. 8p+7, dword d = columns 8p+2d, 8p+2d+1.  A
                // 4 x 4 dword transpose across the rows (two permlane32 and
                // two permlane16 swaps, gfx950) leaves row q with dword q of
                // all four K rows, i.e. columns 8p+2q and 8p+2q+1 at four
                // consecutive K: two 8-byte stores instead of eight 2-byte
                // ones (which all fell on the same two LDS banks).
                const int q = (t >> 4) & 3, p = t & 15, w = t >> 6;
                unsigned x0 = v[j][0], x1 = v[j][1], x2 = v[j][2], x3 = v[j][3];
                const auto a = __builtin_amdgcn_permlane32_swap(x0, x2, false, false);
                const auto b = __builtin_amdgcn_permlane32_swap(x1, x3, false, false);
                const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
                const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
                x0 = c[0];   // x_i: columns 8p+2q, 8p+2q+1 at K row 4w + 16j + i
                x1 = c[1];
                x2 = d[0];
                x3 = d[1];
                const int col = 8 * p + 2 * q, k = 16 * j + 4 * w;
                u2v lo, hi;
                lo.x = (x0 & 0xFFFFu) | (x1 << 16);
                lo.y = (x2 & 0xFFFFu) | (x3 << 16);
                hi.x = (x0 >> 16) | (x1 & 0xFFFF0000u);
                hi.y = (x2 >> 16) | (x3 & 0xFFFF0000u);
                // odd column groups store their odd column first, so that one
                // store instruction covers all eight column residues mod 8
                // (the 80-byte row stride maps a column to its LDS bank
                // group by that residue)
                const bool odd = p & 1;
                *reinterpret_cast<u2v *>(s + (col + odd) * DenseTile::LDK + k) = odd ? hi : lo;
                *reinterpret_cast<u2v *>(s + (col + !odd) * DenseTile::LDK + k) = odd ? lo : hi;
            }
        }
    }
};

template <int T, int TA, int TB, int OUT>
__global__ __launch_bounds__(256) void mx_dense_gemm_kernel(DenseArgs p)
{
    using D = DenseTile;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][D::TILE];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][D::TILE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 31, g = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;
    const int m0 = blockIdx.y * D::BM, n0 = blockIdx.x * D::BN;

    // A is K-contiguous when stored [M][K]; B when stored [N][K]
    DenseLoader<TA == 0> la{make_rsrc(p.a, (unsigned)((size_t)p.M * p.K * 2)), TA == 0 ? p.K : p.M,
                            p.M, p.K, m0};
    DenseLoader<TB == 1> lb{make_rsrc(p.b, (unsigned)((size_t)p.N * p.K * 2)), TB == 1 ? p.K : p.N,
                            p.N, p.K, n0};

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.f;

    const int KT = (p.K + D::BK - 1) / D::BK;
    u4v va[2], vb[2];
    la.load(va, 0);
    lb.load(vb, 0);
    la.store(sA[0], va);
    lb.store(sB[0], vb);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) {
            la.load(va, kt + 1);
            lb.load(vb, kt + 1);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u4v fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fa[i] = *reinterpret_cast<const u4v *>(&sA[cur][(wm * 64 + 32 * i + r) * D::LDK + 16 * ks + 8 * g]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                fb[j] = *reinterpret_cast<const u4v *>(&sB[cur][(wn * 64 + 32 * j + r) * D::LDK + 16 * ks + 8 * g]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = dense_mfma<T>(fb[j], fa[i], acc[i][j]);
        }
        if (more) {
            la.store(sA[cur ^ 1], va);
            lb.store(sB[cur ^ 1], vb);
        }
        __syncthreads();
    }

    const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + wm * 64 + 32 * i + r;
        if (m >= p.M)
            continue;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = n0 + wn * 64 + 32 * j + 8 * v + 4 * g;
                if (n < p.N) {
                    const v4f q = {acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2],
                                   acc[i][j][4 * v + 3]};
                    store4<OUT>(p.c, p.N, m, n, q, vec_ok && n + 3 < p.N);
                }
            }
    }
}

}  // namespace mxg
