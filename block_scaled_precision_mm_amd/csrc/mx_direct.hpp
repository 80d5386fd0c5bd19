// mx_direct.hpp -- register-streaming NT MX block-scaled GEMM kernels for
// gfx950 (CDNA4), built on the scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4.
//
// What is computed ("PyTorch 接上 FlyDSL", 5ulink.com, support-matrix row
// "MXFP 缩放 GEMM" and the paragraph under it): C = A * B^T over packed
// MXFP4 (E2M1) or MXFP8 (E4M3) operands with one E8M0 scale per 32
// consecutive K values, FP32 accumulation, BF16/FP16 output.
//
// Operand delivery.  One scaled MFMA consumes a 128-deep K step of a 16-row
// tile of each operand.  Lane l = 16*g + r (r = l & 15, g = l >> 4) supplies
// row r, and the instruction's own lane layout (measured on gfx950) is:
//   FP4: 16 bytes = K [32g, 32g+32) of the step, i.e. exactly one MX block;
//   FP8: 32 bytes; bytes 0..15 = K [16g, 16g+16), bytes 16..31 =
//        K [64+16g, 64+16g+16) of the step.
// The E8M0 operand of lane 16*b + r scales block b (K [32b, 32b+32)) of row
// r in both cases, so lane g's scale is byte g of the step's 4 scale bytes.
// Each lane therefore reads 16 bytes (FP4) or two 16-byte pieces (FP8) of
// its own row per step, and one dword of scales that it shifts by 8*g.  In
// one load instruction the 4 lanes of a row read 64 contiguous bytes.
//
// The operands are swapped in the instruction (B rows feed the "A" side) so
// that the accumulator lane layout gives each lane 4 consecutive output
// columns of one row: lane (r, g) of tile (x, y) holds
//   C[m0 + 16x + r][n0 + 16y + 4g + i], i = 0..3,
// which is one 8-byte store in BF16/FP16.
//
// Pipelining: a ring of D steps of fragments lives in VGPRs; the loads for
// step s+D are issued as soon as step s's MFMAs have been issued, so D
// steps of loads are in flight per wave.  B is streamed with non-temporal
// loads (read once); A is re-read by every column tile and stays in L2.
//
// Split-K: with S > 1, split z covers K steps [z*T/S, (z+1)*T/S); each
// workgroup writes an FP32 partial tile to the workspace, and the last
// workgroup to finish a tile (per-tile arrival counter) sums the S partials
// in split order 0..S-1 -- a fixed order, so results are deterministic --
// converts them and resets the counter to zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));

enum { FMT_FP8 = 0, FMT_FP4 = 1 };
enum { OUT_BF16 = 0, OUT_F16 = 1, OUT_F32 = 2 };

template <int F> struct FmtTraits;
template <> struct FmtTraits<FMT_FP8> {
    static constexpr int step_bytes = 128;  // bytes of one 128-deep K step per row
    static constexpr int nvec = 2;          // 16-byte pieces per lane per step
    static constexpr int mfma_code = 0;     // instruction format code for E4M3
};
template <> struct FmtTraits<FMT_FP4> {
    static constexpr int step_bytes = 64;
    static constexpr int nvec = 1;
    static constexpr int mfma_code = 4;     // instruction format code for E2M1
};

struct GemmArgs {
    const uint8_t *a, *b, *sa, *sb;
    void *c;
    int M, N;
    int ksteps;        // K / 128
    int splits;        // S >= 1
    float *part;       // S * M * N floats (split-K only)
    unsigned *cnt;     // one counter per workgroup tile (split-K only)
};

template <int F>
struct Frag {
    u4v d[FmtTraits<F>::nvec];
    unsigned s;
};

template <int F, bool NT>
__device__ __forceinline__ void load_frag(Frag<F> &f, const uint8_t *row, const uint8_t *srow,
                                          int step, int g)
{
    constexpr int SB = FmtTraits<F>::step_bytes;
    const uint8_t *p = row + (size_t)step * SB + 16 * g;
#pragma unroll
    for (int v = 0; v < FmtTraits<F>::nvec; ++v) {
        const u4v *q = reinterpret_cast<const u4v *>(p + 64 * v);
        if constexpr (NT)
            f.d[v] = __builtin_nontemporal_load(q);
        else
            f.d[v] = *q;
    }
    unsigned w = *reinterpret_cast<const unsigned *>(srow + 4 * step);
    f.s = w >> (8 * g);
}

template <int F>
__device__ __forceinline__ v4f mfma_step(const Frag<F> &fb, const Frag<F> &fa, v4f acc)
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
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc, c, c, 0, (int)fb.s, 0,
                                                            (int)fa.s);
}

// Store 4 consecutive columns n..n+3 of row m: one vector store when `full`
// (n+3 < N and N % 4 == 0, so the address is aligned), else element-wise
// with bounds checks.
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

// WM x WN 16x16 subtiles per wave; WAVES_M x WAVES_N waves per workgroup;
// D steps of fragments in flight.  SPLIT compiles the split-K epilogue.
template <int F, int WM, int WN, int WAVES_M, int WAVES_N, int D, int OUT, bool SPLIT>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N)
void mx_gemm_direct(GemmArgs p)
{
    constexpr int RB = FmtTraits<F>::step_bytes;   // row bytes per step
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    const int m0 = (blockIdx.y * WAVES_M + wm) * (WM * 16);
    const int n0 = (blockIdx.x * WAVES_N + wn) * (WN * 16);
    const size_t row_bytes = (size_t)p.ksteps * RB;
    const size_t srow_bytes = (size_t)p.ksteps * 4;

    // Row pointers; rows past the end are clamped to the last row (their
    // results are never stored), so every load stays inside the operands.
    const uint8_t *arow[WM], *asrow[WM], *brow[WN], *bsrow[WN];
#pragma unroll
    for (int x = 0; x < WM; ++x) {
        int m = min(m0 + 16 * x + r, p.M - 1);
        arow[x] = p.a + (size_t)m * row_bytes;
        asrow[x] = p.sa + (size_t)m * srow_bytes;
    }
#pragma unroll
    for (int y = 0; y < WN; ++y) {
        int n = min(n0 + 16 * y + r, p.N - 1);
        brow[y] = p.b + (size_t)n * row_bytes;
        bsrow[y] = p.sb + (size_t)n * srow_bytes;
    }

    int s0 = 0, s1 = p.ksteps;
    if constexpr (SPLIT) {
        s0 = (int)(((long long)blockIdx.z * p.ksteps) / p.splits);
        s1 = (int)(((long long)(blockIdx.z + 1) * p.ksteps) / p.splits);
    }
    const int nst = s1 - s0;
    // 4-wide vector stores/loads of C rows need N % 4 == 0 for alignment
    const bool vec_ok = (p.N & 3) == 0;

    Frag<F> fa[D][WM], fb[D][WN];
    v4f acc[WM][WN];
#pragma unroll
    for (int x = 0; x < WM; ++x)
#pragma unroll
        for (int y = 0; y < WN; ++y)
            acc[x][y] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < D; ++i) {
        if (i < nst) {
#pragma unroll
            for (int y = 0; y < WN; ++y)
                load_frag<F, true>(fb[i][y], brow[y], bsrow[y], s0 + i, g);
#pragma unroll
            for (int x = 0; x < WM; ++x)
                load_frag<F, false>(fa[i][x], arow[x], asrow[x], s0 + i, g);
        }
    }

    for (int base = 0; base < nst; base += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int st = base + i;
            if (st < nst) {
#pragma unroll
                for (int x = 0; x < WM; ++x)
#pragma unroll
                    for (int y = 0; y < WN; ++y)
                        acc[x][y] = mfma_step<F>(fb[i][y], fa[i][x], acc[x][y]);
                if (st + D < nst) {
#pragma unroll
                    for (int y = 0; y < WN; ++y)
                        load_frag<F, true>(fb[i][y], brow[y], bsrow[y], s0 + st + D, g);
#pragma unroll
                    for (int x = 0; x < WM; ++x)
                        load_frag<F, false>(fa[i][x], arow[x], asrow[x], s0 + st + D, g);
                }
            }
        }
    }

    if constexpr (!SPLIT) {
#pragma unroll
        for (int x = 0; x < WM; ++x) {
            const int m = m0 + 16 * x + r;
            if (m >= p.M)
                continue;
#pragma unroll
            for (int y = 0; y < WN; ++y) {
                const int n = n0 + 16 * y + 4 * g;
                if (n < p.N)
                    store4<OUT>(p.c, p.N, m, n, acc[x][y], vec_ok && n + 3 < p.N);
            }
        }
    } else {
        // 1. this split's FP32 partial tile
        float *part = p.part + (size_t)blockIdx.z * p.M * p.N;
#pragma unroll
        for (int x = 0; x < WM; ++x) {
            const int m = m0 + 16 * x + r;
            if (m >= p.M)
                continue;
#pragma unroll
            for (int y = 0; y < WN; ++y) {
                const int n = n0 + 16 * y + 4 * g;
                if (n < p.N)
                    store4<OUT_F32>(part, p.N, m, n, acc[x][y], vec_ok && n + 3 < p.N);
            }
        }
        // 2. publish, count arrivals
        __shared__ int last;
        __threadfence();
        __syncthreads();
        const unsigned tile = blockIdx.y * gridDim.x + blockIdx.x;
        if (threadIdx.x == 0) {
            unsigned prev = __hip_atomic_fetch_add(p.cnt + tile, 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            last = (prev == (unsigned)(p.splits - 1));
        }
        __syncthreads();
        if (!last)
            return;
        __threadfence();
        // 3. the last arrival sums the splits in order 0..S-1
#pragma unroll
        for (int x = 0; x < WM; ++x) {
            const int m = m0 + 16 * x + r;
            if (m >= p.M)
                continue;
#pragma unroll
            for (int y = 0; y < WN; ++y) {
                const int n = n0 + 16 * y + 4 * g;
                if (n >= p.N)
                    continue;
                const bool full = vec_ok && n + 3 < p.N;
                v4f s = v4f{0.f, 0.f, 0.f, 0.f};
                for (int z = 0; z < p.splits; ++z) {
                    const float *q = p.part + (size_t)z * p.M * p.N + (size_t)m * p.N + n;
                    v4f t;
                    if (full) {
                        t = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(q));
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            t[i] = (n + i < p.N) ? q[i] : 0.f;
                    }
                    s += t;
                }
                store4<OUT>(p.c, p.N, m, n, s, full);
            }
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(p.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace mxg
