// mx_stream.hpp -- NT MX block-scaled GEMM for small M (decode-width
// products), gfx950.
//
// For M up to a few dozen rows the product is bound by HBM bandwidth: every
// byte of B (N x K packed codes plus N x K/32 scales) is used exactly once,
// and A is small enough to come from L2.  The kernel therefore moves B from
// HBM straight into the registers the scaled MFMA reads, with no LDS
// staging, and keeps many loads in flight per wave.
//
// Work decomposition.  A workgroup owns one output tile of 16*MT rows by
// 16*WN columns and the whole K range; its KW waves split K between them
// (split-K inside the workgroup).  Wave w takes a contiguous run of 4-step
// groups (a group is 512 K values: 4 MFMA steps of 128).  At the end each
// wave parks its FP32 partial tile in LDS and the workgroup sums the KW
// partials in wave order 0, 1, ..., KW-1 -- a fixed order, so the result is
// deterministic -- converts it and stores it.  No workgroup ever waits for
// another, so no device-wide synchronisation or workspace is needed.
//
// Per wave and group the loads are: for each of the MT A subtiles and WN B
// subtiles, 4 steps of packed bytes (16 B per lane per step for FP4, 32 B
// for FP8) and one 16-byte load of the row's 16 scale codes (4 steps x 4
// blocks).  A ring of D groups lives in registers; the loads of group t+D
// are issued right after group t's MFMAs, so D groups are in flight.  Each
// wave starts its run of groups at a rotated position (by workgroup index)
// so that concurrent waves read A at different addresses instead of all
// hitting the same L2 channels at once.
//
// Rows past M or N, and ring slots past the end of a wave's run, are read
// through buffer descriptors whose range excludes them: such loads return
// zeros without touching memory, and zero codes with zero scale codes add
// exactly +0 to the accumulators.  The last wave also handles the K steps
// left over when K/128 is not a multiple of 4.
#pragma once

#include "mx_common.hpp"

namespace mxg {

struct StreamArgs {
    const uint8_t *a, *b, *sa, *sb;
    void *c;
    int M, N;
    int nsteps;           // K / 128
    unsigned row_bytes;   // packed bytes per operand row: K/2 (FP4) or K (FP8)
    unsigned srow_bytes;  // scale bytes per row: K/32
};

template <int F, int MT, int WN>
struct StreamGroup {
    StepFrag<F> a[MT][4], b[WN][4];
    u4v sa[MT], sb[WN];
};

template <int F, int MT, int WN>
__device__ __forceinline__ void stream_load_group(StreamGroup<F, MT, WN> &gr,
                                                  __amdgpu_buffer_rsrc_t ra,
                                                  __amdgpu_buffer_rsrc_t rb,
                                                  __amdgpu_buffer_rsrc_t rsa,
                                                  __amdgpu_buffer_rsrc_t rsb,
                                                  const unsigned (&aoff)[MT],
                                                  const unsigned (&boff)[WN],
                                                  const unsigned (&asoff)[MT],
                                                  const unsigned (&bsoff)[WN], int grp, bool valid,
                                                  int g)
{
    constexpr unsigned GB = 4 * FmtTraits<F>::step_bytes;   // packed bytes of a group per row
    const unsigned k = valid ? (unsigned)grp * GB : kOutOfRange;
    const unsigned ks = valid ? (unsigned)grp * 16u : kOutOfRange;
#pragma unroll
    for (int y = 0; y < WN; ++y) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            load_step<F, CPOL_NT>(gr.b[y][s], rb, boff[y] + k, s, g);
        gr.sb[y] = load16<CPOL_NT>(rsb, bsoff[y] + ks);
    }
#pragma unroll
    for (int x = 0; x < MT; ++x) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            load_step<F, CPOL_NONE>(gr.a[x][s], ra, aoff[x] + k, s, g);
        gr.sa[x] = load16<CPOL_NONE>(rsa, asoff[x] + ks);
    }
}

template <int F, int MT, int WN>
__device__ __forceinline__ void stream_mfma_group(const StreamGroup<F, MT, WN> &gr,
                                                  v4f (&acc)[MT][WN], int g)
{
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        unsigned sb[WN], sa[MT];
#pragma unroll
        for (int y = 0; y < WN; ++y)
            sb[y] = gr.sb[y][s] >> (8 * g);
#pragma unroll
        for (int x = 0; x < MT; ++x)
            sa[x] = gr.sa[x][s] >> (8 * g);
#pragma unroll
        for (int x = 0; x < MT; ++x)
#pragma unroll
            for (int y = 0; y < WN; ++y)
                acc[x][y] = mfma<F>(gr.b[y][s], sb[y], gr.a[x][s], sa[x], acc[x][y]);
    }
}

// MT x WN 16x16 subtiles per workgroup, KW waves splitting K, D groups in
// flight per wave.
template <int F, int MT, int WN, int KW, int D, int OUT>
__global__ __launch_bounds__(64 * KW)
void mx_gemm_stream(StreamArgs p)
{
    const int lane = threadIdx.x & 63;
    const int kw = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.y * (16 * MT);
    const int n0 = blockIdx.x * (16 * WN);

    // Buffers over this workgroup's rows only: rows past M or N fall
    // outside the range and read as zeros.
    const int mrows = min(16 * MT, p.M - m0);
    const int nrows = min(16 * WN, p.N - n0);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (size_t)m0 * p.row_bytes, mrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (size_t)n0 * p.row_bytes, nrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(p.sa + (size_t)m0 * p.srow_bytes, mrows * p.srow_bytes);
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(p.sb + (size_t)n0 * p.srow_bytes, nrows * p.srow_bytes);
    unsigned aoff[MT], asoff[MT], boff[WN], bsoff[WN];
#pragma unroll
    for (int x = 0; x < MT; ++x) {
        aoff[x] = (unsigned)(16 * x + r) * p.row_bytes;
        asoff[x] = (unsigned)(16 * x + r) * p.srow_bytes;
    }
#pragma unroll
    for (int y = 0; y < WN; ++y) {
        boff[y] = (unsigned)(16 * y + r) * p.row_bytes;
        bsoff[y] = (unsigned)(16 * y + r) * p.srow_bytes;
    }

    // This wave's run of groups, [g0, g0 + ng), visited from a rotated start.
    const int ngroups = p.nsteps >> 2;
    const int g0 = (int)(((long long)kw * ngroups) / KW);
    const int ng = (int)(((long long)(kw + 1) * ngroups) / KW) - g0;
    const int phase = ng > 0 ? (int)((blockIdx.x + 3u * blockIdx.y) % (unsigned)ng) : 0;

    v4f acc[MT][WN];
#pragma unroll
    for (int x = 0; x < MT; ++x)
#pragma unroll
        for (int y = 0; y < WN; ++y)
            acc[x][y] = v4f{0.f, 0.f, 0.f, 0.f};

    StreamGroup<F, MT, WN> ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
        int idx = i + phase;
        if (idx >= ng) idx -= ng;
        stream_load_group<F, MT, WN>(ring[i], ra, rb, rsa, rsb, aoff, boff, asoff, bsoff, g0 + idx,
                                     i < ng, g);
        // keep the slots' loads in ring order: the wait counts at the MFMAs
        // rely on slot i being issued before slot i+1
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int t = 0; t < ng; t += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            stream_mfma_group<F, MT, WN>(ring[i], acc, g);
            const int nt = t + i + D;
            int idx = nt + phase;
            if (idx >= ng) idx -= ng;
            stream_load_group<F, MT, WN>(ring[i], ra, rb, rsa, rsb, aoff, boff, asoff, bsoff,
                                         g0 + idx, nt < ng, g);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // K steps beyond the last whole group (K/128 not a multiple of 4).
    const int tail = p.nsteps & 3;
    if (tail && kw == KW - 1) {
        for (int s = ngroups * 4; s < p.nsteps; ++s) {
            StepFrag<F> fa[MT], fb[WN];
            unsigned sa[MT], sb[WN];
#pragma unroll
            for (int y = 0; y < WN; ++y) {
                load_step<F, CPOL_NT>(fb[y], rb, boff[y], s, g);
                sb[y] = load4(rsb, bsoff[y] + 4u * s) >> (8 * g);
            }
#pragma unroll
            for (int x = 0; x < MT; ++x) {
                load_step<F, CPOL_NONE>(fa[x], ra, aoff[x], s, g);
                sa[x] = load4(rsa, asoff[x] + 4u * s) >> (8 * g);
            }
#pragma unroll
            for (int x = 0; x < MT; ++x)
#pragma unroll
                for (int y = 0; y < WN; ++y)
                    acc[x][y] = mfma<F>(fb[y], sb[y], fa[x], sa[x], acc[x][y]);
        }
    }

    const bool vec_ok = (p.N & 3) == 0;
    if constexpr (KW == 1) {
#pragma unroll
        for (int x = 0; x < MT; ++x) {
            const int m = m0 + 16 * x + r;
#pragma unroll
            for (int y = 0; y < WN; ++y) {
                const int n = n0 + 16 * y + 4 * g;
                if (m < p.M && n < p.N)
                    store4<OUT>(p.c, p.N, m, n, acc[x][y], vec_ok && n + 3 < p.N);
            }
        }
    } else {
        // Partial tiles in LDS, rows padded by 4 floats so that the 16-byte
        // writes of one wave spread over all banks.
        constexpr int RS = 16 * WN + 4;
        __shared__ float red[KW][16 * MT][RS];
#pragma unroll
        for (int x = 0; x < MT; ++x)
#pragma unroll
            for (int y = 0; y < WN; ++y)
                *reinterpret_cast<v4f *>(&red[kw][16 * x + r][16 * y + 4 * g]) = acc[x][y];
        __syncthreads();
        constexpr int NQ = 16 * MT * 4 * WN;   // float4 column groups in the tile
        for (int q = threadIdx.x; q < NQ; q += 64 * KW) {
            const int row = q / (4 * WN), c4 = q % (4 * WN);
            v4f s = *reinterpret_cast<const v4f *>(&red[0][row][4 * c4]);
#pragma unroll
            for (int w = 1; w < KW; ++w)
                s += *reinterpret_cast<const v4f *>(&red[w][row][4 * c4]);
            const int m = m0 + row, n = n0 + 4 * c4;
            if (m < p.M && n < p.N)
                store4<OUT>(p.c, p.N, m, n, s, vec_ok && n + 3 < p.N);
        }
    }
}

}  // namespace mxg
