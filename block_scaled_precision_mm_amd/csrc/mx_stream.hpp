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
// for FP8), and for each operand one load that gives every lane the 16
// scale codes (4 steps x 4 blocks) of one row.  The packed bytes are loaded
// in row order -- lanes 4q .. 4q+3 read the 64 contiguous bytes of row q --
// and moved into the MFMA's lane order (lane 16g + r: row r, 16-byte chunk
// g) with ds_bpermute right before the MFMAs: on MI355X the address unit
// takes a row-ordered 16-byte load about 2.5x faster than one in the MFMA's
// order, which puts 16 different rows into 16 consecutive lanes (c2,
// 32 x 14336 x 4096 MXFP4: 11.41 -> 10.56 us per call; results bit-identical).  The vector-memory address
// unit, not HBM, limits a kernel that issues many small loads, so the loads
// are as few as the MFMA layout allows and a ring slot is only refilled
// with a real group.  A ring of D groups lives in registers; the loads of
// group t+D are issued right after group t's MFMAs, so D groups are in
// flight.  Each wave starts its run of groups at a rotated position (by
// workgroup index) so that concurrent waves read A at different addresses
// instead of all hitting the same L2 channels at once.
//
// Rows past M or N (and, when a wave has fewer groups than ring slots, the
// unused slots) are read through buffer descriptors whose range excludes
// them: such loads return zeros without touching memory, and zero codes
// with zero scale codes add exactly +0 to the accumulators.  The last wave
// also handles the K steps left over when K/128 is not a multiple of 4.
#pragma once

#include "mx_common.hpp"
#include "mx_epilogue.hpp"
#include "mx_group.hpp"
#include "mx_splitk.hpp"

namespace mxg {

template <int F, int MT, int WN>
struct StreamGroup {
    StepFrag<F> a[MT][4], b[WN][4];
    u4v sca, scb;   // lane L: the group's 16 scale codes of A row L / B row L
};

// Per-lane offsets of one workgroup's rows.
template <int MT, int WN>
struct StreamOffsets {
    unsigned a[MT], b[WN];   // packed-operand row (lane / 4) of the lane's row-order load in subtile x / y
    unsigned sa, sb;         // scale row of lane L (A row L, B row L), or out of range
};

template <int F, int MT, int WN>
__device__ __forceinline__ void stream_load_group(StreamGroup<F, MT, WN> &gr,
                                                  __amdgpu_buffer_rsrc_t ra,
                                                  __amdgpu_buffer_rsrc_t rb,
                                                  __amdgpu_buffer_rsrc_t rsa,
                                                  __amdgpu_buffer_rsrc_t rsb,
                                                  const StreamOffsets<MT, WN> &o, int grp,
                                                  bool valid, int chunk)
{
    constexpr unsigned GB = 4 * FmtTraits<F>::step_bytes;   // packed bytes of a group per row
    const unsigned k = valid ? (unsigned)grp * GB : kOutOfRange;
    const unsigned ks = valid ? (unsigned)grp * 16u : kOutOfRange;
    // scales first, then step by step, so that step 0's MFMAs can start as
    // soon as the first loads have arrived
    gr.scb = load16<CPOL_NONE>(rsb, o.sb + ks);
    gr.sca = load16<CPOL_NONE>(rsa, o.sa + ks);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int y = 0; y < WN; ++y)
            load_step<F, CPOL_NONE>(gr.b[y][s], rb, o.b[y] + k, s, chunk);
#pragma unroll
        for (int x = 0; x < MT; ++x)
            load_step<F, CPOL_NONE>(gr.a[x][s], ra, o.a[x] + k, s, chunk);
    }
}

// The scale codes arrive one row per lane; the MFMA wants row r's code of
// block g in lane (r, g).  ds_bpermute fetches the row's step dword from the
// lane that loaded it, and the shift picks the block's byte.
// A fragment loaded in row order, in the MFMA's lane order (see above).
template <int F>
__device__ __forceinline__ StepFrag<F> perm_frag(const StepFrag<F> &f, int addr)
{
    StepFrag<F> o;
#pragma unroll
    for (int v = 0; v < FmtTraits<F>::nvec; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o.d[v][i] = (unsigned)__builtin_amdgcn_ds_bpermute(addr, (int)f.d[v][i]);
    return o;
}

template <int F, int MT, int WN>
__device__ __forceinline__ void stream_mfma_group(const StreamGroup<F, MT, WN> &gr,
                                                  v4f (&acc)[MT][WN], int r, int g)
{
    const int paddr = 4 * (4 * r + g);   // lane (r, g) takes row r, chunk g from lane 4r + g
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        unsigned sb[WN], sa[MT];
#pragma unroll
        for (int y = 0; y < WN; ++y)
            sb[y] = (unsigned)__builtin_amdgcn_ds_bpermute(4 * (16 * y + r), (int)gr.scb[s]) >>
                    (8 * g);
#pragma unroll
        for (int x = 0; x < MT; ++x)
            sa[x] = (unsigned)__builtin_amdgcn_ds_bpermute(4 * (16 * x + r), (int)gr.sca[s]) >>
                    (8 * g);
#pragma unroll
        for (int x = 0; x < MT; ++x)
#pragma unroll
            for (int y = 0; y < WN; ++y)
                acc[x][y] = mfma<F>(perm_frag<F>(gr.b[y][s], paddr), sb[y], perm_frag<F>(gr.a[x][s], paddr),
                                    sa[x], acc[x][y]);
    }
}

// MT x WN 16x16 subtiles per workgroup, KW waves splitting K, D groups in
// flight per wave.
template <int F, int MT, int WN, int KW, int D, int OUT, int GRP = 0, int EPI = 0>
__global__ __launch_bounds__(64 * KW)
void mx_gemm_stream(GemmArgs p)
{
    static_assert(MT <= 4 && WN <= 4, "one lane per scale row: at most 64 rows per operand");
    static_assert(!EPI || KW > 1, "the fused epilogue runs on the reduced tile");
    static_assert(EPI || OUT <= OUT_F32, "MX output kinds need the fused epilogue");
    const int lane = threadIdx.x & 63;
    const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int r = lane & 15, g = lane >> 4;
    const int lc = lane & 3, lr = lane >> 2;   // coalesced loads: row lr, 16-byte chunk lc
    int m0 = blockIdx.y * (16 * MT);
    if constexpr (GRP) {
        // grouped product: a unit is one M tile (blockIdx.y) of some group
        int grp, local, row0, rows;
        if (!find_group(p.offs, p.groups, p.M, (int)blockIdx.y, 16 * MT, 1, grp, local, row0, rows))
            return;
        select_group<OUT>(p, grp, row0, rows);
        m0 = local * (16 * MT);
    }
    const int n0 = blockIdx.x * (16 * WN);
    // split-K across workgroups: this workgroup's K part (whole groups);
    // only with KW > 1, whose epilogue holds the cross-workgroup reduction
    if constexpr (!GRP && !EPI && KW > 1)
        select_split<F>(p, 4);

    // Buffers over this workgroup's rows (and K part) only: rows past M or
    // N fall outside the range and read as zeros.
    const int mrows = min(16 * MT, p.M - m0);
    const int nrows = min(16 * WN, p.N - n0);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.a + (size_t)m0 * p.row_bytes, part_range(mrows, p.row_bytes, p.kbytes));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.b + (size_t)n0 * p.row_bytes, part_range(nrows, p.row_bytes, p.kbytes));
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(p.sa + (size_t)m0 * p.srow_bytes, part_range(mrows, p.srow_bytes, 4u * p.nsteps));
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(p.sb + (size_t)n0 * p.srow_bytes, part_range(nrows, p.srow_bytes, 4u * p.nsteps));
    StreamOffsets<MT, WN> o;
#pragma unroll
    for (int x = 0; x < MT; ++x)
        o.a[x] = (unsigned)(16 * x + lr) * p.row_bytes;
#pragma unroll
    for (int y = 0; y < WN; ++y)
        o.b[y] = (unsigned)(16 * y + lr) * p.row_bytes;
    o.sa = lane < 16 * MT ? (unsigned)lane * p.srow_bytes : kOutOfRange;
    o.sb = lane < 16 * WN ? (unsigned)lane * p.srow_bytes : kOutOfRange;

    // This wave's run of groups, [g0, g0 + ng), visited from a rotated start.
    const int ngroups = p.nsteps >> 2;
    const int g0 = (int)(((long long)kw * ngroups) / KW);
    const int ng = (int)(((long long)(kw + 1) * ngroups) / KW) - g0;
    const int phase = ng > 0 ? (int)((blockIdx.x + 3u * blockIdx.y) % (unsigned)ng) : 0;
    auto group_at = [&](int t) {
        int idx = t + phase;
        if (idx >= ng) idx -= ng;
        return g0 + idx;
    };

    v4f acc[MT][WN];
#pragma unroll
    for (int x = 0; x < MT; ++x)
#pragma unroll
        for (int y = 0; y < WN; ++y)
            acc[x][y] = v4f{0.f, 0.f, 0.f, 0.f};

    // Ring prologue: D groups, issued unconditionally (slots past the run
    // read zeros) so that the wait counts of every later MFMA are exact.
    StreamGroup<F, MT, WN> ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
        stream_load_group<F, MT, WN>(ring[i], ra, rb, rsa, rsb, o, group_at(i), i < ng, lc);
        // keep the slots' loads in ring order: the wait counts at the MFMAs
        // rely on slot i being issued before slot i+1
        __builtin_amdgcn_sched_barrier(0);
    }
    // Steady state: every refill is a real group.
    int t = 0;
    for (; t + 2 * D <= ng; t += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            stream_mfma_group<F, MT, WN>(ring[i], acc, r, g);
            stream_load_group<F, MT, WN>(ring[i], ra, rb, rsa, rsb, o, group_at(t + D + i), true,
                                         lc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // Drain: the slots hold groups t .. t+D-1 (those that exist); fewer than
    // D more remain to be loaded.
    const int rem = ng - t;
#pragma unroll
    for (int i = 0; i < D; ++i) {
        if (i < rem)
            stream_mfma_group<F, MT, WN>(ring[i], acc, r, g);
        if (D + i < rem)
            stream_load_group<F, MT, WN>(ring[i], ra, rb, rsa, rsb, o, group_at(t + D + i), true,
                                         lc);
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (D + i < rem)
            stream_mfma_group<F, MT, WN>(ring[i], acc, r, g);

    // K steps beyond the last whole group (K/128 not a multiple of 4).
    const int tail = p.nsteps & 3;
    if (tail && kw == KW - 1) {
        for (int s = ngroups * 4; s < p.nsteps; ++s) {
            StepFrag<F> fa[MT], fb[WN];
            unsigned sa[MT], sb[WN];
#pragma unroll
            for (int y = 0; y < WN; ++y) {
                load_step<F, CPOL_NONE>(fb[y], rb, (unsigned)(16 * y + r) * p.row_bytes, s, g);
                sb[y] = load4(rsb, (unsigned)(16 * y + r) * p.srow_bytes + 4u * s) >> (8 * g);
            }
#pragma unroll
            for (int x = 0; x < MT; ++x) {
                load_step<F, CPOL_NONE>(fa[x], ra, (unsigned)(16 * x + r) * p.row_bytes, s, g);
                sa[x] = load4(rsa, (unsigned)(16 * x + r) * p.srow_bytes + 4u * s) >> (8 * g);
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
        if constexpr (!GRP && !EPI) {
            if (p.splits > 1) {
                // split-K: this part's tile (its KW partials summed in wave
                // order), then the parts summed by the last to finish
                constexpr int CG = 4 * WN, NQ = 16 * MT * CG, NTH = 64 * KW;
                constexpr int QPT = (NQ + NTH - 1) / NTH;
                const int tid = (int)threadIdx.x;
                v4f fin[QPT];
#pragma unroll
                for (int i = 0; i < QPT; ++i) {
                    const int q = tid + i * NTH;
                    v4f sum = {0.f, 0.f, 0.f, 0.f};
                    if (q < NQ) {
                        sum = *reinterpret_cast<const v4f *>(&red[0][q / CG][4 * (q % CG)]);
#pragma unroll
                        for (int w = 1; w < KW; ++w)
                            sum += *reinterpret_cast<const v4f *>(&red[w][q / CG][4 * (q % CG)]);
                    }
                    fin[i] = sum;
                }
                const int tile = (int)(blockIdx.y * gridDim.x + blockIdx.x);
                if (!splitk_reduce<QPT, NTH>(p, tile, tid, [&](int j) { return fin[j]; },
                                             [&](int j, v4f x) { fin[j] = x; }))
                    return;
#pragma unroll
                for (int i = 0; i < QPT; ++i) {
                    const int q = tid + i * NTH;
                    const int m = m0 + q / CG, n = n0 + 4 * (q % CG);
                    if (q < NQ && m < p.M && n < p.N)
                        store4<OUT>(p.c, p.N, m, n, fin[i], vec_ok && n + 3 < p.N);
                }
                return;
            }
        }
        // the KW partials summed in wave order while the output is written
        store_reduced_tile<OUT, EPI, 16 * MT, 4 * WN>(
            p, m0, n0, (int)threadIdx.x, 64 * KW, [&](int row, int c4) {
                v4f sum = *reinterpret_cast<const v4f *>(&red[0][row][4 * c4]);
#pragma unroll
                for (int w = 1; w < KW; ++w)
                    sum += *reinterpret_cast<const v4f *>(&red[w][row][4 * c4]);
                return sum;
            });
    }
}

}  // namespace mxg
