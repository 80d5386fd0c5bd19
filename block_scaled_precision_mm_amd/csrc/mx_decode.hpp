// mx_decode.hpp -- NT MX block-scaled GEMM for decode-width products
// (a few dozen rows of A), gfx950.
//
// At small M every byte of B is used by one workgroup only and the product
// is bound by how fast B streams from HBM.  Measured on MI355X, a workgroup
// that shares its B stages through LDS pays a barrier and an LDS round trip
// per stage, and re-loading the A and scale tiles with every stage adds
// about half as many L1 requests again as B itself.  This kernel instead:
//
//   * loads the whole A tile (16*MT rows x K) and the scale codes of all its
//     A and B rows into LDS once, at the start (one barrier);
//   * gives every wave its own B rows (16*WN of them) and its own ring of D
//     stages in LDS, filled with coalesced direct-to-LDS loads (four
//     consecutive lanes per 64-byte segment) and consumed by the same wave,
//     so the K loop has no barrier at all: a wave only waits for its own
//     loads (s_waitcnt vmcnt);
//   * reads MFMA fragments with ds_read_b128 from XOR-swizzled rows (chunk
//     index ^ row % 16), so the 16 rows of one read fall on different banks.
//
// The workgroup's output tile is 16*MT x 16*WN*NW; every wave covers all of
// K for its 16*WN columns.  The host picks this kernel only when the
// resident A tile and scale codes fit next to the rings (K <= KMAX).
//
// Ragged M / N and the K tail use offsets outside the buffer range: such a
// direct-to-LDS load writes zeros and moves no data.  Every LDS byte the
// kernel reads is written this way or by a real load -- the resident rows
// are loaded over their full KMAX-based stride.  Ragged rows meet zero codes
// and add exactly +0; steps past K in the last stage are skipped.
#pragma once

#include <type_traits>

#include "mx_lds.hpp"

namespace mxg {

template <int F, int MT, int NW, int WN, int SPS, int D, int KMAX>
struct DecodeGeom {
    static constexpr int SB = FmtTraits<F>::step_bytes;     // bytes per row per step
    static constexpr int BM = 16 * MT;
    static constexpr int BNW = 16 * WN;                      // B rows per wave
    static constexpr int BN = BNW * NW;
    static constexpr int RS = KMAX / 128 * SB;               // resident A row stride (bytes)
    static constexpr int SRS = KMAX / 32;                    // resident scale row stride (bytes)
    static constexpr int W = SPS * SB;                       // ring row bytes per stage
    static constexpr int CPR = W / 16;
    static constexpr int RPB = 1024 / W;                     // ring rows per 1 KB block
    static constexpr int LPS = BNW * W / 1024;               // ring loads per stage per wave
    // LDS layout
    static constexpr int A_OFF = 0;
    static constexpr int SA_OFF = A_OFF + BM * RS;
    static constexpr int SB_OFF = SA_OFF + BM * SRS;
    static constexpr int PAD_OFF = SB_OFF + BN * SRS;          // target of padding loads
    static constexpr int RING_OFF = (PAD_OFF + 256 + 1023) / 1024 * 1024;
    static constexpr int SLOT = BNW * W;                     // one stage of one wave
    static constexpr int BYTES = RING_OFF + NW * D * SLOT;
    // resident jobs (1 KB each), spread over the NW waves
    static constexpr int AJOBS = BM * RS / 1024;
    static constexpr int SJOBS = (BM + BN) * SRS / 1024;
    static constexpr int RJOBS = AJOBS + SJOBS;
    static constexpr int RPW = cdiv_c(RJOBS, NW);            // resident loads per wave
    static_assert(RS % 1024 == 0 && BM * SRS % 1024 == 0 && BN * SRS % 1024 == 0,
                  "resident rows in whole blocks, A and B scale rows in separate blocks");
    static_assert(RS / 16 >= 16, "row swizzle needs 16 chunks per resident row");
    static_assert(W <= 1024 && CPR >= 4 && BNW % RPB == 0, "ring stage must be whole blocks");
    static_assert(BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
    static_assert((D - 2) * LPS + RPW < 64, "outstanding loads must fit the vmcnt field");
    // ring row swizzle (rows of one wave's stage): as in the LDS kernel
    static constexpr int ROWS_PER_256 = W >= 256 ? 1 : 256 / W;
    static constexpr int SWZ_MASK = (CPR < 16 ? CPR : 16) - 1;
    __device__ static constexpr int ring_off(int row, int c)
    {
        return (row / RPB) * 1024 + (row % RPB) * W + 16 * (c ^ ((row / ROWS_PER_256) & SWZ_MASK));
    }
    __device__ static constexpr int a_off(int row, int c) { return row * RS + 16 * (c ^ (row & 15)); }
};

template <int LPS, int D>
__device__ __forceinline__ void decode_wait(int later)
{
    static_assert(D >= 2 && D <= 8, "ring depth");
    if constexpr (D >= 8) { if (later >= 6) { wait_vm<6 * LPS>(); return; } }
    if constexpr (D >= 7) { if (later >= 5) { wait_vm<5 * LPS>(); return; } }
    if constexpr (D >= 6) { if (later >= 4) { wait_vm<4 * LPS>(); return; } }
    if constexpr (D >= 5) { if (later >= 3) { wait_vm<3 * LPS>(); return; } }
    if constexpr (D >= 4) { if (later >= 2) { wait_vm<2 * LPS>(); return; } }
    if constexpr (D >= 3) { if (later >= 1) { wait_vm<1 * LPS>(); return; } }
    wait_vm<0>();
}

template <int F, int MT, int NW, int WN, int SPS, int D, int KMAX, int OUT>
__global__ __launch_bounds__(64 * NW)
void mx_gemm_decode(GemmArgs p)
{
    using G = DecodeGeom<F, MT, NW, WN, SPS, D, KMAX>;
    __shared__ __attribute__((aligned(1024))) char smem[G::BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.y * G::BM;
    const int n0 = blockIdx.x * G::BN;
    const int mrows = min(G::BM, p.M - m0);
    const int nrows = min(G::BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (size_t)m0 * p.row_bytes, mrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (size_t)n0 * p.row_bytes, nrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(p.sa + (size_t)m0 * p.srow_bytes, mrows * p.srow_bytes);
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(p.sb + (size_t)n0 * p.srow_bytes, nrows * p.srow_bytes);

    // 1. Resident A tile and scale codes, spread over the waves.  A row is
    //    RS bytes in LDS (K*e of them valid); chunk c of row `row` sits at
    //    chunk c ^ (row % 16).  Scale rows are SRS bytes, unswizzled.
#pragma unroll
    for (int i = 0; i < G::RPW; ++i) {
        const int q = wave + NW * i;
        if (q >= G::RJOBS) {
            dma4(rsa, (lds_ptr_t)(smem + G::PAD_OFF), kOutOfRange);    // count padding
            continue;
        }
        if (q < G::AJOBS) {
            const int row = q / (G::RS / 1024);
            const int cl = (q % (G::RS / 1024)) * 64 + lane;       // LDS chunk of this lane
            const int cg = cl ^ (row & 15);                         // global chunk it holds
            const unsigned off = (row < mrows && 16u * cg < p.row_bytes)
                                     ? (unsigned)row * p.row_bytes + 16u * cg
                                     : kOutOfRange;
            dma16(ra, (lds_ptr_t)(smem + G::A_OFF + q * 1024), off);
        } else {
            const int e = (q - G::AJOBS) * 1024 + 16 * lane;        // byte in [A rows | B rows] x SRS
            const bool isa = (q - G::AJOBS) * 1024 < G::BM * G::SRS;   // wave-uniform
            const int row = e / G::SRS, col = e % G::SRS;
            const int rr = isa ? row : row - G::BM;
            const unsigned off = (rr < (isa ? mrows : nrows) && (unsigned)col < p.srow_bytes)
                                     ? (unsigned)rr * p.srow_bytes + (unsigned)col
                                     : kOutOfRange;
            dma16(isa ? rsa : rsb, (lds_ptr_t)(smem + G::SA_OFF + (q - G::AJOBS) * 1024), off);
        }
    }

    // 2. This wave's B rows stream through its private ring.
    char *ring = smem + G::RING_OFF + wave * D * G::SLOT;
    const int nst = cdiv_c(p.nsteps, SPS);   // stages
    auto issue = [&](int t) {
        char *slot = ring + (t % D) * G::SLOT;
#pragma unroll
        for (int j = 0; j < G::LPS; ++j) {
            const int row = j * G::RPB + lane / G::CPR;              // row within the wave's rows
            const int c = (lane % G::CPR) ^ ((row / G::ROWS_PER_256) & G::SWZ_MASK);
            const int step = t * SPS + c / (G::SB / 16);
            const int brow = wave * G::BNW + row;                    // row within the tile
            const unsigned off = (step < p.nsteps && brow < nrows)
                                     ? (unsigned)brow * p.row_bytes + (unsigned)(t * SPS) * G::SB + 16u * c
                                     : kOutOfRange;
            dma16(rb, (lds_ptr_t)(slot + j * 1024), off);
        }
    };
#pragma unroll
    for (int i = 0; i < D - 1; ++i)
        if (i < nst)
            issue(i);

    // resident loads were issued before any ring load: once at most the ring
    // prologue is outstanding they have landed; the barrier makes every
    // wave's share visible
    decode_wait<G::LPS, D>(min(D - 1, nst));
    block_barrier();

    v4f acc[MT][WN];
#pragma unroll
    for (int x = 0; x < MT; ++x)
#pragma unroll
        for (int y = 0; y < WN; ++y)
            acc[x][y] = v4f{0.f, 0.f, 0.f, 0.f};

    const char *ares = smem + G::A_OFF;
    const unsigned char *sres_a = reinterpret_cast<const unsigned char *>(smem + G::SA_OFF);
    const unsigned char *sres_b =
        reinterpret_cast<const unsigned char *>(smem + G::SB_OFF) + wave * G::BNW * G::SRS;
    // One stage of MFMAs.  In the last, partial stage the steps past K are
    // skipped: their B codes are zeros, but a resident scale row is loaded in
    // 16-byte pieces, so its bytes past K/32 may hold the next row's codes
    // (a NaN code there would poison the sum).
    auto compute = [&](const char *slot, int t, auto tail) {
#pragma unroll
        for (int s = 0; s < SPS; ++s) {
            const int k = t * SPS + s;
            if constexpr (decltype(tail)::value)
                if (k >= p.nsteps) break;
            StepFrag<F> fa[MT], fb[WN];
            unsigned sa[MT], sb[WN];
#pragma unroll
            for (int x = 0; x < MT; ++x) {
                const int row = 16 * x + r;
                if constexpr (F == FMT_FP4) {
                    fa[x].d[0] = *reinterpret_cast<const u4v *>(ares + G::a_off(row, 4 * k + g));
                } else {
                    fa[x].d[0] = *reinterpret_cast<const u4v *>(ares + G::a_off(row, 8 * k + g));
                    fa[x].d[1] = *reinterpret_cast<const u4v *>(ares + G::a_off(row, 8 * k + 4 + g));
                }
                sa[x] = sres_a[row * G::SRS + 4 * k + g];
            }
#pragma unroll
            for (int y = 0; y < WN; ++y) {
                const int row = 16 * y + r;
                if constexpr (F == FMT_FP4) {
                    fb[y].d[0] = *reinterpret_cast<const u4v *>(slot + G::ring_off(row, 4 * s + g));
                } else {
                    fb[y].d[0] = *reinterpret_cast<const u4v *>(slot + G::ring_off(row, 8 * s + g));
                    fb[y].d[1] = *reinterpret_cast<const u4v *>(slot + G::ring_off(row, 8 * s + 4 + g));
                }
                sb[y] = sres_b[row * G::SRS + 4 * k + g];
            }
#pragma unroll
            for (int x = 0; x < MT; ++x)
#pragma unroll
                for (int y = 0; y < WN; ++y)
                    acc[x][y] = mfma<F>(fb[y], sb[y], fa[x], sa[x], acc[x][y]);
        }
    };
    const int nfull = p.nsteps / SPS;
    for (int t = 0; t < nst; ++t) {
        decode_wait<G::LPS, D>(min(D - 2, nst - 1 - t));
        // the slot refilled below was last read by this wave's previous
        // stage; its reads have completed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (t + D - 1 < nst)
            issue(t + D - 1);
        const char *slot = ring + (t % D) * G::SLOT;
        if (t < nfull)
            compute(slot, t, std::false_type{});
        else
            compute(slot, t, std::true_type{});
    }

    const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
    for (int x = 0; x < MT; ++x) {
        const int m = m0 + 16 * x + r;
#pragma unroll
        for (int y = 0; y < WN; ++y) {
            const int n = n0 + wave * G::BNW + 16 * y + 4 * g;
            if (m < p.M && n < p.N)
                store4<OUT>(p.c, p.N, m, n, acc[x][y], vec_ok && n + 3 < p.N);
        }
    }
}

}  // namespace mxg
