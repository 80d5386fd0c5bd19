// mx_decode.hpp -- NT MX block-scaled GEMM for decode-width products (up to
// 32 rows of A), gfx950.
//
// At small M every byte of B is used once: the product is a B stream, and
// the MFMA work is a few percent of the time.  Measured on MI355X, what
// sets the stream's speed is the shape of the loads:
//   * DRAM: B rows read in long contiguous runs by one wave stream faster
//     than the same rows cut into 64-byte slices read by different waves
//     (split-K), and reading A once per workgroup instead of once per wave
//     saves its share of the traffic;
//   * L1: a 16-byte-per-lane load whose lanes follow the MFMA operand layout
//     (16 rows in consecutive lanes) costs ~2.5x the address cycles of a
//     coalesced one, and a one-row-per-lane scale load ~4x.
// So:
//   * a workgroup of NW waves owns 16*NW consecutive B rows and all 16*MT A
//     rows; wave w streams B rows [16w, 16w+16) over the whole of K -- no
//     split-K, no reduction, no barrier in the K loop;
//   * the A tile and the scale codes of all the workgroup's rows are loaded
//     once, as flat coalesced ranges, into LDS (hence the K limit KMAX: the
//     A tile must fit);
//   * B stages of 256 bytes per row are loaded with 16-byte loads in which
//     16 consecutive lanes read one row's 256 contiguous bytes, into a
//     G-deep register ring, stored into one of two private LDS slots and
//     read back as 16x16x128 MFMA fragments.
//
// LDS layouts: code rows in groups of 8, chunk-major inside a group (chunk c
// of the 8 rows = 128 contiguous bytes) with a padded chunk stride of 160
// bytes, so both the fragment reads and the staging stores run at full LDS
// rate; scale codes as [128-K step][row] dwords, so a step's codes of 16
// consecutive rows are contiguous.
//
// Ragged M / N: rows past the operand read as zeros (out of the buffer
// range) and add exactly +0.  K tail: a B stage that runs past the row end
// reads the next row's bytes, so MFMA steps past K are skipped.
#pragma once

#include "mx_lds.hpp"
#include "mx_tile.hpp"

namespace mxg {

template <int F, int MT, int NW, int KMAX>
struct DecodeGeom {
    static constexpr int SB = FmtTraits<F>::step_bytes;      // bytes per row per 128-K step
    static constexpr int BM = 16 * MT;                       // A rows
    static constexpr int BN = 16 * NW;                       // B rows (16 per wave)
    static constexpr int CHUNK = 160;                        // padded 16-byte chunk stride
    static constexpr int SW = 256;                           // B stage: bytes per row
    static constexpr int SPS = SW / SB;                      // MFMA steps per stage
    static constexpr int SCH = SW / 16;                      // chunks per row per stage
    static constexpr int SLOT = 2 * SCH * CHUNK;             // 16 rows = 2 groups of 8
    static constexpr int RB_MAX = KMAX / 128 * SB;           // A row bytes at K = KMAX
    static constexpr int ACH = RB_MAX / 16;                  // A chunks per row at KMAX
    static constexpr int AGROUP = ACH * CHUNK;               // one 8-row group of A
    static constexpr int NSTEP_MAX = KMAX / 128;
    // LDS map
    static constexpr int SA_OFF = BM / 8 * AGROUP;                         // [step][BM] dwords
    static constexpr int SBS_OFF = SA_OFF + NSTEP_MAX * BM * 4;            // [step][BN] dwords
    static constexpr int B_OFF = SBS_OFF + NSTEP_MAX * BN * 4;             // [wave][2] slots
    static constexpr int BYTES = B_OFF + NW * 2 * SLOT;
    // coalesced prologue loads per wave: A chunks (16 bytes), scale dwords
    static constexpr int PA = cdiv_c(BM * ACH, 64 * NW);
    static constexpr int PS = cdiv_c((BM + BN) * NSTEP_MAX, 64 * NW);
    static_assert(BM % 8 == 0 && SW % SB == 0 && KMAX % 512 == 0, "tile geometry");
    static_assert(BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
    __device__ static constexpr int a_off(int row, int c)
    {
        return (row >> 3) * AGROUP + c * CHUNK + (row & 7) * 16;
    }
    __device__ static constexpr int b_off(int row, int c)   // within a wave's slot
    {
        return (row >> 3) * (SCH * CHUNK) + c * CHUNK + (row & 7) * 16;
    }
};

template <int F, int MT, int NW, int KMAX, int G, int OUT>
__global__ __launch_bounds__(64 * NW)
void mx_gemm_decode(GemmArgs p)
{
    using D = DecodeGeom<F, MT, NW, KMAX>;
    constexpr int LB = 4;   // B loads per stage: 4 rows x 256 bytes each
    static_assert(G >= 2 && G * LB + D::PA + 2 * D::PS < 64, "outstanding loads must fit the vmcnt field");
    __shared__ __attribute__((aligned(1024))) char smem[D::BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.y * D::BM, n0 = blockIdx.x * D::BN;
    const int mrows = min(D::BM, p.M - m0);
    const int nrows = min(D::BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (size_t)m0 * p.row_bytes, mrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (size_t)n0 * p.row_bytes, nrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(p.sa + (size_t)m0 * p.srow_bytes, mrows * p.srow_bytes);
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(p.sb + (size_t)n0 * p.srow_bytes, nrows * p.srow_bytes);
    const int T = (int)((p.row_bytes + D::SW - 1) / D::SW);   // B stages
    const int nst = p.nsteps;                                 // 128-K steps (<= NSTEP_MAX)

    // ---- B ring: load j of a stage covers rows 4j .. 4j+3 of this wave's 16
    // (lane l: row 4j + l/16, bytes 16*(l%16) of the stage's 256)
    const unsigned bload = (unsigned)(16 * wave + (lane >> 4)) * p.row_bytes + 16u * (unsigned)(lane & 15);
    const unsigned bstride = 4u * p.row_bytes;
    u4v stg[G][LB];
    auto fill_stage = [&](u4v (&set)[LB], int t) {
        if (t < T) {
#pragma unroll
            for (int j = 0; j < LB; ++j)
                set[j] = load16<CPOL_NONE>(rb, bload + (unsigned)j * bstride + (unsigned)t * D::SW);
        } else {
#pragma unroll
            for (int j = 0; j < LB; ++j)
                set[j] = u4v{0u, 0u, 0u, 0u};
        }
    };
    char *slots = smem + D::B_OFF + wave * 2 * D::SLOT;
    const int bw_lane = D::b_off(lane >> 4, lane & 15);   // row l/16 of a 4-row load, chunk l%16
    auto store_stage = [&](const u4v (&set)[LB], int t) {
        char *slot = slots + (t & 1) * D::SLOT;
#pragma unroll
        for (int j = 0; j < LB; ++j)
            *reinterpret_cast<u4v *>(slot + bw_lane + D::b_off(4 * j, 0)) = set[j];
    };

    // ---- prologue: the first G B stages, then the A tile (flat: chunk i of
    // the tile is bytes [16i, 16i+16) of rows m0.., i.e. row i / CH, chunk
    // i % CH) and the scale dwords (flat: dword f of [A rows | B rows] is
    // row f / NS, step f % NS), all in flight together
#pragma unroll
    for (int i = 0; i < G; ++i)
        fill_stage(stg[i], i);
    const unsigned CH = p.row_bytes / 16u;             // A chunks per row
    const unsigned NS = (unsigned)nst;                  // scale dwords per row
    const unsigned a_chunks = (unsigned)mrows * CH;
    const unsigned s_dwords = (unsigned)(mrows + nrows) * NS;
    u4v av[D::PA];
    unsigned sv[D::PS];
#pragma unroll
    for (int i = 0; i < D::PA; ++i) {
        const unsigned idx = (unsigned)(64 * (NW * i + wave) + lane);
        av[i] = load16<CPOL_NONE>(ra, idx < a_chunks ? 16u * idx : kOutOfRange);
    }
#pragma unroll
    for (int i = 0; i < D::PS; ++i) {
        const unsigned f = (unsigned)(64 * (NW * i + wave) + lane);
        const unsigned fa = (unsigned)mrows * NS;       // A dwords come first
        const bool isa = f < fa;
        const unsigned off = f < s_dwords ? 4u * (isa ? f : f - fa) : kOutOfRange;
        // one load may span A's and B's scale rows; a buffer resource must
        // be uniform, so load from both with the other side's lanes out of
        // range (they read 0)
        sv[i] = load4(rsa, isa ? off : kOutOfRange) | load4(rsb, isa ? kOutOfRange : off);
    }
    wait_vm<0>();
#pragma unroll
    for (int i = 0; i < D::PA; ++i) {
        const unsigned idx = (unsigned)(64 * (NW * i + wave) + lane);
        if (idx < a_chunks) {
            const unsigned row = idx / CH, c = idx % CH;
            *reinterpret_cast<u4v *>(smem + D::a_off((int)row, (int)c)) = av[i];
        }
    }
#pragma unroll
    for (int i = 0; i < D::PS; ++i) {
        const unsigned f = (unsigned)(64 * (NW * i + wave) + lane);
        const unsigned fa = (unsigned)mrows * NS;
        if (f < s_dwords) {
            const bool isa = f < fa;
            const unsigned ff = isa ? f : f - fa;
            const unsigned row = ff / NS, k = ff % NS;
            *reinterpret_cast<unsigned *>(smem + (isa ? D::SA_OFF + 4 * (k * D::BM + row)
                                                      : D::SBS_OFF + 4 * (k * D::BN + row))) = sv[i];
        }
    }
    __syncthreads();   // the A tile and scale codes are shared by all waves

    v4f acc[MT];
#pragma unroll
    for (int x = 0; x < MT; ++x)
        acc[x] = v4f{0.f, 0.f, 0.f, 0.f};

    // one stage: store it, refill its staging set, then its MFMA steps
    auto stage = [&](auto uc, int t) {
        constexpr int u = decltype(uc)::value;
        if (t + G - 1 < T)
            wait_vm<(G - 1) * LB>();   // stage t's loads (the G-1 later stages may be in flight)
        else
            wait_vm<0>();
        store_stage(stg[u], t);
        fill_stage(stg[u], t + G);
        const char *slot = slots + (t & 1) * D::SLOT;
#pragma unroll
        for (int s = 0; s < D::SPS; ++s) {
            const int k = t * D::SPS + s;   // global step
            if (k >= nst)
                break;
            StepFrag<F> fb, fa[MT];
            if constexpr (F == FMT_FP4) {
                fb.d[0] = *reinterpret_cast<const u4v *>(slot + D::b_off(r, 4 * s + g));
            } else {
                fb.d[0] = *reinterpret_cast<const u4v *>(slot + D::b_off(r, 8 * s + g));
                fb.d[1] = *reinterpret_cast<const u4v *>(slot + D::b_off(r, 8 * s + 4 + g));
            }
            const unsigned sb = *reinterpret_cast<const unsigned *>(smem + D::SBS_OFF + 4 * (k * D::BN + 16 * wave + r)) >> (8 * g);
            unsigned sa[MT];
#pragma unroll
            for (int x = 0; x < MT; ++x) {
                const int row = 16 * x + r;
                if constexpr (F == FMT_FP4) {
                    fa[x].d[0] = *reinterpret_cast<const u4v *>(smem + D::a_off(row, 4 * k + g));
                } else {
                    fa[x].d[0] = *reinterpret_cast<const u4v *>(smem + D::a_off(row, 8 * k + g));
                    fa[x].d[1] = *reinterpret_cast<const u4v *>(smem + D::a_off(row, 8 * k + 4 + g));
                }
                sa[x] = *reinterpret_cast<const unsigned *>(smem + D::SA_OFF + 4 * (k * D::BM + row)) >> (8 * g);
            }
#pragma unroll
            for (int x = 0; x < MT; ++x)
                acc[x] = mfma<F>(fb, sb, fa[x], sa[x], acc[x]);
        }
    };
    for (int t0 = 0; t0 < T; t0 += G)
        static_for<G>([&](auto uc) {
            if (t0 + decltype(uc)::value < T)
                stage(uc, t0 + decltype(uc)::value);
        });
    wait_vm<0>();

    const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
    for (int x = 0; x < MT; ++x) {
        const int m = m0 + 16 * x + r;
        const int n = n0 + 16 * wave + 4 * g;
        if (m < p.M && n < p.N)
            store4<OUT>(p.c, p.N, m, n, acc[x], vec_ok && n + 3 < p.N);
    }
}

}  // namespace mxg
