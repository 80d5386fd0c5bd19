// mx_skinny.hpp -- NT MX block-scaled GEMM for decode-width products (up to
// 64 rows of A), gfx950.
//
// At small M every byte of B is used once and the product is a B stream.
// Measured on MI355X, what limits such a stream is not the MFMA work but
// how the loads are shaped: a 16-byte-per-lane load in the MFMA operand
// layout (16 different rows in consecutive lanes) costs the L1 about 2.5x
// the cycles of a load in which every four consecutive lanes read one
// row's 64 contiguous bytes, and a scale load with one row per lane about
// 4x.  This kernel therefore uses the data path of the large-tile kernel
// (mx_tile.hpp) inside each wave:
//
//   * a workgroup owns a (32*MT) x (32*NT) output tile over all of K; its KW
//     waves split K into runs of whole scale periods, and each wave streams
//     its run on its own -- there is no barrier in the K loop;
//   * per 64-byte stage (128 K of E2M1, 64 of E4M3) the wave loads its A and
//     B rows with coalesced 16-byte loads into a G-deep register ring,
//     stores each stage into one of two private LDS slots in the padded,
//     chunk-major layout, and reads the 32x32x64 MFMA fragments back at full
//     LDS rate; a wave's own LDS accesses complete in order, so reusing a
//     slot needs no wait;
//   * scale codes: 16 bytes per row per period of P stages (four 128-K
//     steps), one row per lane, stored transposed ([step][row] dwords);
//   * the KW partial tiles are summed in LDS in wave order (deterministic),
//     converted and stored as whole row segments.
//
// Rows past M / N, stages past K and stages past the wave's run read as zero
// codes with zero scale codes (out-of-range buffer offsets), which add
// exactly +0; a scale dword of a step past K is written as 0 because a
// row's 16-byte scale load can run into the next row there.
#pragma once

#include <utility>

#include "mx_tile.hpp"

namespace mxg {

template <int F, int MT, int NT, int KW>
struct SkinnyGeom {
    static constexpr int BM = 32 * MT, BN = 32 * NT;      // workgroup tile
    static constexpr int W = 64;                           // row bytes per stage
    static constexpr int ROWS = BM + BN;                   // A rows then B rows
    static constexpr int CHUNK = 160, GROUP = 4 * CHUNK;   // padded layout (as mx_tile.hpp)
    static constexpr int SLOT = ROWS / 8 * GROUP;          // one stage of one wave
    static constexpr int LC = ROWS / 16;                   // 16-row loads per stage
    static constexpr int P = F == FMT_FP4 ? 4 : 8;         // stages per scale period
    // 64-row scale loads per period: A rows, then B rows from row SB0, so
    // that no load mixes the two operands (its buffer must be uniform)
    static constexpr int SJA = cdiv_c(BM, 64), SJB = cdiv_c(BN, 64);
    static constexpr int SJ = SJA + SJB;
    static constexpr int SB0 = 64 * SJA;
    static constexpr int SROWS = 64 * SJ;
    static constexpr int SCB = SROWS * 16;                 // one period's codes, [dword][row]
    static constexpr int WAVE_LDS = 2 * SLOT + 2 * SCB;
    static constexpr int BYTES = KW * WAVE_LDS;
    static constexpr int RED_RS = BN + 4;                  // reduction row stride (floats)
    static_assert(KW * BM * RED_RS * 4 <= BYTES, "reduction tile must fit the wave regions");
    static_assert(BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
    __device__ static constexpr int code_off(int row, int c)
    {
        return (row >> 3) * GROUP + c * CHUNK + (row & 7) * 16;
    }
};

template <int F, int MT, int NT, int KW, int G, int OUT>
__global__ __launch_bounds__(64 * KW)
void mx_gemm_skinny(GemmArgs p)
{
    using SG = SkinnyGeom<F, MT, NT, KW>;
    static_assert(G >= 2 && SG::P % G == 0, "staging depth must divide the scale period");
    static_assert((G - 1) * SG::LC + SG::SJ < 64, "outstanding loads must fit the vmcnt field");
    __shared__ __attribute__((aligned(1024))) char smem[SG::BYTES];

    const int lane = threadIdx.x & 63;
    const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 31, g = lane >> 5;
    const int m0 = blockIdx.y * SG::BM, n0 = blockIdx.x * SG::BN;
    const int mrows = min(SG::BM, p.M - m0);
    const int nrows = min(SG::BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (size_t)m0 * p.row_bytes, mrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (size_t)n0 * p.row_bytes, nrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(p.sa + (size_t)m0 * p.srow_bytes, mrows * p.srow_bytes);
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(p.sb + (size_t)n0 * p.srow_bytes, nrows * p.srow_bytes);

    // this wave's run: periods [q0, q1) of the NP periods of K
    const int T = (int)(p.row_bytes / SG::W);
    const int NP = (T + SG::P - 1) / SG::P;
    const int q0 = (int)((long long)NP * kw / KW), q1 = (int)((long long)NP * (kw + 1) / KW);
    const int s0 = q0 * SG::P, s1 = min(q1 * SG::P, T);   // stages [s0, s1) are live
    char *wl = smem + kw * SG::WAVE_LDS;

    // ---- code loads: 16-row block j of [A rows | B rows]; lane l holds row
    // l/4, chunk l%4
    const unsigned lrow = (unsigned)(lane >> 2), lchunk = (unsigned)(lane & 3);
    const unsigned vload = lrow * p.row_bytes + 16u * lchunk;
    const int vwrite = SG::code_off(lrow, lchunk);
    u4v stg[G][SG::LC];
    auto load_stage = [&](u4v (&dst)[SG::LC], int t) {
        const unsigned kadd = (t >= s0 && t < s1) ? (unsigned)t * SG::W : kOutOfRange;
#pragma unroll
        for (int j = 0; j < SG::LC; ++j) {
            constexpr int AB = SG::BM / 16;
            const bool isa = j < AB;
            const unsigned qrow = 16u * (unsigned)(isa ? j : j - AB);
            dst[j] = load16<CPOL_NONE>(isa ? ra : rb, vload + qrow * p.row_bytes + kadd);
        }
    };
    // A stage past the run is not loaded (the load would move no data but
    // still cost address and return cycles); its staging set is zeroed, so
    // the stage adds exactly +0.
    auto fill_stage = [&](u4v (&set)[SG::LC], int t) {
        if (t < s1) {
            load_stage(set, t);
        } else {
#pragma unroll
            for (int j = 0; j < SG::LC; ++j)
                set[j] = u4v{0u, 0u, 0u, 0u};
        }
    };
    // store stage tw from a staging set into slot tw & 1, refill the set
    // with stage tl
    auto cycle = [&](u4v (&set)[SG::LC], int tw, int tl) {
        char *slot = wl + (tw & 1) * SG::SLOT;
#pragma unroll
        for (int j = 0; j < SG::LC; ++j)
            *reinterpret_cast<u4v *>(slot + j * 2 * SG::GROUP + vwrite) = set[j];
        fill_stage(set, tl);
    };

    // ---- scale codes of period q: lane l of job i holds A row 64i + l
    // (i < SJA) or B row 64(i - SJA) + l (16 bytes = four 128-K steps);
    // rows past the tile read as zeros (out of the buffer's range)
    u4v sstg[SG::SJ];
    auto scale_load = [&](int q) {
        const bool live = q >= q0 && q < q1;
#pragma unroll
        for (int i = 0; i < SG::SJ; ++i) {
            const bool isa = i < SG::SJA;
            const int row = 64 * (isa ? i : i - SG::SJA) + lane;
            const unsigned off = live ? (unsigned)row * p.srow_bytes + 16u * (unsigned)q : kOutOfRange;
            sstg[i] = load16<CPOL_NONE>(isa ? rsa : rsb, off);
        }
    };
    auto scale_write = [&](int q) {
        char *buf = wl + 2 * SG::SLOT + (q & 1) * SG::SCB;
#pragma unroll
        for (int i = 0; i < SG::SJ; ++i) {
            const int row = 64 * i + lane;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                *reinterpret_cast<unsigned *>(buf + d * SG::SROWS * 4 + row * 4) =
                    4 * q + d < p.nsteps ? sstg[i][d] : 0u;
        }
    };

    // ---- fragment reads: A tile i rows 32i + r, B tile j rows BM + 32j + r,
    // chunk 2h + g
    const int a_lane = SG::code_off(r, g);
    const int b_lane = SG::code_off(SG::BM + r, g);
    auto read = [&](TileRegs<MT, NT> &R, int t) {
        const char *slot = wl + (t & 1) * SG::SLOT;
        const char *sc = wl + 2 * SG::SLOT + ((t / SG::P) & 1) * SG::SCB +
                         (F == FMT_FP4 ? t % 4 : (t % 8) / 2) * SG::SROWS * 4;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                R.a[i][h] = *reinterpret_cast<const u4v *>(slot + a_lane + 4 * SG::GROUP * i + 2 * SG::CHUNK * h);
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                R.b[j][h] = *reinterpret_cast<const u4v *>(slot + b_lane + 4 * SG::GROUP * j + 2 * SG::CHUNK * h);
#pragma unroll
        for (int i = 0; i < MT; ++i)
            R.sa[i] = *reinterpret_cast<const unsigned *>(sc + 4 * (r + 32 * i));
#pragma unroll
        for (int j = 0; j < NT; ++j)
            R.sb[j] = *reinterpret_cast<const unsigned *>(sc + 4 * (SG::SB0 + r + 32 * j));
    };

    v16f acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.f;

    auto compute = [&](const TileRegs<MT, NT> &R, int t) {
        if constexpr (F == FMT_FP4) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const unsigned sh = 8u * (2 * s + g);
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        const u4v bx = R.b[j][s], ay = R.a[i][s];
                        const v8i x = {(int)bx.x, (int)bx.y, (int)bx.z, (int)bx.w, 0, 0, 0, 0};
                        const v8i y = {(int)ay.x, (int)ay.y, (int)ay.z, (int)ay.w, 0, 0, 0, 0};
                        acc[i][j] = mfma32<F>(x, R.sb[j] >> sh, y, R.sa[i] >> sh, acc[i][j]);
                    }
            }
        } else {
            const unsigned sh = 8u * (2 * (t & 1) + g);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const u4v b0 = R.b[j][0], b1 = R.b[j][1], a0 = R.a[i][0], a1 = R.a[i][1];
                    const v8i x = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                                   (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                    const v8i y = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                   (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    acc[i][j] = mfma32<F>(x, R.sb[j] >> sh, y, R.sa[i] >> sh, acc[i][j]);
                }
        }
    };

    if (q0 < q1) {
        TileRegs<MT, NT> R[2];
        // prologue: stages s0 .. s0+G-1 into the ring and scale period q0,
        // all landed; period q0 stored and q0+1 staged; stages s0, s0+1
        // stored (their sets reloaded with s0+G, s0+G+1); stage s0's
        // fragments read
        // All first loads go out together (one memory round trip, not two).
#pragma unroll
        for (int i = 0; i < G; ++i)
            fill_stage(stg[i], s0 + i);
        scale_load(q0);
        wait_vm<0>();
        scale_write(q0);
        if (q0 + 1 < q1)
            scale_load(q0 + 1);
        cycle(stg[0], s0, s0 + G);
        cycle(stg[1 % G], s0 + 1, s0 + G + 1);
        read(R[0], s0);

        // Iteration t (u = t - s0 mod P): stage t+2's loads have landed
        // (everything issued before them has: the wait leaves only the
        // G-1 later stages, and possibly some scale loads, outstanding);
        // in the second iteration of a period the next period's scale codes
        // are stored and the one after is staged; stage t+2 is stored and
        // its set refilled with stage t+G+2; stage t+1's fragments are read
        // and stage t's MFMAs run.
        // Near the end of the run fewer loads follow the ones waited for,
        // so the waits there drain everything.
        auto iteration = [&](auto uc, int t) {
            constexpr int u = decltype(uc)::value;
            __builtin_amdgcn_sched_barrier(0);
            const bool full = t + G + 1 < s1;
            if constexpr (u == 1) {
                if (full)
                    wait_vm<(G - 1) * SG::LC>();
                else
                    wait_vm<0>();
                scale_write(t / SG::P + 1);
                if (t / SG::P + 2 < q1)
                    scale_load(t / SG::P + 2);
            }
            if (full)
                wait_vm<(G - 1) * SG::LC>();
            else
                wait_vm<0>();
            cycle(stg[(u + 2) % G], t + 2, t + G + 2);
            read(R[(u + 1) & 1], t + 1);
            compute(R[u & 1], t);
            __builtin_amdgcn_sched_barrier(0);
        };
        for (int t0 = s0; t0 < q1 * SG::P; t0 += SG::P)
            static_for<SG::P>([&](auto uc) { iteration(uc, t0 + decltype(uc)::value); });
    }
    wait_vm<0>();

    // ---- split-K reduction in LDS (fixed wave order), 16-bit or FP32 store
    __syncthreads();   // every wave is done with its region
    float *red = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const v4f q = {acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2],
                               acc[i][j][4 * v + 3]};
                *reinterpret_cast<v4f *>(&red[(kw * SG::BM + 32 * i + r) * SG::RED_RS + 32 * j + 8 * v + 4 * g]) = q;
            }
    __syncthreads();
    constexpr int NQ = SG::BM * SG::BN / 4;   // 4-column groups of the tile
    const bool vec_ok = (p.N & 3) == 0;
    for (int qi = threadIdx.x; qi < NQ; qi += 64 * KW) {
        const int row = qi / (SG::BN / 4), c4 = qi % (SG::BN / 4);
        v4f sum = *reinterpret_cast<const v4f *>(&red[row * SG::RED_RS + 4 * c4]);
#pragma unroll
        for (int w = 1; w < KW; ++w)
            sum += *reinterpret_cast<const v4f *>(&red[(w * SG::BM + row) * SG::RED_RS + 4 * c4]);
        const int m = m0 + row, n = n0 + 4 * c4;
        if (m < p.M && n < p.N)
            store4<OUT>(p.c, p.N, m, n, sum, vec_ok && n + 3 < p.N);
    }
}

}  // namespace mxg
