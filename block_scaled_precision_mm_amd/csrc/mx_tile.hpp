// mx_tile.hpp -- NT MX block-scaled GEMM for many-row products (the
// MFMA-bound shapes), gfx950.
//
// Instruction.  v_mfma_scale_f32_32x32x64_f8f6f4: a 32x64 tile times a 64x32
// tile into a 32x32 FP32 accumulator (16 registers per lane), one E8M0 code
// per 32 K values applied in the instruction.  Measured on MI355X it issues
// every 33.6 clocks for E2M1 (17% more work per clock than the 16x16x128
// form) and every 64 clocks for E4M3.  Lane l = 32*g + r (r = l & 31):
//   * supplies row r of its operand tile;
//   * E2M1: its 16 bytes are K [32g, 32g+32) of the 64-deep sub-step;
//   * E4M3: its 32 bytes are K [16g, 16g+16) then K [32+16g, 32+16g+16);
//   * its scale register's byte 0 is the code of block g of row r;
//   * accumulator register 4v+e holds D[8v + 4g + e][r], D = X * Y^T for
//     the instruction's operands X, Y.
// The kernel passes B rows as X and A rows as Y, so lane (r, g) holds
// C[m0 + r][n0 + 8v + 4g + e]: four runs of four consecutive columns.
//
// Stages.  One stage is 64 bytes of every tile row: 128 K values of E2M1
// (two MFMA sub-steps) or 64 of E4M3 (one sub-step), so both formats share
// the loader and the LDS layout.  In either format chunk 2h + g (16 bytes)
// of a row's stage is what lane (r, g) needs for half h.
//
// Data path (measured on MI355X, which settled the design):
//   * global -> registers with 16-byte loads in which every four
//     consecutive lanes read one row's 64 bytes (as cheap per byte as a
//     contiguous load), then registers -> LDS with 16-byte stores.  Direct
//     global-to-LDS loads were tried first: they fix the LDS layout to the
//     load's lane order, which makes the fragment reads bank-conflicted,
//     and their load cost grows with every row touched;
//   * LDS layout: rows in groups of 8, chunk-major inside a group with a
//     padded chunk stride, so a fragment read (8 consecutive lanes = 8 rows
//     of one chunk) and a staging store both run at full LDS rate;
//   * scale codes: 16 bytes per row (four 128-K steps) fetched once per
//     period of P stages and stored transposed ([step][row] dwords), so a
//     stage's scale read is one contiguous dword per lane.
//
// Waves.  Four waves in 2 x 2, each owning a (32*MT) x (32*NT) part of the
// (64*MT) x (64*NT) workgroup tile; at MT = NT = 4 the 256 accumulator
// registers per lane fill the accumulation register file.
//
// Pipeline (iteration t computes stage t).  Two LDS code slots and two
// register staging sets: in iteration t the wave stores stage t+2 from its
// staging set into the slot stage t used, reloads that set with stage t+4,
// reads stage t+1's fragments into the idle fragment set and runs stage t's
// MFMAs.  A load therefore has two iterations to land.  Each iteration
// starts with one wait (everything issued two iterations ago has landed)
// and one barrier; its body has no branch, and sched_group_barrier
// interleaves MFMAs with the stores, loads and reads.  The loop runs whole
// periods; stages past K (and rows past M or N) read as zero codes with zero
// scale codes and add exactly +0.
//
// Epilogue.  FP32 output is stored straight from the accumulators.  16-bit
// output is converted, staged through LDS and written as whole row segments
// (one store instruction covers 4 to 8 rows instead of 32).
//
// Tile order.  MI355X deals workgroups round-robin to its 8 XCDs, each with
// its own L2.  The linear workgroup index is remapped so that consecutive
// tiles of a band of 8 tile rows land on the same XCD, where they share A
// and B traffic in that XCD's L2.
#pragma once

#include <utility>

#include "mx_epilogue.hpp"
#include "mx_group.hpp"
#include "mx_splitk.hpp"
#include "mx_sync.hpp"

namespace mxg {

template <int F, int MT, int NT>
struct TileGeom {
    static constexpr int BM = 64 * MT, BN = 64 * NT;    // workgroup tile
    static constexpr int W = 64;                         // row bytes per stage
    static constexpr int ROWS = BM + BN;                 // A rows then B rows
    // code slot layout: rows in groups of 8; in a group, chunk c (16 bytes of
    // each of the 8 rows, 128 contiguous bytes) starts at c * CHUNK; the 32
    // bytes of padding per chunk put consecutive groups' chunks on
    // complementary LDS bank halves (measured on MI355X: fragment reads at
    // ~92% and stores at 100% of the contiguous rate, against 75% and 40%
    // without padding)
    static constexpr int CHUNK = 160, GROUP = 4 * CHUNK;
    static constexpr int CODE = ROWS / 8 * GROUP;        // one code slot
    static constexpr int LC = ROWS / 16 / 4;             // 16-row code loads per wave per stage
    // scale codes: 16 bytes per row per period of P stages (4 steps of 128 K)
    static constexpr int P = F == FMT_FP4 ? 4 : 8;
    static constexpr int SJOBS = cdiv_c(ROWS, 64);       // 64-row scale loads per period
    static constexpr int LS = cdiv_c(SJOBS, 4);          // per wave (jobs past SJOBS load nothing)
    static constexpr int SROWS = 64 * 4 * LS;            // scale rows incl. padding
    static constexpr int SCB = SROWS * 16;               // one scale buffer: [dword][row]
    static constexpr int SC_OFF = 2 * CODE;
    static constexpr int BYTES = SC_OFF + 2 * SCB;
    static_assert((BM / 16) % 4 == 0 && (BN / 16) % 4 == 0, "code loads must spread evenly over 4 waves");
    // byte offset of 16-byte chunk c (0..3) of tile row `row` in a code slot
    __device__ static constexpr int code_off(int row, int c)
    {
        return (row >> 3) * GROUP + c * CHUNK + (row & 7) * 16;
    }
};

// Linear workgroup index -> position in tile order: workgroups b, b + 8,
// b + 16, ... (one XCD) get consecutive positions.
__device__ __forceinline__ int xcd_remap(int b, int total)
{
    return (total & 7) == 0 ? (b & 7) * (total >> 3) + (b >> 3) : b;
}

// Remap the linear workgroup index to an output tile (see "Tile order").
__device__ __forceinline__ void tile_of(int b, int nbm, int nbn, int &tm, int &tn)
{
    const int pid = xcd_remap(b, nbm * nbn);
    constexpr int GM = 8;
    const int per_group = GM * nbn;
    const int grp = pid / per_group;
    const int first = grp * GM;
    const int gsz = min(nbm - first, GM);
    const int in = pid - grp * per_group;
    tm = first + in % gsz;
    tn = in / gsz;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <class Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The memory operations of one iteration, in program order: at a period
// start the scale-code writes (4 per scale load) and loads; then, per code
// load, the LDS write that empties a staging register and the load that
// refills it; then the fragment and scale reads.  sched_group_barrier masks:
// 0x200 LDS write, 0x020 vector-memory read, 0x100 LDS read.
template <bool PERIOD, int LS, int LC, int NREAD>
struct OpSeq {
    static constexpr int NS = PERIOD ? 5 * LS : 0;
    static constexpr int N = NS + 2 * LC + NREAD;
    static constexpr int mask(int k)
    {
        return k < NS ? (k < 4 * LS ? 0x200 : 0x020)
                      : (k - NS < 2 * LC ? ((k - NS) % 2 == 0 ? 0x200 : 0x020) : 0x100);
    }
};

// Interleave request for one stage: NM MFMA slots; slot K holds one MFMA and
// then its share of the memory operations, in their program order.  The
// operations all go into the first NMEM slots, so the reads of the next
// stage have the rest of the stage to land.
template <int NM, int NMEM, class Ops>
__device__ __forceinline__ void sched_stage()
{
    static_for<NM>([&](auto kc) {
        constexpr int K = decltype(kc)::value;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (K < NMEM) {
            constexpr int k0 = Ops::N * K / NMEM, k1 = Ops::N * (K + 1) / NMEM;
            static_for<k1 - k0>([&](auto ic) {
                constexpr int k = k0 + decltype(ic)::value;
                __builtin_amdgcn_sched_group_barrier(Ops::mask(k), 1, 0);
            });
        }
    });
}

typedef float v16f __attribute__((ext_vector_type(16)));

template <int F>
__device__ __forceinline__ v16f mfma32(v8i x, unsigned sx, v8i y, unsigned sy, v16f acc)
{
    constexpr int c = FmtTraits<F>::mfma_code;
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc, c, c, 0, (int)sx, 0, (int)sy);
}

template <int MT, int NT>
struct TileRegs {
    u4v a[MT][2], b[NT][2];   // [tile][16-byte half]: E2M1 sub-step h / E4M3 half h
    unsigned sa[MT], sb[NT];  // 128-K scale dwords of the lane's rows
};

// One workgroup per CU: the accumulators of the largest tiles need the
// whole register file of a SIMD (the LDS footprint alone would let the
// compiler aim for two).
template <int F, int MT, int NT, int OUT, int GRP = 0, int EPI = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, MT * NT > 4 ? 1 : 2)))
void mx_gemm_tile(GemmArgs p)
{
    static_assert(EPI || OUT <= OUT_F32, "MX output kinds need the fused epilogue");
    using G = TileGeom<F, MT, NT>;
    static_assert(G::BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
    __shared__ __attribute__((aligned(1024))) char smem[G::BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 31, g = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;

    const int nbn = (p.N + G::BN - 1) / G::BN;
    int tm, tn;
    if constexpr (GRP) {
        // grouped product: a unit is one tile; a group's tiles in M-fastest
        // order, so the workgroups of one XCD share the group's B columns
        int grp, local, row0, rows;
        if (!find_group(p.offs, p.groups, p.M, xcd_remap(blockIdx.x, gridDim.x), G::BM, nbn, grp,
                        local, row0, rows))
            return;
        select_group<OUT>(p, grp, row0, rows);
        const int nbm = (rows + G::BM - 1) / G::BM;
        tm = local % nbm;
        tn = local / nbm;
    } else {
        tile_of(blockIdx.x, (p.M + G::BM - 1) / G::BM, nbn, tm, tn);
        // split-K: this workgroup's K part (whole periods of four steps)
        if constexpr (!EPI)
            select_split<F>(p, 4);
    }
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int mrows = min(G::BM, p.M - m0);
    const int nrows = min(G::BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.a + (size_t)m0 * p.row_bytes, part_range(mrows, p.row_bytes, p.kbytes));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.b + (size_t)n0 * p.row_bytes, part_range(nrows, p.row_bytes, p.kbytes));
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(p.sa + (size_t)m0 * p.srow_bytes, part_range(mrows, p.srow_bytes, 4u * p.nsteps));
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(p.sb + (size_t)n0 * p.srow_bytes, part_range(nrows, p.srow_bytes, 4u * p.nsteps));

    const int T = (int)(p.kbytes / G::W);   // stages

    // ---- code loads: job j of this wave is 16-row block q = wave + 4j of
    // [A blocks | B blocks]; lane l holds row l/4, chunk l%4 of the block
    const unsigned lrow = (unsigned)(lane >> 2), lchunk = (unsigned)(lane & 3);
    const unsigned vload = lrow * p.row_bytes + 16u * lchunk;
    const int vwrite = G::code_off(lrow, lchunk);   // within a 16-row block (2 groups)
    u4v stg[2][G::LC];                               // staging sets (stage parity)

    auto load_one = [&](int j, int t) {
        const int q = wave + 4 * j;
        const bool isa = q < G::BM / 16;
        const unsigned qrow = 16u * (unsigned)(isa ? q : q - G::BM / 16);
        const unsigned kadd = t < T ? (unsigned)t * G::W : kOutOfRange;
        return load16<CPOL_NONE>(isa ? ra : rb, vload + qrow * p.row_bytes + kadd);
    };
    auto write_one = [&](int j, const u4v &v, int t) {
        const int q = wave + 4 * j;   // block of [A | B]: 16 rows = 2 groups
        *reinterpret_cast<u4v *>(smem + (t & 1) * G::CODE + q * 2 * G::GROUP + vwrite) = v;
    };
    auto code_load = [&](u4v (&dst)[G::LC], int t) {
#pragma unroll
        for (int j = 0; j < G::LC; ++j)
            dst[j] = load_one(j, t);
    };
    auto code_write = [&](const u4v (&src)[G::LC], int t) {
#pragma unroll
        for (int j = 0; j < G::LC; ++j)
            write_one(j, src[j], t);
    };
    // write stage tw from a staging set, refilling each register with stage tl
    auto code_cycle = [&](u4v (&set)[G::LC], int tw, int tl) {
#pragma unroll
        for (int j = 0; j < G::LC; ++j) {
            write_one(j, set[j], tw);
            set[j] = load_one(j, tl);
        }
    };

    // ---- scale codes: job i of this wave is 64-row block q = wave + 4i of
    // [A rows | B rows]; lane l holds row l's 16 bytes of the period
    u4v sstg[G::LS];
    auto scale_load = [&](int period) {
        const bool live = period * G::P < T;
#pragma unroll
        for (int i = 0; i < G::LS; ++i) {
            const int q = wave + 4 * i;
            const int row = q * 64 + lane;
            const bool isa = q * 64 < G::BM;   // A and B rows never share a 64-row job
            const unsigned off = (live && q < G::SJOBS)
                                     ? (unsigned)(isa ? row : row - G::BM) * p.srow_bytes +
                                           16u * (unsigned)period
                                     : kOutOfRange;
            sstg[i] = load16<CPOL_NONE>(isa ? rsa : rsb, off);
        }
    };
    // Dword d of a period is 128-K step 4*period + d.  Steps past K are
    // written as zero codes: a row's 16-byte load can run into the next
    // row's codes there, and a NaN code would poison the +0 of the padding
    // stages.
    auto scale_write = [&](int period) {
        char *buf = smem + G::SC_OFF + (period & 1) * G::SCB;
#pragma unroll
        for (int i = 0; i < G::LS; ++i) {
            const int row = (wave + 4 * i) * 64 + lane;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                *reinterpret_cast<unsigned *>(buf + d * G::SROWS * 4 + row * 4) =
                    4 * period + d < p.nsteps ? sstg[i][d] : 0u;
        }
    };

    // ---- fragment reads: lane (r, g) reads rows wm*32*MT + 32i + r (A) and
    // wn*32*NT + 32j + r (B), chunk 2h + g
    const int arow = wm * 32 * MT + r, brow = G::BM + wn * 32 * NT + r;
    const int a_lane = G::code_off(arow, g);
    const int b_lane = G::code_off(brow, g);
    auto read = [&](TileRegs<MT, NT> &R, int t) {
        const char *slot = smem + (t & 1) * G::CODE;
        const char *sc = smem + G::SC_OFF + ((t / G::P) & 1) * G::SCB +
                         (F == FMT_FP4 ? t % 4 : (t % 8) / 2) * G::SROWS * 4;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                R.a[i][h] = *reinterpret_cast<const u4v *>(slot + a_lane + 4 * G::GROUP * i + 2 * G::CHUNK * h);
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                R.b[j][h] = *reinterpret_cast<const u4v *>(slot + b_lane + 4 * G::GROUP * j + 2 * G::CHUNK * h);
#pragma unroll
        for (int i = 0; i < MT; ++i)
            R.sa[i] = *reinterpret_cast<const unsigned *>(sc + 4 * (arow + 32 * i));
#pragma unroll
        for (int j = 0; j < NT; ++j)
            R.sb[j] = *reinterpret_cast<const unsigned *>(sc + 4 * (brow + 32 * j));
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
                const unsigned sh = 8u * (2 * s + g);   // block 2s+g of the 128-K dword
                unsigned xs[NT], ys[MT];
#pragma unroll
                for (int j = 0; j < NT; ++j) xs[j] = R.sb[j] >> sh;
#pragma unroll
                for (int i = 0; i < MT; ++i) ys[i] = R.sa[i] >> sh;
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        const u4v bx = R.b[j][s], ay = R.a[i][s];
                        const v8i x = {(int)bx.x, (int)bx.y, (int)bx.z, (int)bx.w, 0, 0, 0, 0};
                        const v8i y = {(int)ay.x, (int)ay.y, (int)ay.z, (int)ay.w, 0, 0, 0, 0};
                        acc[i][j] = mfma32<F>(x, xs[j], y, ys[i], acc[i][j]);
                    }
            }
        } else {
            const unsigned sh = 8u * (2 * (t & 1) + g);   // this 64-K stage's half of the dword
            unsigned xs[NT], ys[MT];
#pragma unroll
            for (int j = 0; j < NT; ++j) xs[j] = R.sb[j] >> sh;
#pragma unroll
            for (int i = 0; i < MT; ++i) ys[i] = R.sa[i] >> sh;
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const u4v b0 = R.b[j][0], b1 = R.b[j][1], a0 = R.a[i][0], a1 = R.a[i][1];
                    const v8i x = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                                   (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                    const v8i y = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                   (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    acc[i][j] = mfma32<F>(x, xs[j], y, ys[i], acc[i][j]);
                }
        }
    };

    constexpr int NM = (F == FMT_FP4 ? 2 : 1) * MT * NT;   // MFMAs per stage
    constexpr int NMEM = NM * 3 / 4;
    constexpr int NREAD = 3 * (MT + NT);                   // fragment and scale reads
    TileRegs<MT, NT> R[2];

    // prologue: scales of periods 0 (written) and 1 (staged); code stages 0
    // and 1 written to the two slots; stages 2 and 3 staged
    scale_load(0);
    wait_vm<0>();
    scale_write(0);
    scale_load(1);
    code_load(stg[0], 0);
    code_load(stg[1], 1);
    wait_vm<0>();
    code_write(stg[0], 0);
    code_write(stg[1], 1);
    code_load(stg[0], 2);
    code_load(stg[1], 3);
    block_barrier();
    read(R[0], 0);

    // Iteration t (u = t mod P): everything issued two or more iterations
    // ago has landed; write stage t+2 from its staging set into the slot
    // stage t used and reload that set with stage t+4; in the second
    // iteration of a period also write the next period's scale codes (first
    // read P-2 iterations later) and stage the one after; read stage t+1's
    // fragments; run stage t's MFMAs.
    auto iteration = [&](auto uc, int t) {
        constexpr int u = decltype(uc)::value;
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<G::LC + (u == 2 ? G::LS : 0)>();
        block_barrier();
        if constexpr (u == 1) {
            scale_write(t / G::P + 1);
            scale_load(t / G::P + 2);
        }
        code_cycle(stg[u & 1], t + 2, t + 4);
        read(R[(u + 1) & 1], t + 1);
        compute(R[u & 1], t);
        sched_stage<NM, NMEM, OpSeq<u == 1, G::LS, G::LC, NREAD>>();
        __builtin_amdgcn_sched_barrier(0);
    };
    // Whole periods without branches.  Stages past K (at most P-1 of them)
    // run on zero codes and zero scale codes, which add exactly +0.
    for (int t0 = 0; t0 < T; t0 += G::P)
        static_for<G::P>([&](auto uc) { iteration(uc, t0 + decltype(uc)::value); });
    wait_vm<0>();

    // split-K: the K parts of this tile are summed by the last one to finish
    if constexpr (!GRP && !EPI) {
        if (p.splits > 1) {
            auto get = [&](int j) {
                const v16f &a = acc[j / (4 * NT)][(j / 4) % NT];
                const int v = j % 4;
                return v4f{a[4 * v], a[4 * v + 1], a[4 * v + 2], a[4 * v + 3]};
            };
            auto set = [&](int j, v4f x) {
                v16f &a = acc[j / (4 * NT)][(j / 4) % NT];
                const int v = j % 4;
                a[4 * v] = x[0];
                a[4 * v + 1] = x[1];
                a[4 * v + 2] = x[2];
                a[4 * v + 3] = x[3];
            };
            if (!splitk_reduce<4 * MT * NT, 256>(p, (int)blockIdx.x, (int)threadIdx.x, get, set))
                return;
        }
    }

    if constexpr (OUT == OUT_F32) {
        // FP32 output (the unrounded accumulator): direct stores
        const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int m = m0 + arow + 32 * i;
            if (m >= p.M)
                continue;
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = n0 + wn * 32 * NT + 32 * j + 8 * v + 4 * g;
                    if (n < p.N) {
                        v4f q = {acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2],
                                 acc[i][j][4 * v + 3]};
                        if constexpr (EPI)
                            q = epilogue4(q, p, n);
                        store4<OUT>(p.c, p.N, m, n, q, vec_ok && n + 3 < p.N);
                    }
                }
        }
    } else {
        // 16-bit output goes through LDS: in the accumulator layout one store
        // instruction would touch 32 rows (32 cache lines); transposed, each
        // instruction writes whole row segments of the wave's tile.  Two
        // passes of half the wave's rows; each wave uses its own region of
        // the (now idle) code slots.
        constexpr int RS = 64 * NT + 16;            // region row stride (bytes, padded)
        constexpr int HR = 16 * MT;                  // rows per pass
        static_assert(4 * HR * RS <= 2 * G::CODE, "epilogue staging must fit the code slots");
        char *region = smem + wave * HR * RS;
        constexpr int LPR = 4 * NT;                  // lanes per row (16 bytes each)
        constexpr int RPI = 64 / LPR;                // rows per store instruction
        const int lr = lane / LPR, lc = lane % LPR;
        const int ncol = n0 + wn * 32 * NT + 8 * lc; // first of this lane's 8 columns
        const bool vec_ok = (p.N & 7) == 0 && ncol + 8 <= p.N;
        block_barrier();                             // every wave is done with the code slots
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int ii = 0; ii < MT / 2; ++ii) {
                const int i = hf * (MT / 2) + ii;
#pragma unroll
                for (int j = 0; j < NT; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        v4f y = {acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2],
                                 acc[i][j][4 * v + 3]};
                        if constexpr (EPI)
                            y = epilogue4(y, p, n0 + wn * 32 * NT + 32 * j + 8 * v + 4 * g);
                        unsigned short h[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if constexpr (OUT == OUT_F16)
                                h[e] = __builtin_bit_cast(unsigned short, (_Float16)y[e]);
                            else   // BF16, and the BF16 rounding before MX quantization
                                h[e] = __builtin_bit_cast(unsigned short, (__bf16)y[e]);
                        }
                        u2v w;
                        w.x = (unsigned)h[0] | ((unsigned)h[1] << 16);
                        w.y = (unsigned)h[2] | ((unsigned)h[3] << 16);
                        *reinterpret_cast<u2v *>(region + (32 * ii + r) * RS + (32 * j + 8 * v + 4 * g) * 2) = w;
                    }
            }
            // the wave's own LDS writes complete before its reads of them
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int k = 0; k < HR / RPI; ++k) {
                const int row = k * RPI + lr;
                const u4v q = *reinterpret_cast<const u4v *>(region + row * RS + 16 * lc);
                const int m = m0 + wm * 32 * MT + hf * HR + row;
                if constexpr (OUT == OUT_MX8 || OUT == OUT_MX4) {
                    // the four consecutive lanes lc = 4b .. 4b+3 hold one
                    // 32-column block of the row; N % 32 == 0, so a block is
                    // wholly inside or outside
                    constexpr int QF = OUT == OUT_MX4 ? FMT_FP4 : FMT_FP8;
                    const unsigned w4[4] = {q[0], q[1], q[2], q[3]};
                    const unsigned sc = block_scale_code<QF>(quad_max(amax_pairs(w4)));
                    unsigned code[QF == FMT_FP4 ? 1 : 2];
                    mx_codes<QF, 4>(w4, sc, code);
                    if (m < p.M && ncol < p.N) {
                        uint8_t *c8 = static_cast<uint8_t *>(p.c);
                        if constexpr (QF == FMT_FP4)
                            *reinterpret_cast<unsigned *>(c8 + (size_t)m * (p.N / 2) + ncol / 2) = code[0];
                        else
                            *reinterpret_cast<u2v *>(c8 + (size_t)m * p.N + ncol) = u2v{code[0], code[1]};
                        if ((lc & 3) == 0)
                            p.c_scale[(size_t)m * (p.N / 32) + ncol / 32] = (uint8_t)sc;
                    }
                } else if (m < p.M) {
                    unsigned short *dst = reinterpret_cast<unsigned short *>(p.c) + (size_t)m * p.N + ncol;
                    if (vec_ok) {
                        *reinterpret_cast<u4v *>(dst) = q;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (ncol + e < p.N)
                                dst[e] = (unsigned short)(q[e / 2] >> (16 * (e % 2)));
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next pass writes
        }
    }
}

}  // namespace mxg
