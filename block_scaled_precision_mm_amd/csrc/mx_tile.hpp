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
// Super-stages.  The K loop advances 128 bytes of every tile row at a
// time: 256 K values of E2M1 (four MFMA sub-steps) or 128 of E4M3 (two).
// What decided the width, measured on MI355X at 8192^3 E2M1 with loads
// alone (every workgroup streaming its 256 + 256 rows from L2): 16-byte
// loads in which 8 lanes read one row's 128 contiguous bytes move the
// operands at 25.6 TB/s over the chip, against 15.2 TB/s when 4 lanes read
// 64 bytes of a row (each L1 request then covers half a cache line, and the
// number of requests in flight, not bytes, sets the rate); loads straight
// into LDS stream as fast as loads into registers (26.5 TB/s).  A copy of
// the loop whose loads touch no memory (out-of-range offsets: same LDS
// traffic and MFMAs) ran 8192^3 in 189-214 us against 270-298, and
// 256 x 28672 x 8192 E4M3 in 48 against 97: a super-stage's loads did not
// land within one super-stage of MFMA work.  LDS holds two 128-byte slots
// of the larger tiles; four 64-byte slots (three super-stages in flight)
// helped E4M3 and cost E2M1 5% at 8192^3 (the half-line loads), and were
// overtaken on every shape by two 128-byte slots with the split barrier
// below (E4M3 2048 x 4096 x 4096: 50.5 -> 41.0 us, 8192^3: 468 -> 437).
//
// Data path.  Global -> LDS directly (gfx950's 16-byte buffer load to LDS:
// no staging registers, no LDS store instructions).  A load instruction
// fills 1 KB of LDS in lane order: 8 rows x 128 bytes, lane l at 16*l, so
// lane l (row l/8 of its block, position p = l%8) fetches the row's chunk
// c = p ^ s(row): the lanes of a row still read its 128 contiguous bytes,
// and chunk c of row `row` sits at 128*row + 16*(c ^ s(row)).  With
// s(row) = (row >> 1) & 7, a fragment read (16 consecutive lanes = 16
// consecutive rows, one chunk) touches 16 different 16-byte bank groups of
// the 256 bytes the LDS banks cover.  Scale codes: 16 bytes per row per
// period of four 128-K steps, through registers, stored transposed
// ([step][row] dwords), so an MFMA's scale operand is one dword read plus a
// shift; the two sub-steps of a 128-K step share the dword (read once).
// The code slots and the scale buffers are separate LDS objects, so the
// compiler can tell a fragment read of one slot from the loads still
// landing in another.
//
// Pipeline (iteration u computes super-stage u; NS = 2 or 4 code slots).
// Sub-step h's fragments are read while sub-step h-1's MFMAs run, so by the
// last sub-step every fragment of slot u is in registers.  Two slots: at
// the last sub-step a barrier (every wave is done reading slot u), the
// loads of u+2 into slot u and at a period start the next period's scale
// codes written, under the first half of its MFMAs; then wait for
// super-stage u+1's loads, a second barrier (every wave's have landed),
// the scale loads of a later period, and super-stage u+1's first fragments
// read under the second half.  Issuing u+2's loads before waiting for u+1
// keeps a late super-stage from also delaying the next one's loads: with
// load latency L above the compute time T of an iteration, a loop that
// waits first runs at L per iteration, this one at (L + T) / 2
// (256 x 28672 x 8192: E2M1 55.5 -> 49.6 us, E4M3 91.5 -> 80.5).  Four
// slots (where a super-stage is little MFMA work and LDS allows: the
// 128 x 128 and 64 x 64 tiles): wait for u+1, one barrier, loads of u+4;
// a load has three iterations to land.  The loop runs whole periods;
// super-stages past K (and rows past M or N) load zero codes through
// out-of-range offsets and have zero scale codes, and add exactly +0.
//
// 16-bit operands (F = FMT_BF16 / FMT_F16: the dense NT product).  A
// v_mfma_f32_32x32x16 sub-step reads 32 bytes per row, lane half g 16 of
// them, as an E2M1 sub-step does, so the same super-stages, slots and
// pipeline run it; there are no scale codes to load, write or read.
//
// Waves.  Four waves in 2 x 2, each owning a (32*MT) x (32*NT) part of the
// (64*MT) x (64*NT) workgroup tile; at MT = NT = 4 the 256 accumulator
// registers per lane fill the accumulation register file.
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

template <int F, int MT, int NT, int NS = 2>
struct TileGeom {
    static constexpr int BM = 64 * MT, BN = 64 * NT;    // workgroup tile
    static constexpr int ROWS = BM + BN;                 // A rows then B rows
    static constexpr int SW = 128;                       // row bytes per super-stage
    static constexpr bool SCALED = FmtTraits<F>::scaled; // E8M0 codes (else 16-bit operands)
    // K values per super-stage: 256 (E2M1), 128 (E4M3), 64 (BF16 / FP16)
    static constexpr int KSS = SCALED ? SW * (F == FMT_FP4 ? 2 : 1) : SW / 2;
    // MFMA sub-steps per super-stage: 32x32x64 (MX) or 32x32x16 (16-bit)
    static constexpr int SUB = SCALED ? KSS / 64 : KSS / 16;
    static constexpr int SLOT = ROWS * SW;               // one code slot (unpadded, swizzled)
    static constexpr int RPL = 1024 / SW;                // rows per 1 KB load
    static constexpr int LPR = SW / 16;                  // lanes per row of a load
    static constexpr int LB = ROWS / RPL / 4;            // 1 KB loads per wave per super-stage
    // scale codes: 16 bytes per row per period of 4 steps (512 K)
    static constexpr int P = SCALED ? 512 / KSS : 2;     // super-stages per period
    static constexpr int SJOBS = cdiv_c(ROWS, 64);       // 64-row scale loads per period
    static constexpr int LS = SCALED ? cdiv_c(SJOBS, 4) : 0;   // per wave (jobs past SJOBS load nothing)
    static constexpr int SROWS = 64 * 4 * LS;            // scale rows incl. padding
    static constexpr int SCB = SROWS * 16;               // one scale buffer: [dword][row]
    static constexpr int BYTES = NS * SLOT + 2 * SCB;
    // A period's scale codes are staged in registers between their load and
    // their write to LDS; with loads in flight for NS-1 iterations they need
    // a lead of more than one period when a period is shorter than that,
    // and then two staging sets that alternate by period.
    static constexpr int SSETS = P >= NS - 1 ? 1 : 2;
    static constexpr int SLEAD = SSETS == 2 ? 3 : 2;     // periods from a period's load to its write
    // super-stages per turn of the loop: whole periods, whole rounds of the
    // NS code slots and (two staging sets) whole pairs of periods, so that
    // every index is known at compile time
    static constexpr int TURN = [] {
        const int per = SSETS * P;
        return per % NS == 0 ? per : (NS % per == 0 ? NS : per * NS);
    }();
    static_assert(NS == 2 || NS == 4, "two or four code slots");
    static_assert(P % 2 == 0, "a period covers whole pairs of code slots");
    static_assert((ROWS / RPL) % 4 == 0, "load blocks must spread evenly over 4 waves");
    static_assert(BM % (4 * RPL) == 0, "A and B rows never share a load block, and the first BM / (4 RPL) of a wave's are A's");
    static_assert(NS * LB + SLEAD * LS < 64, "outstanding loads must fit the vmcnt field");
    // byte offset of 16-byte chunk c of tile row `row` in a code slot: the
    // chunk's place XORed with the row so that the 16 rows of a fragment
    // read fall on 16 different 16-byte bank groups
    __device__ static constexpr int swz(int row) { return (row >> 1) & 7; }
    __device__ static constexpr int code_off(int row, int c) { return row * SW + 16 * (c ^ swz(row)); }
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

typedef float v16f __attribute__((ext_vector_type(16)));

// 16-bit operands: v_mfma_f32_32x32x16_{bf16,f16}, lane (r, g) holding 8 K
// values of row r (B rows as the first operand, A rows as the second)
typedef __bf16 tile_bf16x8 __attribute__((ext_vector_type(8)));
typedef short tile_s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 tile_f16x8 __attribute__((ext_vector_type(8)));
template <int F>
__device__ __forceinline__ v16f mfma16(const u4v &x, const u4v &y, v16f acc)
{
    if constexpr (F == FMT_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(tile_bf16x8, x),
                                                       __builtin_bit_cast(tile_bf16x8, y), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(tile_f16x8, x),
                                                      __builtin_bit_cast(tile_f16x8, y), acc, 0, 0, 0);
}

// SEL: the byte of each scale register that holds the lane's code
template <int F, int SEL = 0>
__device__ __forceinline__ v16f mfma32(v8i x, unsigned sx, v8i y, unsigned sy, v16f acc)
{
    constexpr int c = FmtTraits<F>::mfma_code;
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc, c, c, SEL, (int)sx, SEL, (int)sy);
}

// One sub-step's fragments of a wave's tile: the lane's 16 (E2M1) or 32
// (E4M3) bytes of each A and B subtile, and the step's scale dwords.
template <int F, int MT, int NT>
struct TileFrag {
    u4v a[MT][FmtTraits<F>::nvec], b[NT][FmtTraits<F>::nvec];
    unsigned sa[MT], sb[NT];
    __device__ void sa_from(const TileFrag &o)
    {
        for (int i = 0; i < MT; ++i) sa[i] = o.sa[i];
        for (int j = 0; j < NT; ++j) sb[j] = o.sb[j];
    }
};


// One workgroup per CU: the accumulators of the largest tiles need the
// whole register file of a SIMD (the LDS footprint alone would let the
// compiler aim for two).
// TA / TB (16-bit operands only): A is stored [K][M] / B is stored [K][N]
// (contiguous along M / N, the dense TN, TT and NN layouts); its part of a
// slot holds the super-stage's 64 K rows of the tile's BM / BN columns, and
// its fragments are read with gfx950's transposing LDS read (see
// read_kmajor below).
template <int F, int MT, int NT, int OUT, int GRP = 0, int EPI = 0, int NS = 2, int TB = 0, int TA = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, MT * NT > 4 ? 1 : 2)))
void mx_gemm_tile(GemmArgs p)
{
    static_assert(EPI || OUT <= OUT_F32, "MX output kinds need the fused epilogue");
    using G = TileGeom<F, MT, NT, NS>;
    static_assert(G::BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
    static_assert(!TB || (!G::SCALED && !GRP && !EPI && NT >= 2 && (NT & (NT - 1)) == 0),
                  "B stored [K][N]: 16-bit, plain, BN >= 128 and a power of two");
    static_assert(!TA || (!G::SCALED && !GRP && !EPI && MT >= 2 && (MT & (MT - 1)) == 0),
                  "A stored [K][M]: 16-bit, plain, BM >= 128 and a power of two");
    // The two code slots and the scale buffers are separate LDS objects: the
    // compiler then knows that a fragment read of one slot cannot touch what
    // a direct-to-LDS load still in flight writes into the other, and does
    // not wait for every outstanding load before each such read (with one
    // array it did, once per super-stage, which cost a full memory latency).
    __shared__ __attribute__((aligned(1024))) char slot0[G::SLOT];
    __shared__ __attribute__((aligned(1024))) char slot1[G::SLOT];
    __shared__ __attribute__((aligned(1024))) char slot2[NS == 4 ? G::SLOT : 16];
    __shared__ __attribute__((aligned(1024))) char slot3[NS == 4 ? G::SLOT : 16];
    __shared__ __attribute__((aligned(1024))) char sbuf[G::SCALED ? 2 * G::SCB : 16];

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
        if constexpr (!EPI && G::SCALED)
            select_split<F>(p, 4);
    }
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int mrows = min(G::BM, p.M - m0);
    const int nrows = min(G::BN, p.N - n0);
    // (A stored [K][M]: the whole operand, as B stored [K][N] below)
    const __amdgpu_buffer_rsrc_t ra =
        TA ? make_rsrc(p.a, p.kbytes * (unsigned)p.M)
           : make_rsrc(p.a + (size_t)m0 * p.row_bytes, part_range(mrows, p.row_bytes, p.kbytes));
    // (B stored [K][N]: the whole operand, K rows of N columns; rows past K
    // read zeros)
    const __amdgpu_buffer_rsrc_t rb =
        TB ? make_rsrc(p.b, p.kbytes * (unsigned)p.N)
           : make_rsrc(p.b + (size_t)n0 * p.row_bytes, part_range(nrows, p.row_bytes, p.kbytes));
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(p.sa + (size_t)m0 * p.srow_bytes, part_range(mrows, p.srow_bytes, 4u * p.nsteps));
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(p.sb + (size_t)n0 * p.srow_bytes, part_range(nrows, p.srow_bytes, 4u * p.nsteps));

    // super-stages of this workgroup's K range, rounded up to whole periods
    const int T2 = (int)((p.kbytes + G::SW - 1) / G::SW);
    const int U = (T2 + G::P - 1) / G::P * G::P;

    // ---- code loads, straight into LDS: load j of this wave is 1 KB block
    // q = wave + 4j of [A rows | B rows] (RPL rows x SW bytes); lane l takes
    // row RPL*q + l/LPR and the chunk whose swizzled place is position l%LPR.
    // voff: the lane's byte offset of its chunk from the start of the tile's
    // first row of its operand; vtail: the same for the last super-stage
    // when it is partial (kbytes not a multiple of SW), kOutOfRange for the
    // chunks past the end
    const int lrow = lane / G::LPR;
    const unsigned kb = p.kbytes, ktail = kb % G::SW;
    unsigned voff[G::LB], vtail[G::LB];
    bool vla[G::LB];
    // B stored [K][N]: a 1 KB block holds KPB whole K rows of the tile's BN
    // columns (BCH 16-byte chunks each); chunk c of K row k sits at place
    // c ^ 4 (k mod 4), so that the eight K rows and four chunks of one
    // transposing read fall on different bank groups
    constexpr int BCH = G::BN / 8, KPB = 1024 / (2 * G::BN);
    constexpr int ACH = G::BM / 8, KPA = 1024 / (2 * G::BM);   // (A stored [K][M]: the same)
#pragma unroll
    for (int j = 0; j < G::LB; ++j) {
        const int q = wave + 4 * j;
        const int row = G::RPL * q + lrow;                    // tile row in [A | B]
        const unsigned cb = 16u * (unsigned)((lane % G::LPR) ^ G::swz(row));   // this lane's chunk, in bytes
        // A and B rows never share a block: block q = wave + 4j is an A block
        // when RPL * q < BM, i.e. (BM / RPL being a multiple of 4, wave < 4)
        // when j < BM / (4 RPL) -- known at compile time
        vla[j] = j < G::BM / (4 * G::RPL);
        voff[j] = (unsigned)(vla[j] ? row : row - G::BM) * p.row_bytes + cb;
        vtail[j] = cb < ktail ? voff[j] : kOutOfRange;
        if (TB && !vla[j]) {
            const int kr = KPB * (q - G::BM / G::RPL) + lane / BCH;   // K row of the super-stage
            const int n = n0 + 8 * ((lane % BCH) ^ (4 * (kr & 3)));
            voff[j] = n < p.N ? ((unsigned)kr * (unsigned)p.N + (unsigned)n) * 2u : kOutOfRange;
            vtail[j] = voff[j];   // (a partial super-stage's rows past K are past the range)
        }
        if (TA && vla[j]) {
            const int kr = KPA * q + lane / ACH;
            const int m = m0 + 8 * ((lane % ACH) ^ (4 * (kr & 3)));
            voff[j] = m < p.M ? ((unsigned)kr * (unsigned)p.M + (unsigned)m) * 2u : kOutOfRange;
            vtail[j] = voff[j];
        }
    }
    // slot of super-stage u: u mod NS, always known at compile time
    auto slot_of = [&](auto k) -> char * {
        constexpr int K = decltype(k)::value;
        if constexpr (K == 3)
            return slot3;
        else if constexpr (K == 2)
            return slot2;
        else if constexpr (K == 1)
            return slot1;
        else
            return slot0;
    };
    auto code_load = [&](auto k, int u) {   // super-stage u into slot k = u mod NS
        char *slot = slot_of(k);
        // the super-stage's place in the row goes in the scalar offset, so
        // the per-lane offsets stay the same for every super-stage (nothing
        // per super-stage for the compiler to precompute and hold)
        const unsigned ko = (unsigned)u * G::SW;
        const bool whole = ko + G::SW <= kb, live = ko < kb;
        // stored [K][M] / [K][N]: the super-stage's 64 K rows start M / N
        // times 128 bytes per super-stage in; rows past K are past the range
        const unsigned kob = live ? (unsigned)u * 128u * (unsigned)p.N : 0u;
        const unsigned koa = live ? (unsigned)u * 128u * (unsigned)p.M : 0u;
#pragma unroll
        for (int j = 0; j < G::LB; ++j) {
            const int q = wave + 4 * j;
            // past this K range: an offset no buffer range reaches (zeros);
            // stored [K][..], the super-stage's rows are added (0 when not live)
            const bool kmaj = vla[j] ? TA : TB;
            const unsigned off = (whole ? voff[j] : live ? vtail[j] : kOutOfRange) + (!kmaj ? 0u : vla[j] ? koa : kob);
            // (a branch, not a select of the two resources: the latter is
            // rejected by the host pass of a __global__ template, which
            // then silently emits no launch stub)
            const unsigned so = kmaj ? 0u : ko;   // (stored [K][..]: all in off)
            if (vla[j])
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + 1024 * q), 16, off, so, 0, CPOL_NONE);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(slot + 1024 * q), 16, off, so, 0, CPOL_NONE);
        }
    };

    // ---- scale codes: job i of this wave is 64-row block q = wave + 4i of
    // [A rows | B rows]; lane l holds row l's 16 bytes of the period
    // staging registers of a period's codes (G::SSETS sets, see TileGeom)
    constexpr int SSETS = G::SSETS, SLEAD = G::SLEAD;
    u4v sstg[SSETS + 1][G::LS];   // (set SSETS: period 0, in the prologue)
    auto scale_load = [&](auto set, int period) {   // set = period % SSETS
        const bool live = period * G::P < U;
#pragma unroll
        for (int i = 0; i < G::LS; ++i) {
            const int q = wave + 4 * i;
            const int row = q * 64 + lane;
            const bool isa = q * 64 < G::BM;   // A and B rows never share a 64-row job
            const unsigned off = (live && q < G::SJOBS)
                                     ? (unsigned)(isa ? row : row - G::BM) * p.srow_bytes +
                                           16u * (unsigned)period
                                     : kOutOfRange;
            sstg[decltype(set)::value][i] = load16<CPOL_NONE>(isa ? rsa : rsb, off);
        }
    };
    // Dword d of a period is 128-K step 4*period + d.  Steps past K are
    // written as zero codes: a row's 16-byte load can run into the next
    // row's codes there, and a NaN code would poison the +0 of the padding
    // super-stages.
    auto scale_write = [&](auto set, int period) {   // set = period % SSETS
        char *buf = sbuf + (period & 1) * G::SCB;
#pragma unroll
        for (int i = 0; i < G::LS; ++i) {
            const int row = (wave + 4 * i) * 64 + lane;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                *reinterpret_cast<unsigned *>(buf + d * G::SROWS * 4 + row * 4) =
                    4 * period + d < p.nsteps ? sstg[decltype(set)::value][i][d] : 0u;
        }
    };

    // ---- fragments of one sub-step: lane (r, g) reads rows wm*32*MT + 32i
    // + r (A) and wn*32*NT + 32j + r (B).  kk is the sub-step's 64-K index
    // within its period.  E4M3 sub-step h of a super-stage is chunks 4h + g
    // and 4h + 2 + g, and its scale dword is that of 128-K step kk / 2.
    // E2M1 sub-step h takes K-block h of each of the super-stage's two
    // 128-K steps, lane half g step g (chunk h + 4g): the products of a
    // super-stage are summed in another order, and a lane uses one scale
    // dword (its step's) for all four sub-steps, byte h selected by the
    // instruction.
    constexpr int NV = FmtTraits<F>::nvec;
    using Frag = TileFrag<F, MT, NT>;
    // whether sub-step kk reads scale dwords (else it reuses the previous one's)
    constexpr auto new_scales = [](int kk) {
        return !G::SCALED ? false : F == FMT_FP4 ? kk % G::SUB == 0 : kk % 2 == 0;
    };
    const int arow = wm * 32 * MT + r, brow = G::BM + wn * 32 * NT + r;
    // Fragment of an operand stored [K][rows] (its region of a slot: 64 K
    // rows of `cols` columns, chunk x of K row k at place x ^ 4 (k mod 4)),
    // read transposed: for each group of 16 lanes the instruction takes four
    // K rows of 16 columns, lanes 4i .. 4i+3 giving row i's four 8-byte
    // pieces, and hands lane t of the group column t of the four rows.  So
    // lane (r, g) gets column 16 (r >> 4) + (r & 15) of the 32 that start at
    // column chunk cn - 2 (r >> 4) - ((r & 3) >> 1), at K rows 8 c8 .. +3
    // from one read and 8 c8 + 4 .. +7 from another (c8 = h + 4g: the K
    // values the other operand's fragment holds).
    auto read_kmajor = [&](const char *region, const int cols, const int cn, const int c8) -> u4v {
        const int jr = (r & 15) >> 2;
        u2v half[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int k = 8 * c8 + 4 * e + jr;
            // (the mask, a no-op here, bounds the offset to the region: the
            // compiler then sees which slot the read touches and does not
            // wait for the loads into the other)
            const int o = (k * (2 * cols) + 16 * (cn ^ (4 * (k & 3))) + 8 * (r & 1)) & (cols * G::SW - 1);
            half[e] = __builtin_bit_cast(
                u2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tile_s16x4 *)(region + o)));
        }
        return u4v{half[0].x, half[0].y, half[1].x, half[1].y};
    };
    auto read = [&](Frag &R, auto k, int u, auto kkc, const Frag *prev) {
        constexpr int kk = decltype(kkc)::value;
        constexpr int h = kk % G::SUB;
        const char *slot = slot_of(k);
        const int step = F == FMT_FP4 ? kk / G::SUB * 2 + g : kk / 2;   // of the scale dword
        const char *sc = sbuf + ((u / G::P) & 1) * G::SCB + step * G::SROWS * 4;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            // (16-bit operands: sub-step h takes 8 K values of each half
            // super-stage, like E2M1; with no scale codes any fixed K order
            // shared by A and B computes the product)
            const int c = F == FMT_FP8 ? 4 * h + 2 * v + g : h + 4 * g;
            if constexpr (TA) {
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int cm = 4 * (wm * MT + i) + 2 * (r >> 4) + ((r & 3) >> 1);   // column chunk
                    R.a[i][v] = read_kmajor(slot, G::BM, cm, c);
                }
            } else {
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    R.a[i][v] = *reinterpret_cast<const u4v *>(slot + G::code_off(arow + 32 * i, c));
            }
            if constexpr (TB) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int cn = 4 * (wn * NT + j) + 2 * (r >> 4) + ((r & 3) >> 1);   // column chunk
                    R.b[j][v] = read_kmajor(slot + G::BM * G::SW, G::BN, cn, c);
                }
            } else {
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    R.b[j][v] = *reinterpret_cast<const u4v *>(slot + G::code_off(brow + 32 * j, c));
            }
        }
        if constexpr (!G::SCALED)
            return;
        // sub-steps that share a scale dword take it from the first one's
        // registers
        if constexpr (!new_scales(kk)) {
            R.sa_from(*prev);
            return;
        }
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

    // the half of a 128-K step: blocks 2*half + g of the step's scale dword
    // MFMAs lo .. hi-1 of sub-step kk, in (i, j) order; the scale byte
    // of sub-step kk: E2M1 byte kk % SUB of the lane's dword, E4M3 byte
    // 2 * (kk % 2) + g (shifted down to byte 0)
    auto compute = [&](const Frag &R, auto kkc, auto lo, auto hi) {
        constexpr int kk = decltype(kkc)::value;
        const unsigned sh = F == FMT_FP4 ? 0u : 8u * (2 * (kk % 2) + g);
        unsigned xs[NT], ys[MT];
#pragma unroll
        for (int j = 0; j < NT; ++j) xs[j] = R.sb[j] >> sh;
#pragma unroll
        for (int i = 0; i < MT; ++i) ys[i] = R.sa[i] >> sh;
#pragma unroll
        for (int ij = decltype(lo)::value; ij < decltype(hi)::value; ++ij) {
                const int i = ij / NT, j = ij % NT;
                if constexpr (!G::SCALED) {
                    acc[i][j] = mfma16<F>(R.b[j][0], R.a[i][0], acc[i][j]);
                } else {
                    v8i x, y;
                    if constexpr (F == FMT_FP4) {
                        const u4v bx = R.b[j][0], ay = R.a[i][0];
                        x = v8i{(int)bx.x, (int)bx.y, (int)bx.z, (int)bx.w, 0, 0, 0, 0};
                        y = v8i{(int)ay.x, (int)ay.y, (int)ay.z, (int)ay.w, 0, 0, 0, 0};
                    } else {
                        const u4v b0 = R.b[j][0], b1 = R.b[j][NV - 1], a0 = R.a[i][0], a1 = R.a[i][NV - 1];
                        x = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                        y = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    }
                    acc[i][j] = mfma32<F, F == FMT_FP4 ? kk % G::SUB : 0>(x, xs[j], y, ys[i], acc[i][j]);
                }
        }
    };

    constexpr int NM = MT * NT;                  // MFMAs per sub-step
    constexpr int NCR = NV * ((TA ? 2 : 1) * MT + (TB ? 2 : 1) * NT);   // fragment reads per sub-step
    Frag R[2];

    // prologue: period 0's scale codes written, the next staged;
    // super-stages 0 .. NS-1 requested; super-stage 0's first fragments read
    using slot_0 = std::integral_constant<int, 0>;
    using kk_0 = std::integral_constant<int, 0>;
    // All requested before any is waited for (one memory latency, not
    // two).  The staging loads first: the loop then starts, as it
    // continues, with code loads as the most recent ones (the compiler's
    // own wait bookkeeping merges the two at the loop head).
    using set_p0 = std::integral_constant<int, SSETS>;
    scale_load(set_p0{}, 0);
    static_for<SLEAD - 1>([&](auto pc) {
        constexpr int q = 1 + decltype(pc)::value;
        scale_load(std::integral_constant<int, q % SSETS>{}, q);
    });
    __builtin_amdgcn_sched_barrier(0);   // (the scheduler keeps that order)
    static_for<NS>([&](auto sc) { code_load(sc, decltype(sc)::value); });
    scale_write(set_p0{}, 0);            // (the compiler waits for its registers)
    wait_vm_known<(NS - 1) * G::LB>();   // super-stage 0 has landed
    block_barrier();
    read(R[0], slot_0{}, 0, kk_0{}, nullptr);

    // Iteration u: sub-steps 0 .. SUB-2 read the next sub-step while
    // computing; the last one refills slot u with super-stage u+NS, at a
    // period start writes the next period's scale codes and stages a later
    // one, and reads super-stage u+1's first fragments (see "Pipeline").
    auto iteration = [&](auto uc, int u) {
        constexpr int i = decltype(uc)::value;   // u % TURN
        constexpr int pu = i % G::P;             // u % P
        using mine = std::integral_constant<int, i % NS>;         // slot of u and u + NS
        using next = std::integral_constant<int, (i + 1) % NS>;   // slot of u + 1
        // Four slots: loads issued after super-stage u+1's, which may stay
        // in flight while it is waited for: the code loads of u+2 .. u+NS-1 and the
        // scale loads issued with those (iterations u+2-NS .. u-1 that start
        // a period).  Not counted, since counting too few only waits longer
        // while counting one too many races with a load still landing: the
        // scale loads issued in the same iteration as u+1's code loads (the
        // scheduler may put them on either side of those), and those of
        // iterations before this turn (in the first turn there are none:
        // the prologue issues its scale loads before its code loads).
        constexpr int AFTER = NS == 2 ? 0 : [] {
            int n = (NS - 2) * G::LB;
            for (int j = i + 2 - NS > 0 ? i + 2 - NS : 0; j <= i - 1; ++j)
                if (j % G::P == 0)
                    n += G::LS;
            return n;
        }();
        static_for<G::SUB>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            constexpr int kk = pu * G::SUB + h;              // this sub-step within the period
            constexpr int fb = (i * G::SUB + h) & 1;         // its fragment buffer
            __builtin_amdgcn_sched_barrier(0);
            constexpr int kn = h == G::SUB - 1 ? (pu + 1) % G::P * G::SUB : kk + 1;   // the next one's
            using wset = std::integral_constant<int, (i / G::P + 1) % SSETS>;
            using lset = std::integral_constant<int, (i / G::P + SLEAD) % SSETS>;
            using c0 = std::integral_constant<int, 0>;
            using cN = std::integral_constant<int, NM>;
            if constexpr (NS == 2 && h == G::SUB - 1) {
                // two slots: slot u refilled as soon as every wave has read
                // it, super-stage u+1 waited for after that
                using cH = std::integral_constant<int, NM / 2>;
                block_barrier();
                if constexpr (pu == 0)
                    scale_write(wset{}, u / G::P + 1);
                code_load(mine{}, u + NS);
                compute(R[fb], std::integral_constant<int, kk>{}, c0{}, cH{});
                constexpr int NM1 = NM / 2, NMEM1 = G::LB + (pu == 0 ? 4 * G::LS : 0);
                static_for<NM1>([&](auto kc) {
                    constexpr int K = decltype(kc)::value;
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    constexpr int m0 = NMEM1 * K / NM1, m1 = NMEM1 * (K + 1) / NM1;
                    if constexpr (m1 > m0)
                        __builtin_amdgcn_sched_group_barrier(0x020 | 0x200, m1 - m0, 0);
                });
                __builtin_amdgcn_sched_barrier(0);
                wait_vm_known<G::LB>();   // super-stage u+1 has landed; u+2's loads may not have
                block_barrier();
                if constexpr (pu == 0)
                    scale_load(lset{}, u / G::P + SLEAD);
                read(R[fb ^ 1], next{}, u + 1, std::integral_constant<int, kn>{}, &R[fb]);
                compute(R[fb], std::integral_constant<int, kk>{}, cH{}, cN{});
                constexpr int NM2 = NM - NM1, NRD2 = NCR + (new_scales(kn) ? MT + NT : 0);
                static_for<NM2>([&](auto kc) {
                    constexpr int K = decltype(kc)::value;
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    constexpr int r0 = NRD2 * K / NM2, r1 = NRD2 * (K + 1) / NM2;
                    if constexpr (r1 > r0)
                        __builtin_amdgcn_sched_group_barrier(0x100, r1 - r0, 0);
                    if constexpr (pu == 0 && K < G::LS)
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                });
                __builtin_amdgcn_sched_barrier(0);
                return;
            }
            if constexpr (h == G::SUB - 1) {
                // super-stage u+1 (and any scale loads issued before it) has landed
                wait_vm_known<AFTER>();
                block_barrier();
                // the period of u is u0 / P + i / P with u0 / P a multiple of
                // SSETS, so the staging set of any period is known here
                if constexpr (pu == 0)
                    scale_write(wset{}, u / G::P + 1);
                code_load(mine{}, u + NS);
                if constexpr (pu == 0)
                    scale_load(lset{}, u / G::P + SLEAD);
                read(R[fb ^ 1], next{}, u + 1, std::integral_constant<int, kn>{}, &R[fb]);
            } else {
                read(R[fb ^ 1], mine{}, u, std::integral_constant<int, kn>{}, &R[fb]);
            }
            compute(R[fb], std::integral_constant<int, kk>{}, c0{}, cN{});
            // interleave: each MFMA followed by its share of the memory
            // operations (loads and scale writes at the last sub-step)
            constexpr int NMEM = h == G::SUB - 1 ? G::LB + (pu == 0 ? 5 * G::LS : 0) : 0;
            constexpr int NRD = NCR + (new_scales(kn) ? MT + NT : 0);
            static_for<NM>([&](auto kc) {
                constexpr int K = decltype(kc)::value;
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                constexpr int r0 = NRD * K / NM, r1 = NRD * (K + 1) / NM;
                if constexpr (r1 > r0)
                    __builtin_amdgcn_sched_group_barrier(0x100, r1 - r0, 0);
                constexpr int m0 = NMEM * K / NM, m1 = NMEM * (K + 1) / NM;
                if constexpr (m1 > m0)
                    __builtin_amdgcn_sched_group_barrier(0x020 | 0x200, m1 - m0, 0);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // whole turns (no branch inside one, so the compiler's own wait
    // bookkeeping stays exact), then the periods left
    int u0 = 0;
    for (; u0 + G::TURN <= U; u0 += G::TURN)
        static_for<G::TURN>([&](auto uc) { iteration(uc, u0 + decltype(uc)::value); });
    if constexpr (G::TURN > G::P) {
        static_for<G::TURN / G::P - 1>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            if (u0 + q * G::P < U)
                static_for<G::P>([&](auto uc) {
                    constexpr int i = q * G::P + decltype(uc)::value;
                    iteration(std::integral_constant<int, i>{}, u0 + i);
                });
        });
    }
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
        // passes of half the wave's rows (one pass when the wave has a single
        // row of 32x32 tiles); each wave uses its own region of the (now
        // idle) code slots.
        constexpr int RS = 64 * NT + 16;            // region row stride (bytes, padded)
        constexpr int PASSES = MT >= 2 ? 2 : 1;
        constexpr int TPP = MT / PASSES;             // 32-row tiles per pass
        constexpr int HR = 32 * TPP;                 // rows per pass
        // two waves per slot with two slots, one per slot with four
        static_assert((NS == 2 ? 2 : 1) * HR * RS <= G::SLOT, "epilogue staging must fit the code slots");
        char *region;
        if constexpr (NS == 2)
            region = (wave < 2 ? slot0 : slot1) + (wave & 1) * HR * RS;
        else
            region = wave == 0 ? slot0 : wave == 1 ? slot1 : wave == 2 ? slot2 : slot3;
        constexpr int LPR = 4 * NT;                  // lanes per row (16 bytes each)
        constexpr int RPI = 64 / LPR;                // rows per store instruction
        const int lr = lane / LPR, lc = lane % LPR;
        const int ncol = n0 + wn * 32 * NT + 8 * lc; // first of this lane's 8 columns
        const bool vec_ok = (p.N & 7) == 0 && ncol + 8 <= p.N;
        block_barrier();                             // every wave is done with the code slots
#pragma unroll
        for (int hf = 0; hf < PASSES; ++hf) {
#pragma unroll
            for (int ii = 0; ii < TPP; ++ii) {
                const int i = hf * TPP + ii;
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
                        // non-temporal: the output is not read again here, and
                        // kept out of L2 it leaves the operands there (measured
                        // 5% on 256 x 28672 x 8192 and 2048 x 14336 x 4096)
                        __builtin_nontemporal_store(q, reinterpret_cast<u4v *>(dst));
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
