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
//   * L1: a scale load with one row per lane (what a wave that owns a K
//     slice of many rows needs) costs as much as all of a split-K kernel's
//     MFMA and permute work together: at 32 x 14336 x 4096 E2M1, dropping
//     those loads alone took a split-K stream kernel from 10.6 to 9.0 us.
//     Here every scale byte is read once, in flat coalesced 16-byte pieces;
//   * issue order: the A tile and the scale codes are requested first and
//     are the only loads the workgroup waits for before its one barrier; the
//     B ring is already in flight behind them, so HBM streams from the start.
//     With one wave per row group, a ring of three 256-byte stages (12 KB)
//     beat deeper ones (four to eight stages) on MI355X; non-temporal B
//     loads (B is read once) gained about 1 us at 32 x 14336 x 4096.
// So:
//   * a workgroup owns 16*NW consecutive B rows and all 16*MT A rows; each
//     16-row group of B is streamed by KS waves, wave (w, q) taking rows
//     [16w, 16w+16) over the q-th of KS equal runs of K -- no barrier in the
//     K loop; with KS > 1 the KS partial tiles are summed in LDS at the end,
//     in part order.  With register rings two waves per row group and two
//     stages streamed 32 x 14336 x 4096 faster than one wave with three (a
//     pure read of the same bytes in that pattern: 6.3 against 7.3 us); with
//     the LDS ring below one wave and three slots is as fast or faster;
//   * the A tile and the scale codes of all the workgroup's rows are loaded
//     once into LDS (hence the K limit KMAX: the A tile must fit);
//   * B stages of 256 bytes per row are loaded with 16-byte loads in which
//     16 consecutive lanes read one row's 256 contiguous bytes (loading the
//     fragments straight into registers instead, 64 bytes of 16 rows per
//     load, streamed B slower), and reach the wave's LDS in one of two ways:
//     a G-deep register ring stored stage by stage into the wave's private
//     slot (two alternating slots when KS = 1), or (DMA) G slots that the
//     buffer loads write themselves, each lane's chunk XOR-swizzled by its
//     row -- no staging registers and no LDS store instructions (32 x 14336
//     x 4096 with one wave per row group and three slots: 8.6 us against
//     9.0-9.4 with two waves and register rings).  Either is read back as
//     16x16x128 MFMA fragments;
//   * with EPI the summed tile goes through LDS to the shared reduced-tile
//     epilogue (bias, activation, 16-bit / FP32 or MX-requantized output).
//
// LDS layouts: code rows in groups of 8, chunk-major inside a group (chunk c
// of the 8 rows = 128 contiguous bytes) with a padded chunk stride of 144
// bytes (36 dwords: the fragment reads take 8 rows of one chunk, the staging
// stores consecutive chunks of one row, and both land on distinct banks; a
// stride of 160 put chunks c and c + 4 of a row on the same banks); scale
// codes as [128-K step][row] dwords, so a step's codes of 16 consecutive rows
// are contiguous, with one spare dword after each step (the prologue's lanes
// that store one row's steps would otherwise share a bank).
//
// Ragged M / N: B rows past N read as zeros (out of the buffer range) and add
// exactly +0; A rows past M are neither loaded nor stored into LDS, and as
// every output row depends on its own A row only, the rows whose LDS holds
// stale bytes are exactly the ones never written to C.  K tail: a B stage that runs past the row end
// reads the next row's bytes, so MFMA steps past K are skipped; a row's last
// 16-byte scale piece may likewise run into the next row (or past the
// buffer, reading zeros there), and only its dwords below K/128 are kept.
#pragma once

#include "mx_epilogue.hpp"
#include "mx_sync.hpp"
#include "mx_tile.hpp"

namespace mxg {

template <int F, int MT, int NW, int KMAX, int KS = 1>
struct DecodeGeom {
    static constexpr int NWT = NW * KS;                      // waves: NW row groups x KS K parts
    static constexpr int SB = FmtTraits<F>::step_bytes;      // bytes per row per 128-K step
    static constexpr int BM = 16 * MT;                       // A rows
    static constexpr int BN = 16 * NW;                       // B rows (16 per wave)
    static constexpr int CHUNK = 144;                        // padded 16-byte chunk stride
    static constexpr int SW = 256;                           // B stage: bytes per row
    static constexpr int SPS = SW / SB;                      // MFMA steps per stage
    static constexpr int SCH = SW / 16;                      // chunks per row per stage
    static constexpr int SLOT = 2 * SCH * CHUNK;             // 16 rows = 2 groups of 8
    static constexpr int RB_MAX = KMAX / 128 * SB;           // A row bytes at K = KMAX
    static constexpr int ACH = RB_MAX / 16;                  // A chunks per row at KMAX
    static constexpr int AGROUP = ACH * CHUNK;               // one 8-row group of A
    static constexpr int NSTEP_MAX = KMAX / 128;
    // LDS map
    // scale codes [step][row] with one spare dword per step: the prologue
    // stores of one row's steps then fall on different banks
    static constexpr int SAS = BM + 1, SBSS = BN + 1;                      // step strides (dwords)
    static constexpr int SA_OFF = BM / 8 * AGROUP;                         // [step][SAS] dwords
    static constexpr int SBS_OFF = SA_OFF + NSTEP_MAX * SAS * 4;           // [step][SBSS] dwords
    // B slots per wave: two with one wave per row group; one when KS waves
    // share a row group (a wave's LDS operations run in order, so its next
    // stage's stores cannot overtake the reads of the current one)
    static constexpr int SLOTS = KS == 1 ? 2 : 1;
    static constexpr int B_OFF = SBS_OFF + NSTEP_MAX * SBSS * 4;           // [wave][SLOTS] slots
    static constexpr int BYTES = B_OFF + NWT * SLOTS * SLOT;
    // coalesced prologue loads per wave: A chunks (16 bytes)
    static constexpr int PA = cdiv_c(BM * ACH, 64 * NWT);
    // 16-byte scale pieces per row (4 steps each) and per wave
    static constexpr int SQ_MAX = cdiv_c(NSTEP_MAX, 4);
    static constexpr int PSA = cdiv_c(BM * SQ_MAX, 64 * NWT);
    static constexpr int PSB = cdiv_c(BN * SQ_MAX, 64 * NWT);
    // partial tiles of the K parts past the first, summed at the end (in
    // the A region, free by then)
    static_assert((KS - 1) * NW * MT * 64 * 16 <= SA_OFF, "partials must fit the A region");
    static_assert(B_OFF % 16 == 0, "B slots hold 16-byte pieces");
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
    // LDS ring (the loads write LDS themselves): one unpadded 16-row stage
    // per slot, chunk c of row r at 16 (c ^ r) -- the 16 rows of a fragment
    // read then fall on 16 different 4-bank groups
    static constexpr int DSLOT = 16 * SW;
    __device__ static constexpr int d_off(int row, int c) { return 256 * row + 16 * (c ^ row); }
};

// Wait until at most `later` stages of LB loads each are outstanding.
template <int LB, int G>
__device__ __forceinline__ void wait_later(int later)
{
    if constexpr (G > 7) { if (later >= 7) { wait_vm<7 * LB>(); return; } }
    if constexpr (G > 6) { if (later >= 6) { wait_vm<6 * LB>(); return; } }
    if constexpr (G > 5) { if (later >= 5) { wait_vm<5 * LB>(); return; } }
    if constexpr (G > 4) { if (later >= 4) { wait_vm<4 * LB>(); return; } }
    if constexpr (G > 3) { if (later >= 3) { wait_vm<3 * LB>(); return; } }
    if constexpr (G > 2) { if (later >= 2) { wait_vm<2 * LB>(); return; } }
    if constexpr (G > 1) { if (later >= 1) { wait_vm<1 * LB>(); return; } }
    wait_vm<0>();
}

// EPI: the fused epilogue (bias, activation, and the MX output kinds) on
// the final tile, which then goes through LDS.
// DMA: the B ring lives in LDS, G slots per wave that the buffer loads write
// directly (no register staging and no LDS store instructions); otherwise
// it is a register ring stored into the wave's LDS slot stage by stage.
template <int F, int MT, int NW, int KMAX, int G, int OUT, int KS = 1, int EPI = 0, int DMA = 0>
__global__ __launch_bounds__(64 * NW * KS)
void mx_gemm_decode(GemmArgs p)
{
    using D = DecodeGeom<F, MT, NW, KMAX, KS>;
    constexpr int NWT = D::NWT;
    static_assert(EPI || OUT <= OUT_F32, "MX output kinds need the fused epilogue");
    constexpr int LB = 4;
    constexpr int PSA = D::PSA, PSB = D::PSB;
    static_assert(G * LB + D::PA + PSA + PSB < 64, "outstanding loads must fit the vmcnt field");
    constexpr int LDS_BYTES = DMA ? D::B_OFF + NWT * G * D::DSLOT : D::BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rw = wave % NW, kh = wave / NW;   // row group, K part
    const int r = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.y * D::BM, n0 = blockIdx.x * D::BN;
    const int mrows = min(D::BM, p.M - m0);
    const int nrows = min(D::BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (size_t)m0 * p.row_bytes, mrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (size_t)n0 * p.row_bytes, nrows * p.row_bytes);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.sa + (size_t)m0 * p.srow_bytes, mrows * p.srow_bytes);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(p.sb + (size_t)n0 * p.srow_bytes, nrows * p.srow_bytes);
    const int T = (int)((p.row_bytes + D::SW - 1) / D::SW);
    const int nst = p.nsteps;
    // this wave's stages [t0, t0 + nt) of the row group's T
    const int t0 = kh * T / KS, nt = (kh + 1) * T / KS - t0;

    // prologue: the A tile (flat: chunk i is bytes [16i, 16i+16) of rows m0..,
    // i.e. row i / CH, chunk i % CH) and the scale pieces (piece c is row
    // c / CQ, steps 4 (c % CQ) ..) first, then the first G B stages
    const unsigned CH = p.row_bytes / 16u;            // A chunks per row
    const unsigned CQ = ((unsigned)nst + 3u) / 4u;    // 16-byte scale pieces per row
    const unsigned a_chunks = (unsigned)mrows * CH;
    const unsigned sa_chunks = (unsigned)mrows * CQ, sb_chunks = (unsigned)nrows * CQ;
    // x / d as a multiply-high by ceil(2^32 / d) (exact for x < 2^32 / d, far
    // above any index here); d = 1 has no 32-bit multiplier
    const unsigned mch = 0xFFFFFFFFu / CH + 1u, mcq = 0xFFFFFFFFu / CQ + 1u;
    auto row_of_piece = [&](unsigned c) { return CQ == 1u ? c : __umulhi(c, mcq); };
    u4v av[D::PA], sva[PSA], svb[PSB];
#pragma unroll
    for (int i = 0; i < D::PA; ++i) {
        const unsigned idx = (unsigned)(64 * (NWT * i + wave) + lane);
        av[i] = load16<CPOL_NONE>(ra, idx < a_chunks ? 16u * idx : kOutOfRange);
    }
#pragma unroll
    for (int i = 0; i < PSA; ++i) {
        const unsigned c = (unsigned)(64 * (NWT * i + wave) + lane);
        const unsigned row = row_of_piece(c);
        sva[i] = load16<CPOL_NONE>(rsa, c < sa_chunks ? row * p.srow_bytes + 16u * (c - row * CQ) : kOutOfRange);
    }
#pragma unroll
    for (int i = 0; i < PSB; ++i) {
        const unsigned c = (unsigned)(64 * (NWT * i + wave) + lane);
        const unsigned row = row_of_piece(c);
        svb[i] = load16<CPOL_NONE>(rsb, c < sb_chunks ? row * p.srow_bytes + 16u * (c - row * CQ) : kOutOfRange);
    }

    // load j of a stage covers rows 4j .. 4j+3 of this wave's 16 (lane l:
    // row 4j + l/16, 16 bytes of the stage's 256 at chunk l%16, XOR the row
    // with the LDS ring), read once, so non-temporal
    const unsigned bload = (unsigned)(16 * rw + (lane >> 4)) * p.row_bytes + 16u * (unsigned)(lane & 15);
    const unsigned bstride = 4u * p.row_bytes;
    u4v stg[DMA ? 1 : G][LB];
    // stages past K read zeros but are issued all the same, so that the
    // outstanding-load counts below are exact
    auto fill_stage = [&](u4v (&set)[LB], int i) {   // the wave's i-th stage
        const unsigned kt = i < nt ? (unsigned)(t0 + i) * D::SW : kOutOfRange;
#pragma unroll
        for (int j = 0; j < LB; ++j)
            set[j] = load16<CPOL_NT>(rb, bload + (unsigned)j * bstride + kt);
    };
    char *ring = smem + D::B_OFF + wave * G * D::DSLOT;   // DMA: this wave's G slots
    auto fill_slot = [&](int u, int i) {   // the wave's i-th stage into LDS slot u
        const unsigned kt = i < nt ? (unsigned)(t0 + i) * D::SW : kOutOfRange;
        const unsigned brow = (unsigned)(16 * rw + (lane >> 4)) * p.row_bytes;
#pragma unroll
        for (int j = 0; j < LB; ++j) {
            // lane l lands at byte 1024 j + 16 l of the slot = d_off(row, l%16 ^ row)
            const unsigned c = (unsigned)(lane & 15) ^ (unsigned)(4 * j + (lane >> 4));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(ring + u * D::DSLOT + 1024 * j), 16,
                                                     brow + (unsigned)j * bstride + 16u * c + kt, 0, 0, CPOL_NT);
        }
    };
#pragma unroll
    for (int i = 0; i < G; ++i) {
        if constexpr (DMA)
            fill_slot(i, i);
        else
            fill_stage(stg[i], i);
    }

    wait_vm<G * LB>();   // the A tile and the scale pieces have landed
#pragma unroll
    for (int i = 0; i < D::PA; ++i) {
        const unsigned idx = (unsigned)(64 * (NWT * i + wave) + lane);
        if (idx < a_chunks) {
            const unsigned row = __umulhi(idx, mch), c = idx - row * CH;
            *reinterpret_cast<u4v *>(smem + D::a_off((int)row, (int)c)) = av[i];
        }
    }
#pragma unroll
    for (int i = 0; i < PSA; ++i) {
        const unsigned c = (unsigned)(64 * (NWT * i + wave) + lane);
        if (c < sa_chunks) {
            const unsigned row = row_of_piece(c), k = 4u * (c - row * CQ);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k + e < (unsigned)nst)
                    *reinterpret_cast<unsigned *>(smem + D::SA_OFF + 4 * ((k + e) * D::SAS + row)) = sva[i][e];
        }
    }
#pragma unroll
    for (int i = 0; i < PSB; ++i) {
        const unsigned c = (unsigned)(64 * (NWT * i + wave) + lane);
        if (c < sb_chunks) {
            const unsigned row = row_of_piece(c), k = 4u * (c - row * CQ);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k + e < (unsigned)nst)
                    *reinterpret_cast<unsigned *>(smem + D::SBS_OFF + 4 * ((k + e) * D::SBSS + row)) = svb[i][e];
        }
    }
    __syncthreads();   // the A tile and scale codes are shared by all waves

    // register ring: each stage is stored into the wave's LDS slot(s)
    char *slots = smem + D::B_OFF + wave * D::SLOTS * D::SLOT;
    const int bw_lane = D::b_off(lane >> 4, lane & 15);
    auto store_stage = [&](const u4v (&set)[LB], int i) {
        char *slot = slots + (D::SLOTS == 2 ? (i & 1) * D::SLOT : 0);
#pragma unroll
        for (int j = 0; j < LB; ++j)
            *reinterpret_cast<u4v *>(slot + bw_lane + D::b_off(4 * j, 0)) = set[j];
    };

    v4f acc[MT];
#pragma unroll
    for (int x = 0; x < MT; ++x)
        acc[x] = v4f{0.f, 0.f, 0.f, 0.f};

    // one stage (the wave's i-th): wait for its loads (the stages issued
    // after it may stay in flight: the prologue issued G, each earlier stage
    // refilled one below nt); register ring: store it and refill its staging
    // set, then its MFMA steps; LDS ring: its MFMA steps, then the refill of
    // its slot
    auto stage = [&](auto uc, int i) {
        constexpr int u = decltype(uc)::value;
        wait_later<LB, G>(min(i + G, max(G, nt)) - i - 1);
        if constexpr (!DMA) {
            store_stage(stg[u], i);
            if (i + G < nt)
                fill_stage(stg[u], i + G);
        }
        const char *slot = DMA ? ring + u * D::DSLOT : slots + (D::SLOTS == 2 ? (i & 1) * D::SLOT : 0);
        auto boff = [&](int c) { return DMA ? D::d_off(r, c) : D::b_off(r, c); };
        const int t = t0 + i;
        // fragments and scale codes of 128-K step k (the s-th of the stage)
        auto read_step = [&](int s, int k, StepFrag<F> &fb, StepFrag<F> (&fa)[MT], unsigned &sb,
                             unsigned (&sa)[MT]) {
            if constexpr (F == FMT_FP4) {
                fb.d[0] = *reinterpret_cast<const u4v *>(slot + boff(4 * s + g));
            } else {
                fb.d[0] = *reinterpret_cast<const u4v *>(slot + boff(8 * s + g));
                fb.d[1] = *reinterpret_cast<const u4v *>(slot + boff(8 * s + 4 + g));
            }
            sb = *reinterpret_cast<const unsigned *>(smem + D::SBS_OFF + 4 * (k * D::SBSS + 16 * rw + r)) >> (8 * g);
#pragma unroll
            for (int x = 0; x < MT; ++x) {
                const int row = 16 * x + r;
                if constexpr (F == FMT_FP4) {
                    fa[x].d[0] = *reinterpret_cast<const u4v *>(smem + D::a_off(row, 4 * k + g));
                } else {
                    fa[x].d[0] = *reinterpret_cast<const u4v *>(smem + D::a_off(row, 8 * k + g));
                    fa[x].d[1] = *reinterpret_cast<const u4v *>(smem + D::a_off(row, 8 * k + 4 + g));
                }
                sa[x] = *reinterpret_cast<const unsigned *>(smem + D::SA_OFF + 4 * (k * D::SAS + row)) >> (8 * g);
            }
        };
        if ((t + 1) * D::SPS <= nst) {
            // a whole stage inside K: every read issued before the first
            // MFMA, so the LDS round trips of the steps overlap
            StepFrag<F> fb[D::SPS], fa[D::SPS][MT];
            unsigned sb[D::SPS], sa[D::SPS][MT];
#pragma unroll
            for (int s = 0; s < D::SPS; ++s)
                read_step(s, t * D::SPS + s, fb[s], fa[s], sb[s], sa[s]);
#pragma unroll
            for (int s = 0; s < D::SPS; ++s)
#pragma unroll
                for (int x = 0; x < MT; ++x)
                    acc[x] = mfma<F>(fb[s], sb[s], fa[s][x], sa[s][x], acc[x]);
        } else {
            // the stage that holds the end of K: its steps past K are skipped
#pragma unroll
            for (int s = 0; s < D::SPS; ++s) {
                const int k = t * D::SPS + s;
                if (k >= nst)
                    break;
                StepFrag<F> fb, fa[MT];
                unsigned sb, sa[MT];
                read_step(s, k, fb, fa, sb, sa);
#pragma unroll
                for (int x = 0; x < MT; ++x)
                    acc[x] = mfma<F>(fb, sb, fa[x], sa[x], acc[x]);
            }
        }
        if constexpr (DMA) {
            if (i + G < nt) {
                // the slot's fragment reads have returned before its next
                // stage can land in it
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                fill_slot(u, i + G);
            }
        }
    };
    for (int i0 = 0; i0 < nt; i0 += G)
        static_for<G>([&](auto uc) {
            if (i0 + decltype(uc)::value < nt)
                stage(uc, i0 + decltype(uc)::value);
        });
    if constexpr (DMA)
        wait_vm<0>();   // zero stages past nt may still be landing in the ring

    if constexpr (EPI) {
        // every K part parks its partial tile in the A region (free once all
        // waves are past the K loop); the parts are summed in part order
        // while the epilogue writes the output, any thread taking any group
        // of four columns (the MX kinds want a row's 32-column block in 8
        // consecutive lanes)
        constexpr int RS = D::BN + 4;   // padded row stride (floats)
        static_assert(KS * D::BM * RS * 4 <= D::SA_OFF, "partial tiles must fit the A region");
        float *red = reinterpret_cast<float *>(smem);
        __syncthreads();   // every wave is done reading the A tile
#pragma unroll
        for (int x = 0; x < MT; ++x)
            *reinterpret_cast<v4f *>(&red[(kh * D::BM + 16 * x + r) * RS + 16 * rw + 4 * g]) = acc[x];
        __syncthreads();
        store_reduced_tile<OUT, 1, D::BM, D::BN / 4>(
            p, m0, n0, (int)threadIdx.x, 64 * NWT, [&](int row, int c4) {
                v4f sum = *reinterpret_cast<const v4f *>(&red[row * RS + 4 * c4]);
#pragma unroll
                for (int q = 1; q < KS; ++q)
                    sum += *reinterpret_cast<const v4f *>(&red[(q * D::BM + row) * RS + 4 * c4]);
                return sum;
            });
        return;
    }

    if constexpr (KS > 1) {
        // the K parts past the first park their partial tiles in the A
        // region; the first part's wave adds them in part order (fixed, so
        // the result is deterministic)
        v4f *part = reinterpret_cast<v4f *>(smem);
        __syncthreads();   // every wave is done reading the A tile
        if (kh > 0) {
#pragma unroll
            for (int x = 0; x < MT; ++x)
                part[(((kh - 1) * NW + rw) * MT + x) * 64 + lane] = acc[x];
        }
        __syncthreads();
        if (kh > 0)
            return;
#pragma unroll
        for (int q = 1; q < KS; ++q)
#pragma unroll
            for (int x = 0; x < MT; ++x)
                acc[x] += part[(((q - 1) * NW + rw) * MT + x) * 64 + lane];
    }

    const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
    for (int x = 0; x < MT; ++x) {
        const int m = m0 + 16 * x + r;
        const int n = n0 + 16 * rw + 4 * g;
        if (m < p.M && n < p.N)
            store4<OUT>(p.c, p.N, m, n, acc[x], vec_ok && n + 3 < p.N);
    }
}

}  // namespace mxg
