// mx_lds.hpp -- LDS-staged NT MX block-scaled GEMM for gfx950.
//
// Why stage through LDS.  The scaled MFMA wants each lane to hold 16 (FP4)
// or 32 (FP8) bytes of one row, with 16 different rows in 16 consecutive
// lanes.  Loaded straight from memory in that layout, no two neighbouring
// lanes touch the same 64-byte segment, so the L1 cannot merge lane
// requests and its access rate, not HBM, limits the kernel.  Here every
// global load is a direct-to-LDS 16-byte-per-lane load in which each run of
// four consecutive lanes covers one 64-byte segment of one row; the MFMA
// fragments are then read from LDS with ds_read_b128.
//
// Tiles.  A workgroup owns a BM x BN output tile (BM = 16*MT*WAVES_M,
// BN = 16*WN*WAVES_N).  Its waves form KW x WAVES_M x WAVES_N: KW groups
// split K between them (split-K inside the workgroup), and within a group
// wave (wm, wn) computes MT x WN 16x16 subtiles.  K is consumed in stages of
// SPS MFMA steps (128*SPS K values); a ring of STAGES stages lives in LDS.
//
// Stage layout in LDS, per K group kw: the A tile (BM rows) and the B tile
// (BN rows) as 1 KB blocks of RPB = 1024/W whole rows (W = bytes of one row
// per stage), then the scale codes of the A and B rows as [row][step] dwords.
// Within a row the 16-byte chunks are XOR-swizzled with a function of the
// row, so that the 16 rows one ds_read_b128 touches fall on different banks;
// the swizzle is applied on the load side (each lane fetches the chunk that
// belongs at its LDS slot), and it only permutes chunks inside aligned
// groups of four, so every quad of lanes still reads one 64-byte segment.
//
// Pipeline.  The loads of one stage are 1 KB jobs spread evenly over all
// waves (LPS per wave, padded with out-of-range loads that move no data), so
// every wave issues the same number of loads per stage and a wave's
// "stage t has landed" test is s_waitcnt vmcnt(#loads it issued after stage
// t).  Each iteration: wait for stage t, barrier (now every wave's share of
// stage t is in LDS and every wave has finished reading stage t-1), issue
// stage t+STAGES-1 into the slot stage t-1 used, then compute stage t.
//
// K tails and ragged M, N: loads past the operand rows or past a K group's
// last step use an offset outside the buffer range and deliver zeros, which
// add exactly +0 (zero codes, zero scale codes).
#pragma once

#include "mx_common.hpp"

namespace mxg {

constexpr int cdiv_c(int a, int b) { return (a + b - 1) / b; }

// K group k of KW covers MFMA steps [kbegin(k), kbegin(k+1)).
template <int KW>
__device__ __forceinline__ int kbegin(int k, int nsteps)
{
    return (int)(((long long)k * nsteps) / KW);
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_ptr_t dst, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
}

__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, lds_ptr_t dst, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, off, 0, 0, 0);
}

// Wait until at most n of this wave's vector-memory loads are outstanding.
// The compiler does not track direct-to-LDS loads, so the pipeline waits are
// explicit; the memory clobber keeps LDS reads from moving above them.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the implicit memory fence of __syncthreads (which
// would wait for every outstanding load, including later stages).  The
// wave's own LDS reads are complete first, so a slot is never refilled
// while a read of it is still in flight.
__device__ __forceinline__ void block_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int F, int KW, int WAVES_M, int WAVES_N, int MT, int WN, int SPS>
struct LdsGeom {
    static constexpr int NW = KW * WAVES_M * WAVES_N;       // waves per workgroup
    static constexpr int SB = FmtTraits<F>::step_bytes;
    static constexpr int W = SPS * SB;                       // bytes per row per stage
    static constexpr int CPR = W / 16;                       // 16-byte chunks per row
    static constexpr int RPB = 1024 / W;                     // rows per 1 KB block
    static constexpr int BM = 16 * MT * WAVES_M;
    static constexpr int BN = 16 * WN * WAVES_N;
    static constexpr int ABLK = BM / RPB, BBLK = BN / RPB;   // 1 KB blocks per K group
    static constexpr int ASJ = cdiv_c(BM * SPS, 64);         // scale jobs per K group
    static constexpr int BSJ = cdiv_c(BN * SPS, 64);
    static constexpr int GJOBS = ABLK + BBLK + ASJ + BSJ;    // jobs per K group and stage
    static constexpr int JOBS = KW * GJOBS;
    static constexpr int LPS = cdiv_c(JOBS, NW);             // loads per wave per stage
    // byte offsets inside one stage; every area a job writes is a whole
    // number of that job's 1 KB / 256 B footprint, so lanes past the end of
    // an area never write into the next one
    static constexpr int GROUP_DATA = (ABLK + BBLK) * 1024;
    static constexpr int SA_STRIDE = ASJ * 256;                      // [BM][SPS] dwords, padded
    static constexpr int SB_STRIDE = BSJ * 256;
    static constexpr int SCALE_A = KW * GROUP_DATA;                  // [kw] A scale areas
    static constexpr int SCALE_B = SCALE_A + KW * SA_STRIDE;         // [kw] B scale areas
    static constexpr int PAD = SCALE_B + KW * SB_STRIDE;             // target of padding loads
    static constexpr int STAGE_BYTES = (PAD + 256 + 1023) / 1024 * 1024;
    // rows sharing one 256-byte bank window, and the chunk swizzle
    static constexpr int ROWS_PER_256 = W >= 256 ? 1 : 256 / W;
    static constexpr int SWZ_MASK = (CPR < 16 ? CPR : 16) - 1;
    static_assert(W <= 1024, "one row per stage must fit one 1 KB block");
    static_assert(BM % RPB == 0 && BN % RPB == 0, "tiles must be whole blocks");
    __device__ static constexpr int swz(int row) { return (row / ROWS_PER_256) & SWZ_MASK; }
    // LDS byte offset of chunk c of tile row `row` within its tile
    __device__ static constexpr int chunk_off(int row, int c)
    {
        return (row / RPB) * 1024 + (row % RPB) * W + 16 * (c ^ swz(row));
    }
};

// Issue this wave's loads of stage `t` (steps kbegin(kw) + t*SPS ... of
// every K group kw) into the stage slot at `slot`.  The job dispatch is
// recomputed per stage from the wave-uniform job index (scalar work);
// keeping per-job offsets live across the K loop would cost registers the
// large tiles do not have.
template <int F, int KW, int WAVES_M, int WAVES_N, int MT, int WN, int SPS>
__device__ __forceinline__ void lds_issue_stage(char *slot, int t, int wave, int lane, int mrows,
                                                int nrows, __amdgpu_buffer_rsrc_t ra,
                                                __amdgpu_buffer_rsrc_t rb,
                                                __amdgpu_buffer_rsrc_t rsa,
                                                __amdgpu_buffer_rsrc_t rsb, const GemmArgs &p)
{
    using G = LdsGeom<F, KW, WAVES_M, WAVES_N, MT, WN, SPS>;
#pragma unroll
    for (int i = 0; i < G::LPS; ++i) {
        const int q = wave + G::NW * i;            // wave-uniform job index
        if (q >= G::JOBS) {
            // padding: an out-of-range load (into the stage's pad area) keeps
            // every wave's load count per stage equal
            dma4(rsa, (lds_ptr_t)(slot + G::PAD), kOutOfRange);
            continue;
        }
        const int kw = q / G::GJOBS;
        int j = q % G::GJOBS;
        const int step0 = kbegin<KW>(kw, p.nsteps) + t * SPS;
        const int kend = kbegin<KW>(kw + 1, p.nsteps);
        if (j < G::ABLK + G::BBLK) {
            const bool isa = j < G::ABLK;
            if (!isa)
                j -= G::ABLK;
            const int row = j * G::RPB + lane / G::CPR;
            const int c = (lane % G::CPR) ^ G::swz(row);
            const int step = step0 + c / (G::SB / 16);
            const unsigned off = (step < kend && row < (isa ? mrows : nrows))
                                     ? (unsigned)row * p.row_bytes + (unsigned)step0 * G::SB + 16u * c
                                     : kOutOfRange;
            char *dst = slot + kw * G::GROUP_DATA + (isa ? 0 : G::ABLK * 1024) + j * 1024;
            dma16(isa ? ra : rb, (lds_ptr_t)dst, off);
        } else {
            j -= G::ABLK + G::BBLK;
            const bool isa = j < G::ASJ;
            if (!isa)
                j -= G::ASJ;
            const int e = j * 64 + lane;           // [row][step] dword index
            const int row = e / SPS, s = e % SPS;
            const unsigned off = (row < (isa ? mrows : nrows) && step0 + s < kend)
                                     ? (unsigned)row * p.srow_bytes + 4u * (step0 + s)
                                     : kOutOfRange;
            char *dst = slot + (isa ? G::SCALE_A + kw * G::SA_STRIDE
                                    : G::SCALE_B + kw * G::SB_STRIDE) + j * 256;
            dma4(isa ? rsa : rsb, (lds_ptr_t)dst, off);
        }
    }
}

template <class G, int F>
__device__ __forceinline__ StepFrag<F> lds_frag(const char *tile, int row, int s, int g)
{
    StepFrag<F> f;
    if constexpr (F == FMT_FP4) {
        f.d[0] = *reinterpret_cast<const u4v *>(tile + G::chunk_off(row, 4 * s + g));
    } else {
        f.d[0] = *reinterpret_cast<const u4v *>(tile + G::chunk_off(row, 8 * s + g));
        f.d[1] = *reinterpret_cast<const u4v *>(tile + G::chunk_off(row, 8 * s + 4 + g));
    }
    return f;
}

// Compute one stage from `slot`: SPS steps of MT x WN MFMAs for this wave.
// All of the stage's fragments and scale codes are read first, so the LDS
// latency is paid once per stage rather than once per step.
template <int F, int KW, int WAVES_M, int WAVES_N, int MT, int WN, int SPS>
__device__ __forceinline__ void lds_compute_stage(const char *slot, int kw, int wm, int wn,
                                                  int r, int g, v4f (&acc)[MT][WN])
{
    using G = LdsGeom<F, KW, WAVES_M, WAVES_N, MT, WN, SPS>;
    const char *ta = slot + kw * G::GROUP_DATA;
    const char *tb = ta + G::ABLK * 1024;
    const unsigned char *sca =
        reinterpret_cast<const unsigned char *>(slot + G::SCALE_A + kw * G::SA_STRIDE);
    const unsigned char *scb =
        reinterpret_cast<const unsigned char *>(slot + G::SCALE_B + kw * G::SB_STRIDE);
    StepFrag<F> fa[SPS][MT], fb[SPS][WN];
    unsigned sa[SPS][MT], sb[SPS][WN];
#pragma unroll
    for (int s = 0; s < SPS; ++s) {
#pragma unroll
        for (int x = 0; x < MT; ++x) {
            const int row = wm * 16 * MT + 16 * x + r;
            fa[s][x] = lds_frag<G, F>(ta, row, s, g);
            sa[s][x] = sca[(row * SPS + s) * 4 + g];
        }
#pragma unroll
        for (int y = 0; y < WN; ++y) {
            const int row = wn * 16 * WN + 16 * y + r;
            fb[s][y] = lds_frag<G, F>(tb, row, s, g);
            sb[s][y] = scb[(row * SPS + s) * 4 + g];
        }
    }
#pragma unroll
    for (int s = 0; s < SPS; ++s)
#pragma unroll
        for (int x = 0; x < MT; ++x)
#pragma unroll
            for (int y = 0; y < WN; ++y)
                acc[x][y] = mfma<F>(fb[s][y], sb[s][y], fa[s][x], sa[s][x], acc[x][y]);
}

template <int LPS, int STAGES>
__device__ __forceinline__ void wait_stage(int later)
{
    // `later` = stages issued after the one we wait for (0 .. STAGES-2)
    static_assert(STAGES >= 2 && STAGES <= 6, "ring depth");
    if constexpr (STAGES >= 6) { if (later >= 4) { wait_vm<4 * LPS>(); return; } }
    if constexpr (STAGES >= 5) { if (later >= 3) { wait_vm<3 * LPS>(); return; } }
    if constexpr (STAGES >= 4) { if (later >= 2) { wait_vm<2 * LPS>(); return; } }
    if constexpr (STAGES >= 3) { if (later >= 1) { wait_vm<1 * LPS>(); return; } }
    wait_vm<0>();
}

template <int F, int KW, int WAVES_M, int WAVES_N, int MT, int WN, int SPS, int STAGES, int OUT>
__global__ __launch_bounds__(64 * KW * WAVES_M * WAVES_N)
void mx_gemm_lds(GemmArgs p)
{
    using G = LdsGeom<F, KW, WAVES_M, WAVES_N, MT, WN, SPS>;
    static_assert((STAGES - 2) * G::LPS < 64, "outstanding loads must fit the vmcnt field");
    static_assert(STAGES * G::STAGE_BYTES <= 160 * 1024, "gfx950 has 160 KB of LDS per CU");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * G::STAGE_BYTES];

    const int lane = threadIdx.x & 63;
    // wave-uniform by construction; saying so lets the compiler keep the
    // job dispatch and buffer descriptors in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int kw = wave / (WAVES_M * WAVES_N);
    const int wm = (wave % (WAVES_M * WAVES_N)) % WAVES_M;
    const int wn = (wave % (WAVES_M * WAVES_N)) / WAVES_M;
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

    // All K groups run the same number of stages T, set by the longest
    // group (the last one, of ceil(nsteps/KW) steps); the shorter ones read
    // zeros at the end.
    const int T = cdiv_c(cdiv_c(p.nsteps, KW), SPS);

    v4f acc[MT][WN];
#pragma unroll
    for (int x = 0; x < MT; ++x)
#pragma unroll
        for (int y = 0; y < WN; ++y)
            acc[x][y] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i)
        if (i < T)
            lds_issue_stage<F, KW, WAVES_M, WAVES_N, MT, WN, SPS>(smem + i * G::STAGE_BYTES, i, wave,
                                                                  lane, mrows, nrows, ra, rb, rsa,
                                                                  rsb, p);
    for (int t = 0; t < T; ++t) {
        const int later = min(STAGES - 2, T - 1 - t);
        wait_stage<G::LPS, STAGES>(later);
        block_barrier();
        const int nt = t + STAGES - 1;
        if (nt < T)
            lds_issue_stage<F, KW, WAVES_M, WAVES_N, MT, WN, SPS>(
                smem + (nt % STAGES) * G::STAGE_BYTES, nt, wave, lane, mrows, nrows, ra, rb, rsa,
                rsb, p);
        lds_compute_stage<F, KW, WAVES_M, WAVES_N, MT, WN, SPS>(smem + (t % STAGES) * G::STAGE_BYTES,
                                                                kw, wm, wn, r, g, acc);
    }

    const bool vec_ok = (p.N & 3) == 0;
    if constexpr (KW == 1) {
#pragma unroll
        for (int x = 0; x < MT; ++x) {
            const int m = m0 + wm * 16 * MT + 16 * x + r;
#pragma unroll
            for (int y = 0; y < WN; ++y) {
                const int n = n0 + wn * 16 * WN + 16 * y + 4 * g;
                if (m < p.M && n < p.N)
                    store4<OUT>(p.c, p.N, m, n, acc[x][y], vec_ok && n + 3 < p.N);
            }
        }
    } else {
        // Split-K inside the workgroup: partial tiles of the KW groups are
        // summed in LDS in group order 0..KW-1.  Rows padded by 4 floats.
        constexpr int RS = G::BN + 4;
        static_assert((size_t)KW * G::BM * RS * 4 <= (size_t)STAGES * G::STAGE_BYTES,
                      "reduction tile must fit in the stage ring");
        float *red = reinterpret_cast<float *>(smem);
        block_barrier();   // every wave is done reading the ring
#pragma unroll
        for (int x = 0; x < MT; ++x)
#pragma unroll
            for (int y = 0; y < WN; ++y) {
                const int row = wm * 16 * MT + 16 * x + r, col = wn * 16 * WN + 16 * y + 4 * g;
                *reinterpret_cast<v4f *>(&red[(kw * G::BM + row) * RS + col]) = acc[x][y];
            }
        __syncthreads();
        constexpr int NQ = G::BM * (G::BN / 4);
        for (int q = threadIdx.x; q < NQ; q += 64 * G::NW) {
            const int row = q / (G::BN / 4), c4 = q % (G::BN / 4);
            v4f sum = *reinterpret_cast<const v4f *>(&red[row * RS + 4 * c4]);
#pragma unroll
            for (int k = 1; k < KW; ++k)
                sum += *reinterpret_cast<const v4f *>(&red[(k * G::BM + row) * RS + 4 * c4]);
            const int m = m0 + row, n = n0 + 4 * c4;
            if (m < p.M && n < p.N)
                store4<OUT>(p.c, p.N, m, n, sum, vec_ok && n + 3 < p.N);
        }
    }
}

}  // namespace mxg
