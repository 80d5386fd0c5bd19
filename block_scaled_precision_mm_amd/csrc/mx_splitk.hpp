// mx_splitk.hpp -- split-K across workgroups for the NT MX GEMM, gfx950.
//
// Small-M products have too few output tiles to give every compute unit
// work.  Split-K cuts K into S parts: the launch grid gets a third
// dimension, and workgroup (tile, s) computes the tile's partial product
// over K part s.  The parts are then summed with a fixed order, so the
// result does not depend on which workgroup finishes last:
//
//   * every workgroup writes its FP32 partial tile to its own slot of a
//     workspace the caller provides (part s of tile t), in the thread layout
//     it holds it in (so the write is coalesced and no workgroup needs
//     another's layout);
//   * those stores and the reads below carry the cache policy of
//     device-scope accesses (write through / read past the XCD's L2:
//     MI355X's eight L2s are not coherent with each other for ordinary
//     accesses), 16 bytes per thread each, and the tile's arrival counter
//     is a device-scope atomic -- no fence, so no workgroup writes back or
//     invalidates a whole L2, which made the first version of this scheme
//     ten times slower than no split at all (dword-sized accesses cost the
//     last workgroup of a tile another factor of two to four at eight
//     parts); each thread waits for its stores to complete before the
//     workgroup bumps the counter;
//   * the workgroup that sees S-1 arrivals before its own is the last: it
//     reads the S parts back (its own too) and adds them in part order
//     0, 1, .., S-1, so the sequence of FP32 additions is the same whoever
//     arrives last; it resets the counter to zero for the next call on the
//     same workspace, and stores the sum through the kernel's normal
//     epilogue.  The others exit.  No workgroup ever waits for another.
//
// K parts are whole multiples of `gran` 128-K steps (the kernel's natural
// period: its scale codes come 16 bytes, i.e. four steps, per row at a
// time), balanced to within one such unit.
//
// Workspace layout: a fixed counter region (kSplitCounters uint32, zero
// before the first call and left at zero by every call) that partial tiles
// never overlap, whatever configuration used the workspace before; then the
// partial tiles, [tile][part][TILE floats].  Concurrent calls must use
// different workspaces.
#pragma once

#include "mx_common.hpp"

namespace mxg {

// Counters at the start of every split-K workspace: split-K runs only on
// launches of at most this many output tiles.
constexpr int kSplitCounters = 16384;

// 128-K steps [s0, s1) of part `part` of `parts` over `nsteps` steps, in
// whole units of `gran` steps.
__device__ __forceinline__ void split_steps(int nsteps, int parts, int part, int gran, int &s0, int &s1)
{
    const int units = (nsteps + gran - 1) / gran;
    const int u0 = (int)(((long long)part * units) / parts);
    const int u1 = (int)(((long long)(part + 1) * units) / parts);
    s0 = min(u0 * gran, nsteps);
    s1 = min(u1 * gran, nsteps);
}

// Narrow the arguments to this workgroup's K part (blockIdx.z): operand and
// scale pointers move to the part's first step, nsteps and kbytes become
// the part's.  row_bytes and srow_bytes stay the row strides.
template <int F>
__device__ __forceinline__ void select_split(GemmArgs &p, int gran)
{
    if (p.splits <= 1)
        return;
    int s0, s1;
    split_steps(p.nsteps, p.splits, (int)blockIdx.z, gran, s0, s1);
    constexpr int SB = FmtTraits<F>::step_bytes;
    p.a += (size_t)s0 * SB;
    p.b += (size_t)s0 * SB;
    p.sa += (size_t)s0 * 4;
    p.sb += (size_t)s0 * 4;
    p.nsteps = s1 - s0;
    p.kbytes = (unsigned)(s1 - s0) * SB;
}

// Buffer range of `rows` rows of stride `stride` of which the first
// `extent` bytes belong to this workgroup's K part: loads past the part's
// end of the last row read zeros instead of whatever follows the operand.
__device__ __forceinline__ unsigned part_range(int rows, unsigned stride, unsigned extent)
{
    return rows > 0 ? (unsigned)(rows - 1) * stride + extent : 0u;
}

// The cross-workgroup reduction of one tile (see the file comment).  Each
// of the NTHR threads holds NV four-float pieces of the partial tile:
// get(j) returns piece j, set(j, v) replaces it.  `tile` is the tile's index
// among the launch's tiles.  Every thread of the workgroup calls it.
// Returns true in the last-arriving workgroup, whose pieces then hold the
// full sum; false elsewhere (the caller exits without storing).
template <int NV, int NTHR, class Get, class Set>
__device__ __forceinline__ bool splitk_reduce(const GemmArgs &p, int tile, int tid, Get &&get, Set &&set)
{
    constexpr int FL = NV * NTHR * 4;   // floats per partial tile
    constexpr int DEV = 16;             // cache policy of a device-scope access
    __shared__ unsigned arrived;
    const int S = p.splits, part = (int)blockIdx.z;
    // slot layout [part][piece j][thread][4 floats]: every access below
    // moves 16 contiguous bytes per thread, 1 KB per wave
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.ws + (size_t)tile * S * FL, (unsigned)(S * FL * 4));
    auto at = [&](int q, int j) { return (unsigned)(((q * NV + j) * NTHR + tid) * 16); };
#pragma unroll
    for (int j = 0; j < NV; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4v, get(j)), rs, at(part, j), 0, DEV);
    // this thread's stores have completed (device-wide visible) before the
    // workgroup's arrival is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
        arrived = __hip_atomic_fetch_add(p.flags + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != (unsigned)(S - 1))
        return false;
    // the last part: sum in part order, JG pieces at a time (their loads
    // in flight together)
    constexpr int JG = NV < 8 ? NV : 8;
#pragma unroll
    for (int j0 = 0; j0 < NV; j0 += JG) {
        v4f sum[JG];
        for (int q = 0; q < S; ++q) {
            v4f v[JG];
#pragma unroll
            for (int jj = 0; jj < JG; ++jj)
                if (j0 + jj < NV)
                    v[jj] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, at(q, j0 + jj), 0, DEV));
#pragma unroll
            for (int jj = 0; jj < JG; ++jj)
                if (j0 + jj < NV)
                    sum[jj] = q == 0 ? v[jj] : sum[jj] + v[jj];
        }
#pragma unroll
        for (int jj = 0; jj < JG; ++jj)
            if (j0 + jj < NV)
                set(j0 + jj, sum[jj]);
    }
    if (tid == 0)
        __hip_atomic_store(p.flags + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

}  // namespace mxg
