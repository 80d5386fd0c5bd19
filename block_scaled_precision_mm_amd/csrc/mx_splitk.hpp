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
//   * those stores, the tile's arrival counter and the reads below are
//     device-scope accesses (coherent across MI355X's XCDs, whose L2s are
//     not coherent with each other for ordinary accesses) -- no fence, so
//     no workgroup writes back or invalidates a whole L2, which made the
//     first version of this scheme ten times slower than no split at all;
//     each thread waits for its stores to complete before the workgroup
//     bumps the counter with a device-scope atomic add;
//   * the workgroup that sees S-1 arrivals before its own is the last: it
//     adds the S parts in part order 0, 1, .., S-1 (the others' read back
//     from their slots, its own from its registers at its place in that
//     order), so the sequence of FP32 additions is the same whoever
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
    __shared__ unsigned arrived;
    const int S = p.splits, part = (int)blockIdx.z;
    float *slots = p.ws + (size_t)tile * S * FL;
    // slot layout [piece j][float e][thread]: every store and load below
    // moves 256 contiguous bytes per wave
    float *mine = slots + (size_t)part * FL;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const v4f v = get(j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            __hip_atomic_store(mine + (4 * j + e) * NTHR + tid, v[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // this thread's stores have completed (device-wide visible) before the
    // workgroup's arrival is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
        arrived = __hip_atomic_fetch_add(p.flags + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != (unsigned)(S - 1))
        return false;
    // the last part: sum in part order, every part (its own too, stored
    // above) read back, so no piece is needed in registers past its store
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        v4f sum;
        for (int q = 0; q < S; ++q) {
            const float *src = slots + (size_t)q * FL + 4 * j * NTHR + tid;
            v4f v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = __hip_atomic_load(src + e * NTHR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sum = q == 0 ? v : sum + v;
        }
        set(j, sum);
    }
    if (tid == 0)
        __hip_atomic_store(p.flags + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

}  // namespace mxg
