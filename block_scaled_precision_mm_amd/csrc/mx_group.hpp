// mx_group.hpp -- grouped (mixture-of-experts) form of the NT MX GEMM:
// one launch multiplies every group's rows of A by that group's B.
//
// The operation ("PyTorch 接上 FlyDSL", 5ulink.com: the support-matrix row
// "Grouped GEMM" -- F.grouped_mm, groups of A may have different lengths and
// empty groups are skipped -- and the roadmap item "MXFP8 Grouped GEMM" in
// the closing paragraph): A is [total_rows][K] with the rows of group g at
// [offs[g-1], offs[g]) (offs[-1] = 0), B is [groups][N][K] (one NT operand
// per group, scales [groups][N][K/32]), C is [total_rows][N], and
//   C[rows of g] = A[rows of g] * B[g]^T
// with the same MX arithmetic as the plain product.  Rows of C that no
// group covers are not written.
//
// Work units.  A kernel that tiles one product into units (an M tile times
// all its N tiles, or a single M tile) covers the grouped product with a
// grid sized for the worst case, sum over groups of ceil(rows_g / BM) <=
// ceil(total_rows / BM) + groups M tiles; each workgroup finds its group and
// its unit inside the group from offs, which stays in device memory (no
// host synchronisation), and a workgroup past the last unit exits at once.
// Empty groups own no unit.  The lookup is one pass of a wave over offs,
// 64 groups per iteration: a prefix maximum makes the group ends
// non-decreasing and clamps them into [0, total_rows] (so any offs gives
// in-bounds rows; a decreasing entry makes an empty group), then a prefix
// sum of the units per group and a ballot find the owner.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_common.hpp"

namespace mxg {

// Inclusive wave-wide scans over the 64 lanes (log-step, through ds_bpermute).
__device__ __forceinline__ int wave_scan_max(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d, 64);
        if (lane >= d)
            v = max(v, t);
    }
    return v;
}

__device__ __forceinline__ int wave_scan_add(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d, 64);
        if (lane >= d)
            v += t;
    }
    return v;
}

// Find the group that owns work unit u.  A group of m rows owns
// units_per_mtile * ceil(m / bm) consecutive units, in group order.  On
// success sets the group, the unit's index inside the group and the group's
// first row and row count (all wave-uniform) and returns true; returns
// false when u is past the last unit.  Every lane of the wave must call it.
__device__ __forceinline__ bool find_group(const int *offs, int groups, int total_rows, int u, int bm,
                                           int units_per_mtile, int &grp, int &local, int &row0,
                                           int &rows)
{
    const int lane = threadIdx.x & 63;
    int base = 0;       // units owned by the groups of earlier chunks
    int prev_end = 0;   // clamped end of the last group of the previous chunk
    for (int c0 = 0; c0 < groups; c0 += 64) {
        const int i = c0 + lane;
        const int raw = i < groups ? offs[i] : 0;
        // group ends: prefix maximum (with the previous chunk's end), clamped to total_rows
        const int end = min(max(wave_scan_max(raw, lane), prev_end), total_rows);
        int start = __shfl_up(end, 1, 64);
        if (lane == 0)
            start = prev_end;
        const int m = i < groups ? end - start : 0;
        const int units = units_per_mtile * ((m + bm - 1) / bm);
        const int incl = base + wave_scan_add(units, lane);
        const unsigned long long hit = __ballot(i < groups && incl > u);
        if (hit) {
            const int l = __ffsll((long long)hit) - 1;
            grp = __builtin_amdgcn_readfirstlane(c0 + l);
            local = __builtin_amdgcn_readfirstlane(u - (__shfl(incl, l, 64) - __shfl(units, l, 64)));
            row0 = __builtin_amdgcn_readfirstlane(__shfl(start, l, 64));
            rows = __builtin_amdgcn_readfirstlane(__shfl(m, l, 64));
            return true;
        }
        base = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
        prev_end = __builtin_amdgcn_readfirstlane(__shfl(end, 63, 64));
    }
    return false;
}

// Point the kernel arguments at group grp's operands: its rows of A, C and
// the A scales, and its B and B scales.
template <int OUT>
__device__ __forceinline__ void select_group(GemmArgs &p, int grp, int row0, int rows)
{
    constexpr int ob = OUT == OUT_F32 ? 4 : 2;
    p.a += (size_t)row0 * p.row_bytes;
    p.sa += (size_t)row0 * p.srow_bytes;
    p.b += (size_t)grp * (size_t)p.N * p.row_bytes;
    p.sb += (size_t)grp * (size_t)p.N * p.srow_bytes;
    p.c = static_cast<char *>(p.c) + (size_t)row0 * (size_t)p.N * ob;
    p.M = rows;
}

}  // namespace mxg
