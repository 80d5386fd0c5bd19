// mx_sync.hpp -- small gfx950 helpers shared by the kernels that stage
// operands through LDS: direct-to-LDS buffer loads, explicit vector-memory
// waits and a workgroup barrier without the full memory fence.
#pragma once

#include "mx_common.hpp"

namespace mxg {

constexpr int cdiv_c(int a, int b) { return (a + b - 1) / b; }

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

// The same wait as an s_waitcnt the compiler sees (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt and lgkmcnt left at their maximum): its own
// bookkeeping of outstanding loads then knows what has landed and adds no
// wait of its own for them.  The empty asm keeps memory accesses on their
// side of it.
template <int N>
__device__ __forceinline__ void wait_vm_known()
{
    static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
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

}  // namespace mxg
