// Direct global-to-LDS loads for gfx950 (CDNA4), shared by the attention and decoder-layer kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace piclink {

// Work-group barrier of the direct-load kernels: this wave's LDS operations complete (lgkmcnt),
// then s_barrier; the memory clobber keeps the compiler from moving memory accesses across it. A
// memory fence would also wait for every direct load in flight (they are LDS writes to the memory
// model) and expose their latency at every barrier: the loads a barrier has to cover are waited
// for with an explicit vmcnt before it.
__device__ __forceinline__ void barrier_dl() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One direct load: 16 bytes per lane from `src` into LDS at byte lds + 16 * lane (global_load_lds
// with its LDS base in M0). Issued from asm, so the compiler does not track it: the kernel waits
// for its loads itself (vmcnt) before the barriers that publish them. Loads the compiler does not
// count can only make its own vmcnt waits for other loads stricter, never too weak (they
// complete in order).
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}

// LDS byte address of a __shared__ location.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const void __attribute__((address_space(3))) *)p;
}

// s_waitcnt vmcnt(N) with lgkmcnt and expcnt left at their maxima (gfx9 encoding: vmcnt low bits
// 3:0, high bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace piclink
