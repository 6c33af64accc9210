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

// The same load in buffer form, for sources inside one block of at most 4 GiB (a K/V page): the
// block's base address and size in a buffer resource held in SGPRs, and a 32-bit offset per lane
// (buffer_load_dwordx4 ... offen lds). Against the global form it sends one address VGPR per
// lane instead of two and needs no per-load 64-bit address add; loads at offsets at or past
// `bytes` return zeros instead of reading memory. Resource words: base address (low 32 bits),
// base address bits 47-32 with stride 0, the size in bytes, and data format 32 (the format of
// untyped loads; no swizzle, no thread-id offset).
typedef int i32x4_rsrc __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16_page(const void *base, uint32_t bytes, uint32_t offset, uint32_t lds) {
    const uint64_t b = (uint64_t)base;
    i32x4_rsrc r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu));
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(offset), "s"(r), "s"(lds)
                 : "memory", "m0");
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
