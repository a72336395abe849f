// lds_dma.h -- direct global -> LDS copies and the explicit waits that go
// with them, shared by the tile prefill and the tile scoring kernels.
// Internal to libbsa.
//
// The copies (global_load_lds_dwordx4) are opaque to the compiler: it adds no
// waits for them, so a kernel can keep several staging buffers in flight and
// wait for exactly the one it reads next.  They write no register; the
// compiler's own memory waits can only become stricter because of them.
#pragma once

#include "bsa_internal.h"

namespace bsa {

// s_waitcnt vmcnt(n) alone (expcnt / lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) alone
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier for the staging pipeline.  __syncthreads() would also wait
// for this wave's copies still in flight to a different buffer (vmcnt(0));
// here every wave has already waited for exactly what the next phase reads
// (its own copies, vmcnt; its LDS reads and writes, lgkmcnt), and the empty
// asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void stage_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// LDS byte address of a __shared__ pointer
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One 16-byte-per-lane copy global -> LDS (lane l to lds + 16 l).  Written as
// an opaque statement: the compiler does not track it, so it adds no wait of
// its own before later LDS reads of other buffers; the kernel waits for these
// copies explicitly (vmcnt) before the barrier that publishes a buffer.  It
// writes no register, and the compiler's own counter waits only get stricter.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
    __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
}

// The same copy from a wave-uniform base plus a 32-bit per-lane byte offset
// (the scalar-base address form: no 64-bit address arithmetic per lane).
__device__ __forceinline__ void dma16_sbase(const void *base, uint32_t off, uint32_t lds) {
    __asm__ volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "s"(lds)
                     : "memory", "m0");
}

}  // namespace bsa
