// lds_dma.h -- global -> LDS loads that bypass the registers on gfx950
// (buffer_load_dwordx4 ... lds), shared by the MFMA GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Buffer resource for raw 32-bit byte offsets from a wave-uniform base (gfx9
// descriptor: 48-bit base, stride 0, raw dword format).  num_records bounds
// the per-lane offset: a lane whose offset lies at or past it reads zeros
// (and touches no memory); the default leaves the range open.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t num_records = 0xffffffffu) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = (int32_t)(__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu);
    r[2] = (int32_t)__builtin_amdgcn_readfirstlane(num_records);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from rsrc + soff + voff straight into LDS at lds_base +
// 16 * lane (buffer_load_dwordx4 ... lds; M0 holds the wave-uniform LDS
// address, and one wait state must separate the M0 write from the load).
// Per lane the address is one 32-bit offset register, the per-stage K offset
// rides in soff.  Issued through inline asm so that the compiler's wait-count
// tracking does not treat later LDS reads of other stage buffers as dependent
// on it: the K-loop's explicit vmcnt waits order every fill before the reads
// of its stage.
__device__ __forceinline__ void load_to_lds(i32x4 rsrc, uint32_t voff, uint32_t soff,
                                            uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_void_t*)p;
}

}  // namespace moe
