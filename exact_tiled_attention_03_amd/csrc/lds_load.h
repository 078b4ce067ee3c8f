// lds_load.h -- direct HBM -> LDS loads (buffer_load_dword{,x4} ... lds) for gfx950.
//
// Lane i's bytes, read at buffer offset voff + soff, land at LDS address
// lds_dst + size * i (lds_dst wave-uniform, passed through M0).  Offsets at or
// past the descriptor's size read as zero.
//
// M0 carries the LDS destination.  gfx950 needs one wait state between an SALU
// write of M0 and an LDS-DMA load that reads it; the compiler inserts it for its
// own loads but cannot see inside inline assembly, so each sequence below
// carries its own s_nop 0.
//
// Written as inline assembly: when the compiler sees these loads as builtins it
// treats them as pending LDS stores, so it makes every later LDS transpose read
// and every work-group barrier wait for all of them (including prefetches of
// tiles that the read or the barrier has nothing to do with).  The kernels that
// use these order the loads themselves: a wait on the vector-memory counter
// (wait_vmcnt) for this wave's loads, then a barrier, before any wave reads the
// tile.
#ifndef ETA_LDS_LOAD_H
#define ETA_LDS_LOAD_H

#include <hip/hip_runtime.h>

typedef int eta_desc_t __attribute__((ext_vector_type(4)));

#if defined(__HIP_DEVICE_COMPILE__)

// Raw buffer descriptor of `bytes` bytes at `base` (readfirstlane: the values are
// wave-uniform, and the assembly needs them in scalar registers)
__device__ __forceinline__ eta_desc_t buffer_desc(const void* base, int bytes) {
    const unsigned long long p = (unsigned long long)base;
    return eta_desc_t{__builtin_amdgcn_readfirstlane((int)(unsigned)p),
                      __builtin_amdgcn_readfirstlane((int)((unsigned)(p >> 32) & 0xffffu)),
                      __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

__device__ __forceinline__ void load_lds16(const eta_desc_t& desc, unsigned voff, unsigned soff, unsigned lds_dst) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(desc),
                 "s"(__builtin_amdgcn_readfirstlane(soff)), "s"(__builtin_amdgcn_readfirstlane(lds_dst))
                 : "memory");
}

__device__ __forceinline__ void load_lds4(const eta_desc_t& desc, unsigned voff, unsigned lds_dst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(desc),
                 "s"(__builtin_amdgcn_readfirstlane(lds_dst))
                 : "memory");
}

// wait until at most N of this wave's vector-memory loads are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

#endif  // __HIP_DEVICE_COMPILE__
#endif  // ETA_LDS_LOAD_H
