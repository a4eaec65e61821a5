// lds_direct.hpp -- buffer loads straight into LDS and the explicit waits
// that go with them (used by the block-tiled kernel's stage pipeline and by
// the skinny kernel's shared activation rows).
#pragma once

#include "common.hpp"

namespace w4a8 {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer descriptor in SGPRs (raw, stride 0, num_records = bytes).
__device__ __forceinline__ v4i sgpr_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t b = (uint64_t)base;
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// 64 lanes x 16 (or 4) bytes from the buffer into LDS at lds + lane * 16 (or
// 4).  Issued from inline assembly so that the compiler's wait-count pass,
// which cannot tell the stages apart, does not drain every stage in flight
// before each LDS read; the kernel waits explicitly (wait_vmcnt + barrier).
// M0 (the LDS destination) is set inside each block.  The compiler treats M0
// as reserved and ignores the clobber; it sets M0 itself right before any
// instruction of its own that reads it, and in these kernels M0 appears only
// in these sequences, so no value of the compiler's is live across them.
// The scalar offset is wave-uniform by contract; it is made an SGPR value
// (readfirstlane: the compiler may hold a uniform value in a VGPR) and copied
// inside the block (a value it folds to a constant would otherwise be printed
// as a literal, which the soffset field does not take).
__device__ __forceinline__ void lds_load16(const v4i& r, uint32_t lds, uint32_t voff, uint32_t soff)
{
    uint32_t so;
    soff = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %1\n\ts_mov_b32 %0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, %0 offen lds"
                 : "=&s"(so)
                 : "s"(lds), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const v4i& r, uint32_t lds, uint32_t voff, uint32_t soff)
{
    uint32_t so;
    soff = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %1\n\ts_mov_b32 %0, %4\n\ts_nop 0\n\tbuffer_load_dword %2, %3, %0 offen lds"
                 : "=&s"(so)
                 : "s"(lds), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N), leaving the other counters alone
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// A workgroup barrier that is also a compiler memory barrier; it waits for
// this wave's LDS operations (lgkmcnt) and never for the vector-memory
// counter, so the direct-to-LDS loads of the stages still being filled stay
// in flight across it (their waits are the explicit wait_vmcnt above).
__device__ __forceinline__ void barrier()
{
    // this wave's LDS reads are complete before anyone may overwrite them
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace w4a8
