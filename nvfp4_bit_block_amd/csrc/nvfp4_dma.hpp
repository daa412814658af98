// nvfp4_dma.hpp -- raw buffer resources and global -> LDS loads for gfx950.
//
// Buffer loads address memory through a 128-bit resource held in scalar
// registers; a load whose offset lies past the resource's range returns
// zeros without a memory access.  The "lds" form of buffer_load writes the
// loaded bytes straight into LDS (lane l at LDS byte address M0 + 16 l, or
// 4 l for dword loads) without passing through VGPRs.
#pragma once

#include "nvfp4_device.hpp"

namespace nvfp4 {

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 raw buffer: 32-bit data, range checked
constexpr uint32_t kOob = 0x80000000u;        // an offset past every buffer built here

// Buffer resource over [base, base + bytes), in scalar registers.  Loads past
// the end return zeros without a memory access.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint64_t bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t n = bytes < 0x80000000ull ? (uint32_t)bytes : 0x80000000u;
    u32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)p);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
    r.z = __builtin_amdgcn_readfirstlane(n);
    r.w = kRsrcWord3;
    return r;
}
// Global -> LDS loads: lane l of the wave writes its 16 (or 4) bytes at LDS
// byte address lds + 16 l (4 l); lds is wave-uniform and travels in M0.
// Written as asm so that the compiler does not make every later LDS read
// wait for them: the K loop waits for them itself (vmcnt) before its
// barrier.  They have no register results.
// The compiler's hazard checks do not see the load inside the asm, so the
// asm supplies the wait states itself: one after the M0 write, and five
// after a VALU write of an SGPR the load reads.  The second case arises
// when the compiler restores a spilled resource word with v_readlane just
// before the asm; without the wait the load can take a stale descriptor
// word and read from a wrong address.
__device__ __forceinline__ void lds_load16(u32x4 r, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_load4(u32x4 r, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_address(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
// s_waitcnt immediate (gfx9) that waits until at most n vector memory
// operations are outstanding, leaving the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

}  // namespace nvfp4
