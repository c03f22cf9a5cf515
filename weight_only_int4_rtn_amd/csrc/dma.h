// Direct global -> LDS copies and explicit waits, shared by the streaming kernels.
#pragma once
#include "common.h"

namespace w4a16 {
namespace {

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }
// Workgroup barrier that orders the compiler's memory accesses but waits for nothing
// (the waits are explicit).
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }

// Direct global -> LDS copies (buffer_load ... lds: lane l's 16 or 4 bytes land at the
// wave-uniform LDS address + 16 l or + 4 l).  Issued from inline asm so that the compiler,
// which cannot tell the stages apart, does not wait for every copy in flight before each
// LDS read; the step waits above carry the ordering instead.  The copies write no
// registers.  Buffer descriptor: base, num_records = bytes, gfx9-family word 3.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t dma_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    return i32x4_t{(int32_t)(uint32_t)a, (int32_t)((uint32_t)(a >> 32) & 0xffffu), (int32_t)bytes, 0x00020000};
}
// The same descriptor held in scalar registers (its parts must be wave-uniform).
__device__ __forceinline__ i32x4_t uniform_rsrc(i32x4_t r) {
    return i32x4_t{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                   __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}
// LDS byte address of a pointer into shared memory (wave-uniform).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}
// The LDS address and the scalar offset are wave-uniform by contract; readfirstlane says
// so where the compiler cannot prove it (it folds away where it can).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is set here, on purpose
__device__ __forceinline__ void dma16(i32x4_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(i32x4_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
// The same copies without a memory clobber, for a pipeline whose LDS reads never touch
// the stage being filled and whose barriers and waits carry every ordering: the compiler
// may then schedule LDS reads and arithmetic around them.
__device__ __forceinline__ void dma16_free(i32x4_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)) : "m0");
}
__device__ __forceinline__ void dma4_free(i32x4_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)) : "m0");
}
#pragma clang diagnostic pop

constexpr uint32_t kOob = 0x80000000u;   // a buffer offset past every staged array: reads zero

// s_waitcnt vmcnt(n) for a wave-uniform n that is only known at run time (0..63).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    switch (n) {
#define W4A16_VMCNT_CASE(k) case k: wait_vmcnt<k>(); break;
        W4A16_VMCNT_CASE(1) W4A16_VMCNT_CASE(2) W4A16_VMCNT_CASE(3) W4A16_VMCNT_CASE(4) W4A16_VMCNT_CASE(5)
        W4A16_VMCNT_CASE(6) W4A16_VMCNT_CASE(7) W4A16_VMCNT_CASE(8) W4A16_VMCNT_CASE(9) W4A16_VMCNT_CASE(10)
        W4A16_VMCNT_CASE(11) W4A16_VMCNT_CASE(12) W4A16_VMCNT_CASE(13) W4A16_VMCNT_CASE(14) W4A16_VMCNT_CASE(15)
        W4A16_VMCNT_CASE(16) W4A16_VMCNT_CASE(17) W4A16_VMCNT_CASE(18) W4A16_VMCNT_CASE(19) W4A16_VMCNT_CASE(20)
        W4A16_VMCNT_CASE(21) W4A16_VMCNT_CASE(22) W4A16_VMCNT_CASE(23) W4A16_VMCNT_CASE(24) W4A16_VMCNT_CASE(25)
        W4A16_VMCNT_CASE(26) W4A16_VMCNT_CASE(27) W4A16_VMCNT_CASE(28) W4A16_VMCNT_CASE(29) W4A16_VMCNT_CASE(30)
        W4A16_VMCNT_CASE(31) W4A16_VMCNT_CASE(32) W4A16_VMCNT_CASE(33) W4A16_VMCNT_CASE(34) W4A16_VMCNT_CASE(35)
        W4A16_VMCNT_CASE(36) W4A16_VMCNT_CASE(37) W4A16_VMCNT_CASE(38) W4A16_VMCNT_CASE(39) W4A16_VMCNT_CASE(40)
        W4A16_VMCNT_CASE(41) W4A16_VMCNT_CASE(42) W4A16_VMCNT_CASE(43) W4A16_VMCNT_CASE(44) W4A16_VMCNT_CASE(45)
        W4A16_VMCNT_CASE(46) W4A16_VMCNT_CASE(47) W4A16_VMCNT_CASE(48) W4A16_VMCNT_CASE(49) W4A16_VMCNT_CASE(50)
        W4A16_VMCNT_CASE(51) W4A16_VMCNT_CASE(52) W4A16_VMCNT_CASE(53) W4A16_VMCNT_CASE(54) W4A16_VMCNT_CASE(55)
        W4A16_VMCNT_CASE(56) W4A16_VMCNT_CASE(57) W4A16_VMCNT_CASE(58) W4A16_VMCNT_CASE(59) W4A16_VMCNT_CASE(60)
        W4A16_VMCNT_CASE(61) W4A16_VMCNT_CASE(62) W4A16_VMCNT_CASE(63)
#undef W4A16_VMCNT_CASE
        default: wait_vmcnt<0>(); break;
    }
}

}  // namespace
}  // namespace w4a16
