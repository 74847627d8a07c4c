// Device-side helpers shared by the gfx950 kernels of the k8v4 attention
// library: vector types, fp16 pair casts, exp2, and the direct global->LDS
// copy used for K/V page staging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define Q8K4V_DEV __device__ __forceinline__

namespace q8k4v {

constexpr float kLog2e = 1.4426950408889634f;

Q8K4V_DEV f16x2 as_h2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }
Q8K4V_DEV uint32_t as_u32(f16x2 x) { return __builtin_bit_cast(uint32_t, x); }

Q8K4V_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Direct global -> LDS copy of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): lane i's 16 bytes at sbase + voff land at LDS
// address lds_base + 16 * i.  Written as inline asm so that the compiler does
// not treat the pending copy as aliasing every later LDS access (its own
// tracking would insert a full vmcnt wait before them); completion is waited
// for explicitly (s_waitcnt vmcnt) before the staged bytes are read.  No
// VGPR is written by the instruction.
// ---------------------------------------------------------------------------
Q8K4V_DEV uint32_t sgpr(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
Q8K4V_DEV const void* sgpr_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint64_t lo = sgpr((uint32_t)v), hi = sgpr((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(lo | (hi << 32));
}
// sbase and lds_base must be wave-uniform; they are moved to SGPRs here.
Q8K4V_DEV void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(sgpr(lds_base)), "v"(voff), "s"(sgpr_ptr(sbase)) : "memory");
}
Q8K4V_DEV void wait_lds_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
Q8K4V_DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

Q8K4V_DEV float h2f(uint16_t bits) { return (float)__builtin_bit_cast(_Float16, bits); }

Q8K4V_DEV float bf16_to_f32(uint16_t bits) { return __builtin_bit_cast(float, (uint32_t)bits << 16); }

}  // namespace q8k4v
