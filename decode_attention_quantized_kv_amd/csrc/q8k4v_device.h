// Device-side helpers shared by the gfx950 kernels of the k8v4 attention
// library: vector types, fp16 dot products, code unpacking, DPP row
// reductions and the direct global->LDS copy used for K/V page staging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define Q8K4V_DEV __device__ __forceinline__

namespace q8k4v {

constexpr float kLog2e = 1.4426950408889634f;

Q8K4V_DEV f16x2 as_h2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }
Q8K4V_DEV uint32_t as_u32(f16x2 x) { return __builtin_bit_cast(uint32_t, x); }

// fp32 += a.x*b.x + a.y*b.y with fp16 operands (v_dot2_f32_f16): the products
// of two fp16 values are exact in fp32.
Q8K4V_DEV float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// ---------------------------------------------------------------------------
// Key codes: four int8 codes (two's complement) -> two fp16 pairs holding
// 1152 + code (exact: 1025..1279 lies where fp16 has unit spacing).  XOR 0x80
// turns the byte into code + 128; placing it under the fp16 exponent byte
// 0x64 gives the value 1024 + code + 128.
// ---------------------------------------------------------------------------
Q8K4V_DEV void k_codes_to_f16(uint32_t x, uint32_t& lo, uint32_t& hi) {
    const uint32_t xb = x ^ 0x80808080u;
    lo = __builtin_amdgcn_perm(0x64646464u, xb, 0x04010400u);   // (c0, c1)
    hi = __builtin_amdgcn_perm(0x64646464u, xb, 0x04030402u);   // (c2, c3)
}

// Exact fp16 pairs of key codes (bias removed): used where the operand feeds
// an MFMA and no scalar bias correction is possible.
Q8K4V_DEV void k_codes_to_f16_exact(uint32_t x, uint32_t& lo, uint32_t& hi) {
    k_codes_to_f16(x, lo, hi);
    const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    lo = as_u32(as_h2(lo) + bias);
    hi = as_u32(as_h2(hi) + bias);
}

// ---------------------------------------------------------------------------
// Value codes: eight int4 codes of one dimension row (tokens 8k..8k+7, token
// 8k+2i in the low nibble of byte i) -> four exact fp16 pairs
//   out[0] = (t0, t4), out[1] = (t1, t5), out[2] = (t2, t6), out[3] = (t3, t7)
// (t_i relative to 8k).  A nibble n placed under the fp16 exponent 0x64 with
// its top bit flipped reads 1024 + (n ^ 8) = 1032 + code (or 1024 + 16 (n ^ 8)
// one nibble higher); (x & mask) ^ (0x6400 | flip) does mask, flip and
// exponent in one bit operation, and a packed add / fma removes the offset
// exactly.
// ---------------------------------------------------------------------------
Q8K4V_DEV void v_codes_to_f16(uint32_t x, uint32_t out[4]) {
    const uint32_t y = x >> 8;
    const uint32_t a = (x & 0x000F000Fu) ^ 0x64086408u;
    const uint32_t b = (x & 0x00F000F0u) ^ 0x64806480u;
    const uint32_t c = (y & 0x000F000Fu) ^ 0x64086408u;
    const uint32_t d = (y & 0x00F000F0u) ^ 0x64806480u;
    const f16x2 off1 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const f16x2 inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const f16x2 off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    out[0] = as_u32(as_h2(a) + off1);
    out[1] = as_u32(__builtin_elementwise_fma(as_h2(b), inv16, off16));
    out[2] = as_u32(as_h2(c) + off1);
    out[3] = as_u32(__builtin_elementwise_fma(as_h2(d), inv16, off16));
}

// ---------------------------------------------------------------------------
// DPP within a row of 16 lanes
// ---------------------------------------------------------------------------
template <int CTRL>
Q8K4V_DEV float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

Q8K4V_DEV float row16_max(float x) {
    x = fmaxf(x, dpp<kQuadXor1>(x));
    x = fmaxf(x, dpp<kQuadXor2>(x));
    x = fmaxf(x, dpp<kRowHalfMirror>(x));
    x = fmaxf(x, dpp<kRowMirror>(x));
    return x;
}
Q8K4V_DEV float row16_sum(float x) {
    x += dpp<kQuadXor1>(x);
    x += dpp<kQuadXor2>(x);
    x += dpp<kRowHalfMirror>(x);
    x += dpp<kRowMirror>(x);
    return x;
}
// max / sum over aligned groups of N lanes (N in 1,2,4,8,16)
template <int N>
Q8K4V_DEV float group_max(float x) {
    if (N >= 2) x = fmaxf(x, dpp<kQuadXor1>(x));
    if (N >= 4) x = fmaxf(x, dpp<kQuadXor2>(x));
    if (N >= 8) x = fmaxf(x, dpp<kRowHalfMirror>(x));
    if (N >= 16) x = fmaxf(x, dpp<kRowMirror>(x));
    return x;
}
template <int N>
Q8K4V_DEV float group_sum(float x) {
    if (N >= 2) x += dpp<kQuadXor1>(x);
    if (N >= 4) x += dpp<kQuadXor2>(x);
    if (N >= 8) x += dpp<kRowHalfMirror>(x);
    if (N >= 16) x += dpp<kRowMirror>(x);
    return x;
}

Q8K4V_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Direct global -> LDS copy of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): lane i's 16 bytes at sbase + voff land at LDS
// address lds_base + 16 * i.  Written as inline asm so that the compiler does
// not treat the pending copy as aliasing every later LDS access (its own
// tracking would insert a full vmcnt wait before them); completion is waited
// for explicitly with wait_vmem_all() before the staged bytes are read.  No
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
// Per-lane 64-bit global address; lds_base wave-uniform.
Q8K4V_DEV void lds_dma16_vaddr(const void* addr, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(sgpr(lds_base)), "v"(addr) : "memory");
}
Q8K4V_DEV void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
Q8K4V_DEV void wait_lds_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
Q8K4V_DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

Q8K4V_DEV float h2f(uint16_t bits) { return (float)__builtin_bit_cast(_Float16, bits); }

Q8K4V_DEV float bf16_to_f32(uint16_t bits) { return __builtin_bit_cast(float, (uint32_t)bits << 16); }

}  // namespace q8k4v
