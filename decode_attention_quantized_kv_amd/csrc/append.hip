// Quantize-and-append of new key/value tokens into the paged k8v4 cache.
//
// Codec (blog.123qwe.co.kr/?p=3927, section 5: 8-bit keys, 4-bit values in
// groups of 32 with fp16 scales), symmetric absmax reading:
//   keys, per (token, kv head):            s = fp16_rne(max|x| / 127)
//   values, per (token, kv head, group):   s = fp16_rne(max|x| / 7)
//   code = clamp(rint_half_even(x / s), -q, q); fp16 overflow of s -> 65504;
//   s == 0 -> all codes 0.
// Both divisions are IEEE fp32 divisions (HIP's default correctly rounded
// '/'), rintf is round-half-even and fp16 subnormal scales are kept, so the
// codes and scales are bit-identical to any other implementation of the same
// rule.
//
// One wavefront quantizes one (token, kv head): lane i holds dimensions
// (D/64)*i .. (D/64)*i + D/64 - 1.  Value codes of two tokens share a byte
// (slots 2j and 2j+1 of a page, dimension-major rows); when both tokens of a
// pair are new in the same call, the even token's wavefront quantizes the odd
// token's values too and writes the whole byte, so no byte has two writers.
#include "q8k4v_device.h"
#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

template <int D, bool BF16>
Q8K4V_DEV void load_row(const void* base, size_t row, int lane, float (&x)[D / 64]) {
    constexpr int EPL = D / 64;
    if (BF16) {
        const uint16_t* p = (const uint16_t*)base + row * D + EPL * lane;
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = bf16_to_f32(p[e]);
    } else {
        const float* p = (const float*)base + row * D + EPL * lane;
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = p[e];
    }
}

Q8K4V_DEV float wave_max(float x, int lanes) {
    for (int m = 1; m < lanes; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

// fp16 scale of an absmax: IEEE fp32 division, RNE into fp16, saturating.
Q8K4V_DEV _Float16 scale_of(float absmax, float qmax) {
    const float s32 = absmax / qmax;
    _Float16 s16 = (_Float16)s32;
    if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;
    return s16;
}

Q8K4V_DEV int code_of(float x, float s, float qmax) {
    if (s == 0.0f) return 0;
    float r = rintf(x / s);
    r = fminf(fmaxf(r, -qmax), qmax);
    return (int)r;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void append_kernel(
    int8_t* __restrict__ k_codes, uint16_t* __restrict__ k_scales,
    uint8_t* __restrict__ v_codes, uint16_t* __restrict__ v_scales, int32_t H,
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const int32_t* __restrict__ cu_new, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ page_table, int32_t max_pages, int32_t n_seqs,
    int32_t total_new) {
    constexpr int EPL = D / 64;      // elements per lane
    constexpr int NG = D / 32;       // value groups
    constexpr int LPG = 32 / EPL;    // lanes per value group
    const int lane = threadIdx.x & 63;
    const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (long)total_new * H) return;
    const int tok = (int)(item / H);
    const int h = (int)(item % H);

    // sequence of this token: the largest b with cu_new[b] <= tok
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_new[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int first = cu_new[b];
    const int last = cu_new[b + 1];
    const int pos = start_pos[b] + (tok - first);
    const int page = page_table[(size_t)b * max_pages + (pos >> 4)];
    const int slot = pos & 15;
    const size_t blk = (size_t)page * H + h;

    // ---- keys ------------------------------------------------------------
    float kx[EPL];
    load_row<D, BF16>(k_new, (size_t)tok * H + h, lane, kx);
    float ka = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ka = fmaxf(ka, fabsf(kx[e]));
    ka = wave_max(ka, 64);
    const _Float16 ks16 = scale_of(ka, 127.0f);
    const float ks = (float)ks16;
    int8_t* krow = k_codes + (blk * 16 + slot) * D + EPL * lane;
#pragma unroll
    for (int e = 0; e < EPL; ++e) krow[e] = (int8_t)code_of(kx[e], ks, 127.0f);
    if (lane == 0) k_scales[blk * 16 + slot] = __builtin_bit_cast(uint16_t, ks16);

    // ---- values ----------------------------------------------------------
    float vx[EPL];
    load_row<D, BF16>(v_new, (size_t)tok * H + h, lane, vx);
    float va = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) va = fmaxf(va, fabsf(vx[e]));
    va = wave_max(va, LPG);
    const _Float16 vs16 = scale_of(va, 7.0f);
    const float vs = (float)vs16;
    const int g = lane / LPG;
    if ((lane % LPG) == 0) v_scales[(blk * 16 + slot) * NG + g] = __builtin_bit_cast(uint16_t, vs16);
    int c[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) c[e] = code_of(vx[e], vs, 7.0f);

    const bool odd = slot & 1;
    const bool pair_new = odd ? (tok - 1 >= first) : (tok + 1 < last);
    if (odd && pair_new) return;                  // the even token writes this byte
    int c2[EPL];
    if (!odd && pair_new) {                       // quantize the odd neighbour's values
        float wx[EPL];
        load_row<D, BF16>(v_new, (size_t)(tok + 1) * H + h, lane, wx);
        float wa = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) wa = fmaxf(wa, fabsf(wx[e]));
        wa = wave_max(wa, LPG);
        const float ws = (float)scale_of(wa, 7.0f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) c2[e] = code_of(wx[e], ws, 7.0f);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int d = EPL * lane + e;
        uint8_t* p = v_codes + (blk * D + d) * 8 + (slot >> 1);
        uint32_t byte;
        if (!odd && pair_new) {
            byte = (uint32_t)(c[e] & 0xF) | ((uint32_t)(c2[e] & 0xF) << 4);
        } else if (!odd) {
            byte = (*p & 0xF0u) | (uint32_t)(c[e] & 0xF);
        } else {
            byte = (*p & 0x0Fu) | ((uint32_t)(c[e] & 0xF) << 4);
        }
        *p = (uint8_t)byte;
    }
}

}  // namespace

int32_t launch_append(const AppendArgs& a, hipStream_t stream) {
    const q8k4v_cache& c = *a.cache;
    if (a.total_new == 0) return Q8K4V_OK;
    const long items = (long)a.total_new * c.num_kv_heads;
    const long blocks = (items + 3) / 4;
    if (blocks > 0x7FFFFFFFL) return fail(Q8K4V_EINVAL, "kv_quant_append: too many tokens in one call");
    dim3 grid((unsigned)blocks), block(256);
#define Q8K4V_APPEND(DD, BB)                                                                   \
    hipLaunchKernelGGL((append_kernel<DD, BB>), grid, block, 0, stream, c.k_codes, c.k_scales, \
                       c.v_codes, c.v_scales, c.num_kv_heads, a.k_new, a.v_new, a.cu_new,     \
                       a.start_pos, a.page_table, a.max_pages, a.n_seqs, a.total_new)
    const bool bf = a.dtype == Q8K4V_BF16;
    if (c.head_dim == 128) {
        if (bf) Q8K4V_APPEND(128, true); else Q8K4V_APPEND(128, false);
    } else {
        if (bf) Q8K4V_APPEND(64, true); else Q8K4V_APPEND(64, false);
    }
#undef Q8K4V_APPEND
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "kv_quant_append launch");
    return Q8K4V_OK;
}

}  // namespace q8k4v
