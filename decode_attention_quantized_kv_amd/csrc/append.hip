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
// Affine variant (the same page calls the codec affine): unsigned codes with
// a zero point over the block's range widened to include zero,
//   lo = min(min x, 0), hi = max(max x, 0), s = fp16_rne((hi - lo) / q),
//   z = clamp(rint(-lo / s), 0, q), code = clamp(rint(x / s) + z, 0, q),
// q = 255 for keys and 15 for values; s == 0 -> code and zero point 0.  Key
// code and zero point bytes are stored XOR 0x80 (the value minus 128 as
// int8, ready for the signed int8 MFMA); value nibbles and value zero points
// are unsigned.
//
// One wavefront quantizes one (token, kv head): lane i holds dimensions
// (D/64)*i .. (D/64)*i + D/64 - 1.  Value codes of two tokens share a byte
// (slots 2j and 2j+1 of a page, dimension-major rows); when both tokens of a
// pair are new in the same call, the even token's wavefront quantizes the odd
// token's values too and writes the whole byte, so no byte has two writers.
#include "codec_device.h"
#include "q8k4v_device.h"
#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

template <int D, bool BF16, bool AFF>
__global__ __launch_bounds__(256) void append_kernel(
    int8_t* __restrict__ k_codes, uint16_t* __restrict__ k_scales,
    uint8_t* __restrict__ v_codes, uint16_t* __restrict__ v_scales,
    int8_t* __restrict__ k_zeros, uint8_t* __restrict__ v_zeros, int32_t H,
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const int32_t* __restrict__ cu_new, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ page_table, int32_t max_pages, int32_t n_seqs,
    int32_t total_new, const int32_t* __restrict__ last_of) {
    constexpr int EPL = D / 64;      // elements per lane
    constexpr int NG = D / 32;       // value groups
    constexpr int LPG = 32 / EPL;    // lanes per value group
    const int lane = threadIdx.x & 63;
    const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (long)total_new * H) return;
    const int tok = (int)(item / H);
    const int h = (int)(item % H);

    int b, first, last, pos;
    if (last_of) {                    // one token per sequence, at position last_of[b] - 1
        b = first = tok;
        last = tok + 1;
        pos = last_of[b] - 1;
    } else {
        // sequence of this token: the largest b with cu_new[b] <= tok
        int lo = 0, hi = n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu_new[mid] <= tok) lo = mid; else hi = mid - 1;
        }
        b = lo;
        first = cu_new[b];
        last = cu_new[b + 1];
        pos = start_pos[b] + (tok - first);
    }
    const int page = page_table[(size_t)b * max_pages + (pos >> 4)];
    const int slot = pos & 15;
    const size_t blk = (size_t)page * H + h;

    // ---- keys ------------------------------------------------------------
    float kx[EPL];
    load_row<D, BF16>(k_new, (size_t)tok * H + h, lane, kx);
    int8_t* krow = k_codes + (blk * 16 + slot) * D + EPL * lane;
    if (AFF) {
        float mn = kx[0], mx = kx[0];
#pragma unroll
        for (int e = 1; e < EPL; ++e) { mn = fminf(mn, kx[e]); mx = fmaxf(mx, kx[e]); }
        const Affine a = affine_of(wave_min(mn, 64), wave_max(mx, 64), 255.0f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) krow[e] = (int8_t)(affine_code(kx[e], a, 255.0f) ^ 0x80);
        if (lane == 0) {
            k_scales[blk * 16 + slot] = __builtin_bit_cast(uint16_t, a.s16);
            k_zeros[blk * 16 + slot] = (int8_t)((int)a.z ^ 0x80);
        }
    } else {
        float ka = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) ka = fmaxf(ka, fabsf(kx[e]));
        ka = wave_max(ka, 64);
        const _Float16 ks16 = scale_of(ka, 127.0f);
        const float ks = (float)ks16;
#pragma unroll
        for (int e = 0; e < EPL; ++e) krow[e] = (int8_t)code_of(kx[e], ks, 127.0f);
        if (lane == 0) k_scales[blk * 16 + slot] = __builtin_bit_cast(uint16_t, ks16);
    }

    // ---- values ----------------------------------------------------------
    float vx[EPL];
    load_row<D, BF16>(v_new, (size_t)tok * H + h, lane, vx);
    int c[EPL];
    _Float16 vs16;
    int vz;
    value_codes<EPL, LPG, AFF>(vx, c, &vs16, &vz);
    const int g = lane / LPG;
    if ((lane % LPG) == 0) {
        v_scales[(blk * 16 + slot) * NG + g] = __builtin_bit_cast(uint16_t, vs16);
        if (AFF) v_zeros[(blk * 16 + slot) * NG + g] = (uint8_t)vz;
    }

    const bool odd = slot & 1;
    const bool pair_new = odd ? (tok - 1 >= first) : (tok + 1 < last);
    if (odd && pair_new) return;                  // the even token writes this byte
    int c2[EPL];
    if (!odd && pair_new) {                       // quantize the odd neighbour's values
        float wx[EPL];
        load_row<D, BF16>(v_new, (size_t)(tok + 1) * H + h, lane, wx);
        _Float16 ws16;
        int wz;
        value_codes<EPL, LPG, AFF>(wx, c2, &ws16, &wz);
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
#define Q8K4V_APPEND(DD, BB, AA)                                                                      \
    hipLaunchKernelGGL((append_kernel<DD, BB, AA>), grid, block, 0, stream, c.k_codes, c.k_scales,    \
                       c.v_codes, c.v_scales, c.k_zeros, c.v_zeros, c.num_kv_heads, a.k_new, a.v_new, \
                       a.cu_new, a.start_pos, a.page_table, a.max_pages, a.n_seqs, a.total_new, a.last_of)
    const bool bf = a.dtype == Q8K4V_BF16;
    const bool aff = c.codec == Q8K4V_CODEC_AFFINE;
    if (c.head_dim == 128) {
        if (aff) { if (bf) Q8K4V_APPEND(128, true, true); else Q8K4V_APPEND(128, false, true); }
        else { if (bf) Q8K4V_APPEND(128, true, false); else Q8K4V_APPEND(128, false, false); }
    } else {
        if (aff) { if (bf) Q8K4V_APPEND(64, true, true); else Q8K4V_APPEND(64, false, true); }
        else { if (bf) Q8K4V_APPEND(64, true, false); else Q8K4V_APPEND(64, false, false); }
    }
#undef Q8K4V_APPEND
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "kv_quant_append launch");
    return Q8K4V_OK;
}

}  // namespace q8k4v
