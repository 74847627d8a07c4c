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

#define Q8K4V_APPEND_PARAMS                                                                          \
    int8_t *__restrict__ k_codes, uint16_t *__restrict__ k_scales, uint8_t *__restrict__ v_codes,     \
        uint16_t *__restrict__ v_scales, int8_t *__restrict__ k_zeros, uint8_t *__restrict__ v_zeros,   \
        int32_t H, const void *__restrict__ k_new, const void *__restrict__ v_new,                    \
        const int32_t *__restrict__ cu_new, const int32_t *__restrict__ start_pos,                    \
        const int32_t *__restrict__ page_table, int32_t max_pages, int32_t n_seqs, int32_t total_new,   \
        const int32_t *__restrict__ last_of
#define Q8K4V_APPEND_ARGS                                                                             \
    k_codes, k_scales, v_codes, v_scales, k_zeros, v_zeros, H, k_new, v_new, cu_new, start_pos,         \
        page_table, max_pages, n_seqs, total_new, last_of

// One (token, kv head) by one wavefront: item = token * H + head.
template <int D, bool BF16, bool AFF>
Q8K4V_DEV void append_token(Q8K4V_APPEND_PARAMS, long item, int lane) {
    constexpr int EPL = D / 64;      // elements per lane
    constexpr int NG = D / 32;       // value groups
    constexpr int LPG = 32 / EPL;    // lanes per value group
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

template <int D, bool BF16, bool AFF>
__global__ __launch_bounds__(256) void append_kernel(Q8K4V_APPEND_PARAMS) {
    const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (long)total_new * H) return;
    append_token<D, BF16, AFF>(Q8K4V_APPEND_ARGS, item, threadIdx.x & 63);
}

// EPT consecutive elements of a row (16-byte loads).
template <int D, int EPT, bool BF16>
Q8K4V_DEV void load_seg(const void* base, size_t row, int u, float (&x)[EPT]) {
    if (BF16) {
        const uint16_t* p = (const uint16_t*)base + row * D + EPT * u;
        uint32_t w[EPT / 2];
        if constexpr (EPT == 8) {
            const u32x4 v = *(const u32x4*)p;
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
            const u32x2 v = *(const u32x2*)p;
            w[0] = v.x; w[1] = v.y;
        }
#pragma unroll
        for (int i = 0; i < EPT / 2; ++i) {
            x[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xFFFFu));
            x[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
        }
    } else {
        const f32x4* p = (const f32x4*)((const float*)base + row * D + EPT * u);
#pragma unroll
        for (int i = 0; i < EPT / 4; ++i) {
            const f32x4 v = p[i];
            x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
        }
    }
}

// Bulk append: workgroup (chunk c, kv head h) takes the new tokens
// 16c .. 16c + 15 (flat order) of head h.  When they are exactly one page of
// one sequence (same sequence, first position a multiple of 16: a prompt
// appended from a page boundary), the four wavefronts quantize the page-head
// block together -- thread t holds token t / 16, dimensions EPT (t mod 16) ..
// -- and write it whole: key rows as contiguous 4- or 8-byte stores, the
// value nibble pairs (slots 2j, 2j+1 of one dimension) transposed through
// LDS into the dimension-major rows and written as one contiguous block.  The
// scales, codes (and affine zero points) are those of the per-token path
// (same reductions, same device functions).  Any other chunk runs the
// per-token path, one wavefront per token.
template <int D, bool BF16, bool AFF>
__global__ __launch_bounds__(256) void append_pages_kernel(Q8K4V_APPEND_PARAMS) {
    constexpr int EPT = D / 16;      // elements per thread (16 threads per token)
    constexpr int NG = D / 32;
    constexpr int TPG = 32 / EPT;    // threads per value group
    __shared__ int s_page;
    __shared__ __attribute__((aligned(16))) uint8_t s_v[D * 8];
    const int h = (int)(blockIdx.x % H);
    const long tok0 = (long)(blockIdx.x / H) * 16;
    if (threadIdx.x == 0) {
        int page = -1;
        if (tok0 + 16 <= total_new) {
            int lo = 0, hi = n_seqs - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (cu_new[mid] <= tok0) lo = mid; else hi = mid - 1;
            }
            const long pos0 = start_pos[lo] + (tok0 - cu_new[lo]);
            if (tok0 + 16 <= cu_new[lo + 1] && (pos0 & 15) == 0)
                page = page_table[(size_t)lo * max_pages + (pos0 >> 4)];
        }
        s_page = page;
    }
    __syncthreads();
    const int page = s_page;
    if (page < 0) {
        const int wave = threadIdx.x >> 6;
#pragma unroll 1
        for (int k = 0; k < 4; ++k) {
            const long tok = tok0 + 4 * wave + k;
            if (tok < total_new) append_token<D, BF16, AFF>(Q8K4V_APPEND_ARGS, tok * H + h, threadIdx.x & 63);
        }
        return;
    }
    const int t = threadIdx.x, slot = t >> 4, u = t & 15;
    const size_t blk = (size_t)page * H + h;
    const size_t row = (size_t)(tok0 + slot) * H + h;
    // keys: absmax (affine: min and max) over the token's 16 threads
    float kx[EPT];
    load_seg<D, EPT, BF16>(k_new, row, u, kx);
    int kc[EPT];
    _Float16 ks16;
    int kz = 0;
    if (AFF) {
        float mn = kx[0], mx = kx[0];
#pragma unroll
        for (int e = 1; e < EPT; ++e) { mn = fminf(mn, kx[e]); mx = fmaxf(mx, kx[e]); }
        const Affine a = affine_of(wave_min(mn, 16), wave_max(mx, 16), 255.0f);
#pragma unroll
        for (int e = 0; e < EPT; ++e) kc[e] = affine_code(kx[e], a, 255.0f) ^ 0x80;
        ks16 = a.s16;
        kz = (int)a.z ^ 0x80;
    } else {
        float ka = 0.0f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) ka = fmaxf(ka, fabsf(kx[e]));
        ka = wave_max(ka, 16);
        ks16 = scale_of(ka, 127.0f);
        const float ks = (float)ks16;
#pragma unroll
        for (int e = 0; e < EPT; ++e) kc[e] = code_of(kx[e], ks, 127.0f);
    }
    uint32_t kw[EPT / 4];
#pragma unroll
    for (int i = 0; i < EPT / 4; ++i) {
        kw[i] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) kw[i] |= ((uint32_t)kc[4 * i + e] & 0xFFu) << (8 * e);
    }
    int8_t* krow = k_codes + (blk * 16 + slot) * D + EPT * u;
    if constexpr (EPT == 8) *(u32x2*)krow = u32x2{kw[0], kw[1]};
    else *(uint32_t*)krow = kw[0];
    if (u == 0) {
        k_scales[blk * 16 + slot] = __builtin_bit_cast(uint16_t, ks16);
        if (AFF) k_zeros[blk * 16 + slot] = (int8_t)kz;
    }
    // values: groups of 32 dimensions over TPG threads
    float vx[EPT];
    load_seg<D, EPT, BF16>(v_new, row, u, vx);
    int c[EPT];
    _Float16 vs16;
    int z;
    value_codes<EPT, TPG, AFF>(vx, c, &vs16, &z);
    if (u % TPG == 0) {
        v_scales[(blk * 16 + slot) * NG + u / TPG] = __builtin_bit_cast(uint16_t, vs16);
        if (AFF) v_zeros[(blk * 16 + slot) * NG + u / TPG] = (uint8_t)z;
    }
    uint32_t nib = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) nib |= ((uint32_t)c[e] & 0xFu) << (4 * e);
    const uint32_t odd = __shfl_xor(nib, 16);   // slot ^ 1 sits 16 lanes away
    if ((slot & 1) == 0) {
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            s_v[(EPT * u + e) * 8 + (slot >> 1)] =
                (uint8_t)(((nib >> (4 * e)) & 0xFu) | (((odd >> (4 * e)) & 0xFu) << 4));
    }
    __syncthreads();
    if (t < D / 2) ((u32x4*)(v_codes + blk * D * 8))[t] = ((const u32x4*)s_v)[t];
}
}  // namespace

int32_t launch_append(const AppendArgs& a, hipStream_t stream) {
    const q8k4v_cache& c = *a.cache;
    if (a.total_new == 0) return Q8K4V_OK;
    // bulk calls (prompts, chunks: 256 new tokens or more) take a workgroup
    // per (16 new tokens, head), whole pages at once -- its vector loads and
    // stores want 16-byte aligned inputs and pools; small calls (decode steps,
    // drafts) a wavefront per (token, head), the most parallel mapping
    const uintptr_t al = (uintptr_t)a.k_new | (uintptr_t)a.v_new | (uintptr_t)c.k_codes | (uintptr_t)c.v_codes;
    const bool pages = a.last_of == nullptr && (al & 15) == 0 && a.total_new >= 256;
    const long items = (long)a.total_new * c.num_kv_heads;
    const long blocks = pages ? (long)((a.total_new + 15) / 16) * c.num_kv_heads : (items + 3) / 4;
    if (blocks > 0x7FFFFFFFL) return fail(Q8K4V_EINVAL, "kv_quant_append: too many tokens in one call");
    dim3 grid((unsigned)blocks), block(256);
#define Q8K4V_APPEND(DD, BB, AA)                                                                          \
    do {                                                                                                  \
        if (pages)                                                                                        \
            hipLaunchKernelGGL((append_pages_kernel<DD, BB, AA>), grid, block, 0, stream, c.k_codes,      \
                               c.k_scales, c.v_codes, c.v_scales, c.k_zeros, c.v_zeros, c.num_kv_heads,   \
                               a.k_new, a.v_new, a.cu_new, a.start_pos, a.page_table, a.max_pages,        \
                               a.n_seqs, a.total_new, a.last_of);                                         \
        else                                                                                              \
            hipLaunchKernelGGL((append_kernel<DD, BB, AA>), grid, block, 0, stream, c.k_codes, c.k_scales, \
                               c.v_codes, c.v_scales, c.k_zeros, c.v_zeros, c.num_kv_heads, a.k_new,      \
                               a.v_new, a.cu_new, a.start_pos, a.page_table, a.max_pages, a.n_seqs,       \
                               a.total_new, a.last_of);                                                   \
    } while (0)
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
