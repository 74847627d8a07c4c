// Split-K attention over the paged k8v4 cache for 1 to 16 query rows per kv
// head (a GQA group, or drafts x group), on gfx950's 16x16 MFMAs with the
// query rows replicated across the MFMA columns.
//
// What it computes: exact softmax attention over the dequantized cache (the
// decode unit of blog.123qwe.co.kr/?p=3927, section 5); row r = (draft j,
// group member g) of sequence b sees positions 0 .. L_b - W + j.
//
// Layout of the work.  A workgroup owns a range of pages of one (sequence,
// kv head); its waves take 2-page tiles round robin.  Each wave keeps a ring
// of STAGES tile buffers in LDS filled by global_load_lds_dwordx4, so
// STAGES - 1 tiles are in flight while one is computed; completion is tracked
// with partial vmcnt waits.  The wave's page ids sit one per lane in a VGPR
// (read with v_readlane when a tile is issued), so no table lookup is on the
// critical path.
//
// Per tile (pages P0, P1; lane l = (n = l & 15, q = l >> 4)):
//  * S^T = K Q^T on v_mfma_i32_16x16x64_i8, one instruction chain per page:
//    the page's 16 tokens are the MFMA rows, the stored int8 key codes the A
//    operand.  The B operand holds query row (n mod R) in column n, as a
//    15-bit fixed-point number split into int8 halves (two chains, exact
//    int32 sums).  Lane (n, q) receives the scores of row n mod R for tokens
//    4q .. 4q+3 of the page;
//  * online softmax per row in the log2 domain, reductions across the four
//    lane groups with v_permlane16_swap / v_permlane32_swap (no LDS);
//  * O = P' V on v_mfma_f32_16x16x32_f16: A row m is (query row m mod R, value
//    group (m / R) mod NG) -- the lane already holds that row's
//    probabilities, multiplies them by the token's value-group scale and
//    rounds once to fp16; k = the 32 tokens of the tile (for lane group q:
//    tokens 4q .. 4q+3 of P0 and of P1); B = the value codes as exact fp16
//    (one 32-bit word per lane and output tile: 4 nibbles of P0, 4 of P1).
//    Output tile dt (dims 16dt .. 16dt+15, value group dt/2) keeps the rows
//    of its group.
//
// The same file holds the row-block variant for other row counts (verify,
// chunked prefill, the cascade's prefix pass), the decode body that appends
// the step's new token itself, the fused launch of the cascade's prefix and
// suffix passes, and the affine-codec paths of both bodies.
#include "attn_common.h"
#include "codec_device.h"
#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int N>
Q8K4V_DEV void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

Q8K4V_DEV uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
Q8K4V_DEV float bitsf(uint32_t x) { return __builtin_bit_cast(float, x); }

// max / sum with the lanes 16 and 32 apart (the four lane groups)
Q8K4V_DEV float xgroups_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
    x = fmaxf(bitsf(a[0]), bitsf(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
    return fmaxf(bitsf(b[0]), bitsf(b[1]));
}
Q8K4V_DEV float xgroups_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
    x = bitsf(a[0]) + bitsf(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
    return bitsf(b[0]) + bitsf(b[1]);
}

// 32-bit word of value codes -> four exact fp16 pairs: nibble j (bits
// 4j..4j+3) and nibble j+4 (bits 16+4j..) become pair j.  One v_bitop3 per
// pair copies the nibble's low three bits, inverts its top bit (two's
// complement code -> code + 8) and sets the fp16 exponent of 1024: the pair
// reads 1032 + code (nibble at bit 0 of a half) or 1152 + 16 code (nibble at
// bit 4), and one packed add / fma returns the code exactly.
// bitop3 truth table (sources x, A, B): x where A & ~B, ~x where ~A & B, 1
// where A & B, 0 elsewhere -> 0xCA.
Q8K4V_DEV uint32_t nib_to_f16(uint32_t x, uint32_t a, uint32_t b) { return __builtin_amdgcn_bitop3_b32(x, a, b, 0xCA); }

Q8K4V_DEV void v_word_to_f16(uint32_t x, uint32_t out[4]) {
    const uint32_t y = x >> 8;
    const f16x2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const f16x2 inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const f16x2 off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    out[0] = as_u32(as_h2(nib_to_f16(x, 0x64076407u, 0x64086408u)) + off);
    out[1] = as_u32(__builtin_elementwise_fma(as_h2(nib_to_f16(x, 0x64706470u, 0x64806480u)), inv16, off16));
    out[2] = as_u32(as_h2(nib_to_f16(y, 0x64076407u, 0x64086408u)) + off);
    out[3] = as_u32(__builtin_elementwise_fma(as_h2(nib_to_f16(y, 0x64706470u, 0x64806480u)), inv16, off16));
}

// Bytes of one 2-page tile in LDS: key codes, value codes, key scales,
// value scales of both pages (6464 B at D = 128), then with the affine codec
// the key and value zero points (16 + 16 D/32 B per page; 6624 B at D = 128).
template <int D, bool AFF = false>
constexpr int ring_stage_bytes() { return 2 * (16 * D + 8 * D + 32 + 32 * (D / 32) + (AFF ? 16 + 16 * (D / 32) : 0)); }

// sum over the four lane groups (lanes 16 and 32 apart), integers
Q8K4V_DEV int xgroups_isum(int x) {
    auto a = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    x = (int)a[0] + (int)a[1];
    auto b = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return (int)b[0] + (int)b[1];
}

// Affine value codes: the word's unsigned nibbles become fp16 (code - z).
// A nibble at bit 0 of a half is set into the fp16 1024 + code and the pair
// zl = fp16 (-1024 - z_page0, -1024 - z_page1) is added; a nibble at bit 4
// gives 1024 + 16 code, scaled by 1/16 and zh = fp16 (-64 - z) added.  Every
// value is a small integer, so each step is exact.
Q8K4V_DEV void v_word_to_f16_affine(uint32_t x, const uint32_t (&zl)[2], const uint32_t (&zh)[2], uint32_t out[4]) {
    const uint32_t y = x >> 8;
    const f16x2 inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    out[0] = as_u32(as_h2((x & 0x000F000Fu) | 0x64006400u) + as_h2(zl[0]));
    out[1] = as_u32(__builtin_elementwise_fma(as_h2((x & 0x00F000F0u) | 0x64006400u), inv16, as_h2(zh[0])));
    out[2] = as_u32(as_h2((y & 0x000F000Fu) | 0x64006400u) + as_h2(zl[1]));
    out[3] = as_u32(__builtin_elementwise_fma(as_h2((y & 0x00F000F0u) | 0x64006400u), inv16, as_h2(zh[1])));
}

// Zero-point operands of value group g for the pairs of token 4q4 + j
// (j = 0..3) of pages 0 and 1: vz0 / vz1 hold the lane's 4 NG zero-point
// bytes of each page (token-major, byte j NG + g).  zl for j = 0, 2 (low
// nibbles), zh for j = 1, 3 (high nibbles).
template <int NG>
Q8K4V_DEV void value_zero_pairs(const uint32_t* vz0, const uint32_t* vz1, int g, uint32_t (&zl)[2], uint32_t (&zh)[2]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int bi = j * NG + g, wi = bi >> 2, bb = bi & 3;
        // byte bb of page 0 into bits 0..7, of page 1 into bits 16..23
        const uint32_t zp = __builtin_amdgcn_perm(vz1[wi], vz0[wi], (uint32_t)bb | 0x0C00u | (uint32_t)(4 + bb) << 16 | 0x0C000000u);
        if (j % 2 == 0) zl[j / 2] = zp | 0xE400E400u;            // -(1024 + z)
        else zh[j / 2] = (zp << 4) | 0xD400D400u;                // -(64 + z)
    }
}

// The query row as the int8 B operands of q.K.  Each value x becomes a 23-bit
// fixed-point number Q = rne(x * 2^(22 - e)) with 2^(e-1) <= max|row| < 2^e,
// so |Q| <= 2^22 and the rounding error of an element is at most 2^(e-23) <=
// max|row| * 2^-22 (a bf16 element within 2^15 of the row's largest
// magnitude is exact).  Q is written in base-256 signed digits
// Q = 65536 h + 256 m + l (l, m in -128..127, h in -64..64): three int8
// operands whose int32 MFMA sums are exact.  One fma against 1.5 * 2^23
// rounds x * 2^(22-e) to an integer, ties to even, inside the fp32 mantissa
// (bits = 0x4B400000 + Q); W = Q + 128 * (65536 + 256 + 1) lies in 0 .. 2^24
// and byte k of W is digit k + 128, so digit k as int8 is byte k XOR 0x80.
// Byte t of word c holds element 4c + t (the MFMA B layout of one lane).
struct QDigits { u32x4 h, m, l; };

template <bool SUM>
Q8K4V_DEV QDigits query_digits(const float (&x)[16], float sc, int& qsum) {
    uint32_t hw[4], mw[4], lw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        uint32_t W[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            W[t] = fbits(__builtin_fmaf(x[4 * c + t], sc, 12582912.0f)) - 1254064000u;
            if (SUM) qsum += (int)W[t] - 8421504;            // Q
        }
        const uint32_t a01 = __builtin_amdgcn_perm(W[1], W[0], 0x05040100u);   // bytes 0, 1 of W0, W1
        const uint32_t a23 = __builtin_amdgcn_perm(W[3], W[2], 0x05040100u);
        const uint32_t b01 = __builtin_amdgcn_perm(W[1], W[0], 0x07060302u);   // bytes 2, 3 of W0, W1
        const uint32_t b23 = __builtin_amdgcn_perm(W[3], W[2], 0x07060302u);
        lw[c] = __builtin_amdgcn_perm(a23, a01, 0x06040200u) ^ 0x80808080u;
        mw[c] = __builtin_amdgcn_perm(a23, a01, 0x07050301u) ^ 0x80808080u;
        hw[c] = __builtin_amdgcn_perm(b23, b01, 0x06040200u) ^ 0x80808080u;
    }
    return QDigits{u32x4{hw[0], hw[1], hw[2], hw[3]}, u32x4{mw[0], mw[1], mw[2], mw[3]},
                   u32x4{lw[0], lw[1], lw[2], lw[3]}};
}

// Exponent e of a row maximum (2^(e-1) <= mx < 2^e), clamped so that
// 2^(22-e) and 2^(e-22) stay normal fp32 numbers; rows with max|q| >= 2^100
// are outside the supported range.
Q8K4V_DEV int row_exponent(float mx) {
    int e = 0;
    if (mx > 0.0f) (void)frexpf(mx, &e);
    return min(max(e, -100), 100);
}

// Score of one token from the three digit sums: Q.c = 65536 H + 256 M + L,
// formed as fp32 (65536 H + 256 M is exact in int32; the fp32 result carries
// a relative rounding error of at most 2^-23).  Affine keys subtract the
// key zero point times the row's sum of Q.
template <bool AFF>
Q8K4V_DEV float digit_dot(int H, int M, int L, int zp, float qsumf) {
    float f = __builtin_fmaf((float)(H * 256 + M), 256.0f, (float)L);
    if (AFF) f = __builtin_fmaf(-(float)zp, qsumf, f);
    return f;
}

// The kernel bodies take their tile ring (WAVES x STAGES stages, in LDS) and
// their block index as arguments so that one launch can run two of them
// (the shared-prefix cascade's fused pass).
template <int D, int R, int WAVES, int STAGES, bool QBF16, bool AFF, bool APP = false, bool SQ = false>
Q8K4V_DEV void dec2_body(const AttnParams& p, uint8_t* smem, int bid) {
    constexpr int TP = 2;                      // pages per tile
    constexpr int KB = 16 * D, VB = 8 * D;     // key / value code bytes per page
    constexpr int NG = D / 32;                 // value groups
    constexpr int KSB = 32, VSB = 32 * NG;     // scale bytes per page
    constexpr int OFF_V = TP * KB, OFF_KS = OFF_V + TP * VB, OFF_VS = OFF_KS + TP * KSB;
    constexpr int KZB = 16, VZB = 16 * NG;     // affine zero-point bytes per page
    constexpr int OFF_KZ = OFF_VS + TP * VSB, OFF_VZ = OFF_KZ + TP * KZB;
    constexpr int STAGE = AFF ? OFF_VZ + TP * VZB : OFF_KZ;   // 6464 B at D = 128 (6624 affine)
    constexpr int CPR = D / 16;                // 16-byte chunks per key row
    constexpr int KS = D / 64;                 // 64-dimension k-steps of q.K
    constexpr int NDT = D / 16;                // 16-dimension output tiles
    constexpr int NA = (R * NG + 15) / 16;     // A tiles of (row, group) pairs
    constexpr int KI = KB / 1024;              // 1 KiB key copies per page
    constexpr int IPT = TP * (KI + 3 + (AFF ? 2 : 0));   // copy instructions per tile
    static_assert(16 % R == 0, "R must divide 16");
    static_assert(STAGES >= 2 && STAGES <= 3, "2 or 3 stages");
    static_assert(R * D * 4 <= STAGES * STAGE, "the merge buffer reuses the tile ring");
    static_assert(STAGE == ring_stage_bytes<D, AFF>(), "tile layout");

    __shared__ float s_ml[WAVES][R][2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WorkItem w;
    if (!work_item(p, w, bid)) return;
    if (w.pbeg >= w.pend) {
        if (w.split == 0 && !p.cascade) write_zero_rows<D>(p, w, 0, R);
        return;
    }
    const int n16 = lane & 15;
    const int q4 = lane >> 4;
    const int row = n16 % R;                   // query row of this lane's scores
    const int kh = w.kh, pend = w.pend;
    const int ntile_all = (pend - w.pbeg + TP - 1) / TP;
    const int nt = ntile_all > wave ? (ntile_all - wave + WAVES - 1) / WAVES : 0;   // <= 32 (planner)

    // APP: the step's new token sits at position L - 1, logical page pn; the
    // wave whose tile holds pn quantizes it (the append kernel's rule, same
    // device functions), patches its slot in that tile's LDS copy before the
    // tile is read and writes it to the cache for later calls -- this launch
    // never reads the token from memory
    constexpr int EPL = D / 64;
    bool app_owner = false;
    int app_t = -1, app_u = 0, app_slot = 0;
    if (APP) {
        const int pn = (w.L - 1) >> 4;
        if (w.L > 0 && pn >= w.pbeg && pn < pend && ((pn - w.pbeg) / TP) % WAVES == wave) {
            app_owner = true;
            app_t = ((pn - w.pbeg) / TP) / WAVES;
            app_u = (pn - w.pbeg) % TP;
            app_slot = (w.L - 1) & 15;
        }
    }
    float app_kx[EPL], app_vx[EPL];
    if (APP && app_owner) {   // loads go out before the query's, so one wait covers both
        const size_t row = (size_t)w.b * p.H + kh;
        if (p.new_bf16) {
            load_row<D, true>(p.k_new, row, lane, app_kx);
            load_row<D, true>(p.v_new, row, lane, app_vx);
        } else {
            load_row<D, false>(p.k_new, row, lane, app_kx);
            load_row<D, false>(p.v_new, row, lane, app_vx);
        }
    }

    // page ids of this wave's tiles, one per lane: page u of wave tile t is
    // lane 2t + u (pages past the split end repeat its last page; masked)
    int my_id = 0;
    {
        const int pg = w.pbeg + TP * (wave + WAVES * (lane >> 1)) + (lane & 1);
        if (lane < TP * nt) my_id = p.page_table[(size_t)w.b * p.max_pages + min(pg, pend - 1)];
    }

    uint8_t* const stage0 = smem + wave * STAGES * STAGE;
    const uint32_t lds0 = lds_addr(stage0);
    uint32_t kdma_off[KI];                     // key rows swizzled: chunk c of row t at t*CPR + (c ^ t%CPR)
#pragma unroll
    for (int c = 0; c < KI; ++c) {
        const int s = 64 * c + lane;
        const int t = s / CPR, cc = (s % CPR) ^ (t % CPR);
        kdma_off[c] = (uint32_t)(t * D + 16 * cc);
    }
    auto issue = [&](int t, int slot) {
        const uint32_t base = lds0 + slot * STAGE;
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const int id = __builtin_amdgcn_readlane(my_id, TP * t + u);
            const size_t blk = (size_t)id * p.H + kh;
#pragma unroll
            for (int c = 0; c < KI; ++c) lds_dma16(p.k_codes + blk * KB, kdma_off[c], base + u * KB + c * 1024);
            if (VB >= 1024) {
                lds_dma16(p.v_codes + blk * VB, lane * 16, base + OFF_V + u * VB);
            } else if (lane < VB / 16) {
                lds_dma16(p.v_codes + blk * VB, lane * 16, base + OFF_V + u * VB);
            }
            if (lane < 2) lds_dma16(p.k_scales + blk * 16, lane * 16, base + OFF_KS + u * KSB);
            if (lane < 2 * NG) lds_dma16(p.v_scales + blk * 16 * NG, lane * 16, base + OFF_VS + u * VSB);
            if (AFF) {
                if (lane < 1) lds_dma16(p.k_zeros + blk * 16, lane * 16, base + OFF_KZ + u * KZB);
                if (lane < NG) lds_dma16(p.v_zeros + blk * 16 * NG, lane * 16, base + OFF_VZ + u * VZB);
            }
        }
    };
    // ---- query row (n mod R) as the B operands (query_digits); lane (n, q)
    // holds dims 64 ks + 16 q .. +15 of every k-step ks
    // (the query loads go out with the page-id load, before the first
    // copies: the compiler's wait for them then covers no copy)
    // (SQ: wave 0 converts and hands the operands to the other waves through
    // LDS; those start their first copies at once)
    QDigits qd[KS];
    float coef;
    float qsumf = 0.0f;                        // sum of the row's fixed-point Q (affine keys)
    const int lim = w.L - p.W + 1 + row / p.G;
    __shared__ u32x4 s_q[SQ ? KS * 3 * 64 : 1];
    __shared__ float s_coef[SQ ? 64 : 1];
    __shared__ float s_qsum[SQ ? 64 : 1];
    if (SQ && wave != 0) {
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nt) issue(s, s);
    } else {
        const size_t qoff = out_index(p, w.b, kh, row, D);
        float x[KS][16];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 64 * ks + 16 * q4;
            if (QBF16) {
                const u32x4* src = (const u32x4*)((const uint16_t*)p.q + qoff + d0);
                const u32x4 a = src[0], b = src[1];
                const uint32_t wd[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[ks][2 * i] = bitsf(wd[i] << 16);
                    x[ks][2 * i + 1] = bitsf(wd[i] & 0xFFFF0000u);
                }
            } else {
                const f32x4* src = (const f32x4*)((const float*)p.q + qoff + d0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 v = src[i];
                    x[ks][4 * i] = v.x; x[ks][4 * i + 1] = v.y; x[ks][4 * i + 2] = v.z; x[ks][4 * i + 3] = v.w;
                }
            }
        }
        float mx = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(x[ks][i]));
        mx = xgroups_max(mx);
        // the first tiles' copies go out now; the conversion below overlaps them
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nt) issue(s, s);
        const int e = row_exponent(mx);
        const float sc = ldexpf(1.0f, 22 - e);
        int qsum = 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qd[ks] = query_digits<AFF>(x[ks], sc, qsum);
        coef = p.scale_log2 * ldexpf(1.0f, e - 22);
        if (AFF) qsumf = (float)xgroups_isum(qsum);
        if (SQ) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s_q[(3 * ks) * 64 + lane] = qd[ks].h;
                s_q[(3 * ks + 1) * 64 + lane] = qd[ks].m;
                s_q[(3 * ks + 2) * 64 + lane] = qd[ks].l;
            }
            s_coef[lane] = coef;
            s_qsum[lane] = qsumf;
        }
    }
    if (SQ) {
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qd[ks].h = s_q[(3 * ks) * 64 + lane];
            qd[ks].m = s_q[(3 * ks + 1) * 64 + lane];
            qd[ks].l = s_q[(3 * ks + 2) * 64 + lane];
        }
        coef = s_coef[lane];
        qsumf = s_qsum[lane];
    }
    // APP: codes and scales (affine: and zero points) of the new token, by
    // the append kernel's rule; affine key codes and zero point are stored
    // XOR 0x80 as there
    int app_kc[EPL] = {}, app_vc[EPL] = {};
    _Float16 app_ks16 = 0, app_vs16 = 0;
    int app_kz = 0, app_vz = 0;
    if (APP && app_owner) {
        if (AFF) {
            float mn = app_kx[0], mx = app_kx[0];
#pragma unroll
            for (int e = 1; e < EPL; ++e) { mn = fminf(mn, app_kx[e]); mx = fmaxf(mx, app_kx[e]); }
            const Affine a = affine_of(wave_min(mn, 64), wave_max(mx, 64), 255.0f);
#pragma unroll
            for (int e = 0; e < EPL; ++e) app_kc[e] = affine_code(app_kx[e], a, 255.0f) ^ 0x80;
            app_ks16 = a.s16;
            app_kz = (int)a.z ^ 0x80;
        } else {
            float ka = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) ka = fmaxf(ka, fabsf(app_kx[e]));
            app_ks16 = scale_of(wave_max(ka, 64), 127.0f);
#pragma unroll
            for (int e = 0; e < EPL; ++e) app_kc[e] = code_of(app_kx[e], (float)app_ks16, 127.0f);
        }
        value_codes<EPL, 32 / EPL, AFF>(app_vx, app_vc, &app_vs16, &app_vz);
    }
    const int lim_min = w.L - p.W + 1;         // every row sees the positions below this

    float m_run = kNegInf, l_run = 0.0f;       // row `row`; l_run over this lane's tokens
    f32x4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // value group of A row m = n16 in A tile a
    int grp[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) grp[a] = ((16 * a + n16) / R) % NG;

    // Every path has consumed the page-id load by now; an explicit use says so.
    // Otherwise the compiler's own wait for that load (on the paths that
    // issued no first copy) lands at the top of each iteration, where its
    // vmcnt(0) also drains the copies in flight and breaks the prefetch.
    asm volatile("" ::"v"(my_id));
    for (int t = 0; t < nt; ++t) {
        const int slot = t % STAGES;
        if (t + STAGES - 1 < nt) issue(t + STAGES - 1, (t + STAGES - 1) % STAGES);
        const int after = min(STAGES - 1, nt - 1 - t);   // tiles issued after this one
        if (STAGES == 3 && after >= 2) wait_vmem<2 * IPT>();
        else if (after >= 1) wait_vmem<IPT>();
        else wait_vmem<0>();

        if (APP && app_owner && t == app_t) {
            // the new token's slot in this tile's LDS copy, then the cache
            uint8_t* sw = stage0 + slot * STAGE;
            const int id = __builtin_amdgcn_readlane(my_id, TP * app_t + app_u);
            const size_t blk = (size_t)id * p.H + kh;
            int8_t* kdst = const_cast<int8_t*>(p.k_codes) + (blk * 16 + app_slot) * D;
            uint8_t* vdst = const_cast<uint8_t*>(p.v_codes) + blk * 8 * D;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int d = EPL * lane + e, c = d / 16;
                sw[app_u * KB + (app_slot * CPR + (c ^ (app_slot % CPR))) * 16 + d % 16] = (uint8_t)app_kc[e];
                kdst[d] = (int8_t)app_kc[e];
                uint8_t* vb = sw + OFF_V + app_u * VB + d * 8 + (app_slot >> 1);
                const uint32_t nib = (uint32_t)app_vc[e] & 0xFu;
                const uint8_t byte = (uint8_t)((app_slot & 1) ? ((*vb & 0x0Fu) | (nib << 4)) : ((*vb & 0xF0u) | nib));
                *vb = byte;
                vdst[d * 8 + (app_slot >> 1)] = byte;
            }
            const uint16_t ksb = __builtin_bit_cast(uint16_t, app_ks16), vsb = __builtin_bit_cast(uint16_t, app_vs16);
            if (lane == 0) {
                *(uint16_t*)(sw + OFF_KS + app_u * KSB + app_slot * 2) = ksb;
                const_cast<uint16_t*>(p.k_scales)[blk * 16 + app_slot] = ksb;
                if (AFF) {
                    sw[OFF_KZ + app_u * KZB + app_slot] = (uint8_t)app_kz;
                    const_cast<int8_t*>(p.k_zeros)[blk * 16 + app_slot] = (int8_t)app_kz;
                }
            }
            if (lane % (32 / EPL) == 0) {
                const int g = lane / (32 / EPL);
                *(uint16_t*)(sw + OFF_VS + app_u * VSB + (app_slot * NG + g) * 2) = vsb;
                const_cast<uint16_t*>(p.v_scales)[(blk * 16 + app_slot) * NG + g] = vsb;
                if (AFF) {
                    sw[OFF_VZ + app_u * VZB + app_slot * NG + g] = (uint8_t)app_vz;
                    const_cast<uint8_t*>(p.v_zeros)[(blk * 16 + app_slot) * NG + g] = (uint8_t)app_vz;
                }
            }
        }
        // ---- tile to registers
        const uint8_t* st = stage0 + slot * STAGE;
        u32x4 ka[TP][KS];
#pragma unroll
        for (int u = 0; u < TP; ++u)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = 4 * ks + q4;
                ka[u][ks] = *(const u32x4*)(st + u * KB + (n16 * CPR + (c ^ (n16 % CPR))) * 16);
            }
        uint32_t vx[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int off = OFF_V + (16 * dt + n16) * 8 + 2 * q4;
            vx[dt] = (uint32_t)*(const uint16_t*)(st + off) | ((uint32_t)*(const uint16_t*)(st + off + VB) << 16);
        }
        u32x2 ksw[TP];
#pragma unroll
        for (int u = 0; u < TP; ++u) ksw[u] = *(const u32x2*)(st + OFF_KS + u * KSB + 8 * q4);
        float vsf[NA][TP][4];                  // value scale of (group grp[a], page u, token 4q4 + j)
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int u = 0; u < TP; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    vsf[a][u][j] = h2f(*(const uint16_t*)(st + OFF_VS + u * VSB + ((4 * q4 + j) * NG + grp[a]) * 2));
        // affine: key zero points of tokens 4q4 .. 4q4+3, value zero points
        // of those tokens for every group (token-major bytes)
        uint32_t kzw[TP] = {}, vz[TP][NG] = {};
        if (AFF) {
#pragma unroll
            for (int u = 0; u < TP; ++u) {
                kzw[u] = *(const uint32_t*)(st + OFF_KZ + u * KZB + 4 * q4);
#pragma unroll
                for (int wd = 0; wd < NG; ++wd) vz[u][wd] = *(const uint32_t*)(st + OFF_VZ + u * VZB + 4 * NG * q4 + 4 * wd);
            }
        }
        wait_lds_all();

        // ---- scores: three digit chains per page
        i32x4_t ch[TP], cm[TP], cl[TP];
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            ch[u] = cm[u] = cl[u] = i32x4_t{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const i32x4_t a = __builtin_bit_cast(i32x4_t, ka[u][ks]);
                ch[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, __builtin_bit_cast(i32x4_t, qd[ks].h), ch[u], 0, 0, 0);
                cm[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, __builtin_bit_cast(i32x4_t, qd[ks].m), cm[u], 0, 0, 0);
                cl[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, __builtin_bit_cast(i32x4_t, qd[ks].l), cl[u], 0, 0, 0);
            }
        }
        const int pg0 = w.pbeg + TP * (wave + WAVES * t);
        float s[TP][4];
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const float kf[4] = {h2f((uint16_t)ksw[u].x), h2f((uint16_t)(ksw[u].x >> 16)), h2f((uint16_t)ksw[u].y),
                                 h2f((uint16_t)(ksw[u].y >> 16))};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s[u][i] = digit_dot<AFF>(ch[u][i], cm[u][i], cl[u][i], (int8_t)(kzw[u] >> (8 * i)), qsumf) *
                          (kf[i] * coef);
        }
        if ((pg0 + TP) * 16 > lim_min || pg0 + TP > pend) {      // tile reaches the causal edge / split end
#pragma unroll
            for (int u = 0; u < TP; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = (pg0 + u) * 16 + 4 * q4 + i;
                    if (!(pg0 + u < pend && pos < lim)) s[u][i] = kNegInf;
                }
        }
        // ---- online softmax (row `row`)
        float tmax = kNegInf;
#pragma unroll
        for (int u = 0; u < TP; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[u][i]);
        tmax = xgroups_max(tmax);
        const float r_old = m_run;
        const bool up = tmax > r_old;
        m_run = up ? tmax + kRefHeadroom : r_old;
        const float ref = (m_run == kNegInf) ? 0.0f : m_run;
        float psum = 0.0f;
#pragma unroll
        for (int u = 0; u < TP; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[u][i] = exp2_fast(s[u][i] - ref);
                psum += s[u][i];
            }
        if (__builtin_amdgcn_ballot_w64(up && r_old != kNegInf) != 0) {
            // 0 on rows that had no finite score yet (their sums are 0), 1 on
            // rows whose reference did not move
            const float alpha = exp2_fast(r_old - ref);
            l_run *= alpha;
            // output rows 4q4 + i hold query row (4q4 + i) mod R
            float ai[4];
            if (R <= 4) {
                const int bits = __builtin_bit_cast(int, alpha);
                ai[0] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(bits, 0x00, 0xF, 0xF, false));
                ai[1] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(bits, 0x55, 0xF, 0xF, false));
                ai[2] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(bits, 0xAA, 0xF, 0xF, false));
                ai[3] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(bits, 0xFF, 0xF, 0xF, false));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, (4 * q4 + i) % R);
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                acc[dt][0] *= ai[0]; acc[dt][1] *= ai[1]; acc[dt][2] *= ai[2]; acc[dt][3] *= ai[3];
            }
        }
        l_run += psum;
        // ---- A operands: P' = p * value scale, rounded once to fp16; half
        // 2j + u of the lane = page u, token 4q4 + j
        u32x4 pa[NA];
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            uint32_t wd[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f16x2 h = __builtin_convertvector(
                    (float __attribute__((ext_vector_type(2)))){s[0][j] * vsf[a][0][j], s[1][j] * vsf[a][1][j]}, f16x2);
                wd[j] = as_u32(h);
            }
            pa[a] = u32x4{wd[0], wd[1], wd[2], wd[3]};
        }
        // ---- O += P' V
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int a = ((dt / 2) * R) / 16;
            uint32_t b[4];
            if (AFF) {
                uint32_t zl[2], zh[2];
                value_zero_pairs<NG>(vz[0], vz[1], dt / 2, zl, zh);
                v_word_to_f16_affine(vx[dt], zl, zh, b);
            } else {
                v_word_to_f16(vx[dt], b);
            }
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, pa[a]),
                                                              __builtin_bit_cast(f16x8_t, u32x4{b[0], b[1], b[2], b[3]}),
                                                              acc[dt], 0, 0, 0);
        }
    }

    // ---- per-wave state to LDS, merge the waves, emit
    const float l_tot = xgroups_sum(l_run);
    if (q4 == 0 && n16 < R) {
        s_ml[wave][n16][0] = m_run;
        s_ml[wave][n16][1] = l_tot;
    }
    __syncthreads();           // every wave is done with its ring: reuse it for O
    float* s_o = (float*)smem;   // [WAVES][R][D]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        const int g = dt / 2;
        const int a = (g * R) / 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * q4 + i;                 // C row in A tile a
            const int idx = 16 * a + m;               // (row, group) index
            if (idx >= g * R && idx < g * R + R)
                s_o[(wave * R + idx % R) * D + 16 * dt + n16] = acc[dt][i];
        }
    }
    finish_workgroup<D, R, WAVES>(p, w, 0, s_ml, s_o, smem, WAVES * STAGES * STAGE);
}

template <int D, int R, int WAVES, int STAGES, bool QBF16, bool AFF>
__global__ __launch_bounds__(64 * WAVES) void attn_dec2_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[WAVES * STAGES * ring_stage_bytes<D, AFF>()];
    constexpr bool SQ = WAVES * STAGES * ring_stage_bytes<D, AFF>() + (D / 64) * 3072 + 8192 <= 163840;
    dec2_body<D, R, WAVES, STAGES, QBF16, AFF, false, SQ>(p, s_stage, (int)blockIdx.x);
}

// Decode that appends the step's new token itself (four waves, two stages).
template <int D, int R, bool QBF16, bool AFF>
__global__ __launch_bounds__(256) void attn_dec2_append_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[4 * 2 * ring_stage_bytes<D, AFF>()];
    dec2_body<D, R, 4, 2, QBF16, AFF, true, true>(p, s_stage, (int)blockIdx.x);
}

// ---------------------------------------------------------------------------
// Row-block variant for query blocks of up to 32 rows per workgroup (verify:
// drafts x group), rows padded to RB blocks of 16.  The tile ring, page ids
// and the query's fixed-point form are those of attn_dec2_kernel; here the
// MFMA columns are 16 distinct query rows per block (no replication):
//  * S^T = K Q^T per page and row block on v_mfma_i32_16x16x64_i8: lane
//    (n, q) gets row 16 rb + n's scores of tokens 4q .. 4q+3;
//  * A operand per (row block, value group): the lane's probabilities of
//    its 8 tokens, rounded to fp16, times the tokens' group scales (packed
//    fp16 multiply; products of p <= 1 and an fp16 scale cannot overflow);
//  * O tile dt (value group dt/2) on v_mfma_f32_16x16x32_f16 with the exact
//    fp16 value codes: lane (n, q) holds rows 16 rb + 4q + i, dim 16 dt + n.
// The waves' outputs are merged in a fixed two-round tree through LDS.
// ---------------------------------------------------------------------------
template <int D, int RB, int WAVES, int STAGES, bool QBF16, bool AFF, bool SQ = false>
Q8K4V_DEV void rows_body(const AttnParams& p, uint8_t* smem, int bid) {
    constexpr int TP = 2;
    constexpr int KB = 16 * D, VB = 8 * D;
    constexpr int NG = D / 32;
    constexpr int KSB = 32, VSB = 32 * NG;
    constexpr int OFF_V = TP * KB, OFF_KS = OFF_V + TP * VB, OFF_VS = OFF_KS + TP * KSB;
    constexpr int KZB = 16, VZB = 16 * NG;     // affine zero-point bytes per page
    constexpr int OFF_KZ = OFF_VS + TP * VSB, OFF_VZ = OFF_KZ + TP * KZB;
    constexpr int STAGE = AFF ? OFF_VZ + TP * VZB : OFF_KZ;
    constexpr int CPR = D / 16;
    constexpr int KS = D / 64;
    constexpr int NDT = D / 16;
    constexpr int KI = KB / 1024;
    constexpr int IPT = TP * (KI + 3 + (AFF ? 2 : 0));
    constexpr int RW = 16 * RB;                // rows per workgroup
    constexpr int NVW = NG / 2;                // 32-bit words of one token's value scales
    static_assert(STAGES >= 2 && STAGES <= 3, "2 or 3 stages");
    static_assert(STAGE == ring_stage_bytes<D, AFF>(), "tile layout");

    __shared__ float s_ml[WAVES][RW][2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WorkItem w;
    if (!work_item(p, w, bid)) return;
    const int r0 = w.rchunk * RW;
    if (w.pbeg >= w.pend) {
        if (w.split == 0 && !p.cascade) write_zero_rows<D>(p, w, r0, RW);
        return;
    }
    const int n16 = lane & 15;
    const int q4 = lane >> 4;
    const int kh = w.kh, pend = w.pend;
    const int ntile_all = (pend - w.pbeg + TP - 1) / TP;
    const int nt = ntile_all > wave ? (ntile_all - wave + WAVES - 1) / WAVES : 0;   // <= 32 (planner)

    int my_id = 0;
    {
        const int pg = w.pbeg + TP * (wave + WAVES * (lane >> 1)) + (lane & 1);
        if (lane < TP * nt) my_id = p.page_table[(size_t)w.b * p.max_pages + min(pg, pend - 1)];
    }
    uint8_t* const stage0 = smem + wave * STAGES * STAGE;
    const uint32_t lds0 = lds_addr(stage0);
    uint32_t kdma_off[KI];
#pragma unroll
    for (int c = 0; c < KI; ++c) {
        const int s = 64 * c + lane;
        const int t = s / CPR, cc = (s % CPR) ^ (t % CPR);
        kdma_off[c] = (uint32_t)(t * D + 16 * cc);
    }
    auto issue = [&](int t, int slot) {
        const uint32_t base = lds0 + slot * STAGE;
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const int id = __builtin_amdgcn_readlane(my_id, TP * t + u);
            const size_t blk = (size_t)id * p.H + kh;
#pragma unroll
            for (int c = 0; c < KI; ++c) lds_dma16(p.k_codes + blk * KB, kdma_off[c], base + u * KB + c * 1024);
            if (VB >= 1024) {
                lds_dma16(p.v_codes + blk * VB, lane * 16, base + OFF_V + u * VB);
            } else if (lane < VB / 16) {
                lds_dma16(p.v_codes + blk * VB, lane * 16, base + OFF_V + u * VB);
            }
            if (lane < 2) lds_dma16(p.k_scales + blk * 16, lane * 16, base + OFF_KS + u * KSB);
            if (lane < 2 * NG) lds_dma16(p.v_scales + blk * 16 * NG, lane * 16, base + OFF_VS + u * VSB);
            if (AFF) {
                if (lane < 1) lds_dma16(p.k_zeros + blk * 16, lane * 16, base + OFF_KZ + u * KZB);
                if (lane < NG) lds_dma16(p.v_zeros + blk * 16 * NG, lane * 16, base + OFF_VZ + u * VZB);
            }
        }
    };

    // ---- query rows r0 + 16 rb + n as B operands (query_digits; rows past R
    // are zero).  SQ: wave rb converts row block rb only
    // and hands it to the others through LDS; the other waves start their
    // first copies at once.
    QDigits qd[RB][KS];
    float coef[RB];
    int lim[RB];
    float qsumf[RB];                           // sum of each row's fixed-point Q (affine keys)
    static_assert(!SQ || WAVES >= RB, "one converting wave per row block");
    __shared__ u32x4 s_q[SQ ? RB * KS * 3 * 64 : 1];
    __shared__ float s_coef[SQ ? RB * 16 : 1];
    __shared__ float s_qsum[SQ ? RB * 16 : 1];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = r0 + 16 * rb + n16;
        lim[rb] = r < p.R ? w.L - p.W + 1 + r / p.G : 0;
    }
    if (SQ && wave >= RB) {
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nt) issue(s, s);
    } else {
        float x[RB][KS][16];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (SQ && rb != wave) continue;
            const int r = r0 + 16 * rb + n16;
            const bool ok = r < p.R;
            const size_t qoff = out_index(p, w.b, kh, ok ? r : 0, D);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int d0 = 64 * ks + 16 * q4;
                if (QBF16) {
                    const u32x4* src = (const u32x4*)((const uint16_t*)p.q + qoff + d0);
                    const u32x4 a = src[0], b = src[1];
                    const uint32_t wd[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        x[rb][ks][2 * i] = ok ? bitsf(wd[i] << 16) : 0.0f;
                        x[rb][ks][2 * i + 1] = ok ? bitsf(wd[i] & 0xFFFF0000u) : 0.0f;
                    }
                } else {
                    const f32x4* src = (const f32x4*)((const float*)p.q + qoff + d0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const f32x4 v = src[i];
                        x[rb][ks][4 * i] = ok ? v.x : 0.0f;
                        x[rb][ks][4 * i + 1] = ok ? v.y : 0.0f;
                        x[rb][ks][4 * i + 2] = ok ? v.z : 0.0f;
                        x[rb][ks][4 * i + 3] = ok ? v.w : 0.0f;
                    }
                }
            }
        }
        float mx[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (SQ && rb != wave) continue;
            mx[rb] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx[rb] = fmaxf(mx[rb], fabsf(x[rb][ks][i]));
            mx[rb] = xgroups_max(mx[rb]);
        }
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nt) issue(s, s);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (SQ && rb != wave) continue;
            const int e = row_exponent(mx[rb]);
            const float sc = ldexpf(1.0f, 22 - e);
            int qs = 0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qd[rb][ks] = query_digits<AFF>(x[rb][ks], sc, qs);
            coef[rb] = p.scale_log2 * ldexpf(1.0f, e - 22);
            qsumf[rb] = AFF ? (float)xgroups_isum(qs) : 0.0f;
            if (SQ) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s_q[((rb * KS + ks) * 3) * 64 + lane] = qd[rb][ks].h;
                    s_q[((rb * KS + ks) * 3 + 1) * 64 + lane] = qd[rb][ks].m;
                    s_q[((rb * KS + ks) * 3 + 2) * 64 + lane] = qd[rb][ks].l;
                }
                if (q4 == 0) {
                    s_coef[rb * 16 + n16] = coef[rb];
                    s_qsum[rb * 16 + n16] = qsumf[rb];
                }
            }
        }
    }
    if (SQ) {
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                qd[rb][ks].h = s_q[((rb * KS + ks) * 3) * 64 + lane];
                qd[rb][ks].m = s_q[((rb * KS + ks) * 3 + 1) * 64 + lane];
                qd[rb][ks].l = s_q[((rb * KS + ks) * 3 + 2) * 64 + lane];
            }
            coef[rb] = s_coef[rb * 16 + n16];
            qsumf[rb] = s_qsum[rb * 16 + n16];
        }
    }
    const int lim_min = w.L - p.W + 1;

    float m_run[RB], l_run[RB];
    f32x4 acc[RB][NDT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = kNegInf;
        l_run[rb] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[rb][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // Every path has consumed the page-id load by now; an explicit use says so.
    // Otherwise the compiler's own wait for that load (on the paths that
    // issued no first copy) lands at the top of each iteration, where its
    // vmcnt(0) also drains the copies in flight and breaks the prefetch.
    asm volatile("" ::"v"(my_id));
    for (int t = 0; t < nt; ++t) {
        const int slot = t % STAGES;
        if (t + STAGES - 1 < nt) issue(t + STAGES - 1, (t + STAGES - 1) % STAGES);
        const int after = min(STAGES - 1, nt - 1 - t);
        if (STAGES == 3 && after >= 2) wait_vmem<2 * IPT>();
        else if (after >= 1) wait_vmem<IPT>();
        else wait_vmem<0>();

        const uint8_t* st = stage0 + slot * STAGE;
        u32x4 ka[TP][KS];
#pragma unroll
        for (int u = 0; u < TP; ++u)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = 4 * ks + q4;
                ka[u][ks] = *(const u32x4*)(st + u * KB + (n16 * CPR + (c ^ (n16 % CPR))) * 16);
            }
        uint32_t vx[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int off = OFF_V + (16 * dt + n16) * 8 + 2 * q4;
            vx[dt] = (uint32_t)*(const uint16_t*)(st + off) | ((uint32_t)*(const uint16_t*)(st + off + VB) << 16);
        }
        u32x2 ksw[TP];
#pragma unroll
        for (int u = 0; u < TP; ++u) ksw[u] = *(const u32x2*)(st + OFF_KS + u * KSB + 8 * q4);
        // value scales of tokens 4q4 .. 4q4+3, all groups: NG halves per token
        uint32_t vsr[TP][4 * NVW];
#pragma unroll
        for (int u = 0; u < TP; ++u)
#pragma unroll
            for (int c = 0; c < NVW; ++c) {
                const u32x4 v = *(const u32x4*)(st + OFF_VS + u * VSB + 8 * NG * q4 + 16 * c);
                vsr[u][4 * c] = v.x; vsr[u][4 * c + 1] = v.y; vsr[u][4 * c + 2] = v.z; vsr[u][4 * c + 3] = v.w;
            }
        // affine: key zero points of tokens 4q4 .. 4q4+3, value zero points
        // of those tokens for every group (token-major bytes)
        uint32_t kzw[TP] = {}, vz[TP][NG] = {};
        if (AFF) {
#pragma unroll
            for (int u = 0; u < TP; ++u) {
                kzw[u] = *(const uint32_t*)(st + OFF_KZ + u * KZB + 4 * q4);
#pragma unroll
                for (int wd = 0; wd < NG; ++wd) vz[u][wd] = *(const uint32_t*)(st + OFF_VZ + u * VZB + 4 * NG * q4 + 4 * wd);
            }
        }
        wait_lds_all();

        // ---- scores: three digit chains per page and row block
        i32x4_t ch[RB][TP], cm[RB][TP], cl[RB][TP];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int u = 0; u < TP; ++u) {
                ch[rb][u] = cm[rb][u] = cl[rb][u] = i32x4_t{0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const i32x4_t a = __builtin_bit_cast(i32x4_t, ka[u][ks]);
                    ch[rb][u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, __builtin_bit_cast(i32x4_t, qd[rb][ks].h), ch[rb][u], 0, 0, 0);
                    cm[rb][u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, __builtin_bit_cast(i32x4_t, qd[rb][ks].m), cm[rb][u], 0, 0, 0);
                    cl[rb][u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, __builtin_bit_cast(i32x4_t, qd[rb][ks].l), cl[rb][u], 0, 0, 0);
                }
            }
        const int pg0 = w.pbeg + TP * (wave + WAVES * t);
        float kf[TP][4];
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            kf[u][0] = h2f((uint16_t)ksw[u].x);
            kf[u][1] = h2f((uint16_t)(ksw[u].x >> 16));
            kf[u][2] = h2f((uint16_t)ksw[u].y);
            kf[u][3] = h2f((uint16_t)(ksw[u].y >> 16));
        }
        const bool edge = (pg0 + TP) * 16 > lim_min || pg0 + TP > pend;
        // the fp16 pairs of this tile's value codes, shared by the row blocks
        uint32_t pp[RB][4];                    // probabilities (page 0, page 1) per token 4q4 + j
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float s[TP][4];
#pragma unroll
            for (int u = 0; u < TP; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s[u][i] = digit_dot<AFF>(ch[rb][u][i], cm[rb][u][i], cl[rb][u][i], (int8_t)(kzw[u] >> (8 * i)),
                                             qsumf[rb]) * (kf[u][i] * coef[rb]);
            if (edge) {
#pragma unroll
                for (int u = 0; u < TP; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int pos = (pg0 + u) * 16 + 4 * q4 + i;
                        if (!(pg0 + u < pend && pos < lim[rb])) s[u][i] = kNegInf;
                    }
            }
            float tmax = kNegInf;
#pragma unroll
            for (int u = 0; u < TP; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[u][i]);
            tmax = xgroups_max(tmax);
            const float r_old = m_run[rb];
            const bool up = tmax > r_old;
            m_run[rb] = up ? tmax + kRefHeadroom : r_old;
            const float ref = (m_run[rb] == kNegInf) ? 0.0f : m_run[rb];
            float psum = 0.0f;
#pragma unroll
            for (int u = 0; u < TP; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s[u][i] = exp2_fast(s[u][i] - ref);
                    psum += s[u][i];
                }
            if (__builtin_amdgcn_ballot_w64(up && r_old != kNegInf) != 0) {
                const float alpha = exp2_fast(r_old - ref);
                l_run[rb] *= alpha;
                float ai[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * q4 + i);   // lane 4q4+i holds that row
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    acc[rb][dt][0] *= ai[0]; acc[rb][dt][1] *= ai[1]; acc[rb][dt][2] *= ai[2]; acc[rb][dt][3] *= ai[3];
                }
            }
            l_run[rb] += psum;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pp[rb][j] = as_u32(__builtin_convertvector(
                    (float __attribute__((ext_vector_type(2)))){s[0][j], s[1][j]}, f16x2));
        }
        // ---- O += P' V, group by group
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            // (page 0, page 1) scale pairs of tokens 4q4 + j for group g
            uint32_t sp[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int hidx = j * NG + g;                 // half index in a token-major record
                const int dw = hidx >> 1, h = hidx & 1;
                const uint32_t sel = (uint32_t)(2 * h) | (uint32_t)(2 * h + 1) << 8 | (uint32_t)(4 + 2 * h) << 16 |
                                     (uint32_t)(5 + 2 * h) << 24;
                sp[j] = __builtin_amdgcn_perm(vsr[1][dw], vsr[0][dw], sel);
            }
            u32x4 pa[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                pa[rb] = u32x4{as_u32(as_h2(pp[rb][0]) * as_h2(sp[0])), as_u32(as_h2(pp[rb][1]) * as_h2(sp[1])),
                               as_u32(as_h2(pp[rb][2]) * as_h2(sp[2])), as_u32(as_h2(pp[rb][3]) * as_h2(sp[3]))};
            uint32_t zl[2] = {}, zh[2] = {};
            if (AFF) value_zero_pairs<NG>(vz[0], vz[1], g, zl, zh);
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) {
                const int dt = 2 * g + dd;
                uint32_t b[4];
                if (AFF) v_word_to_f16_affine(vx[dt], zl, zh, b);
                else v_word_to_f16(vx[dt], b);
                const f16x8_t B = __builtin_bit_cast(f16x8_t, u32x4{b[0], b[1], b[2], b[3]});
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, pa[rb]), B, acc[rb][dt], 0, 0, 0);
            }
        }
    }

    // ---- merge the waves: each row's maximum, sum and wave factors, then
    // the outputs through LDS buffers (a fixed two-round tree)
    __shared__ float s_M[RW], s_L[RW];
    __shared__ __attribute__((aligned(16))) float s_f[WAVES][RW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l_tot = xgroups_sum(l_run[rb]);
        if (q4 == 0) {
            s_ml[wave][16 * rb + n16][0] = m_run[rb];
            s_ml[wave][16 * rb + n16][1] = l_tot;
        }
    }
    __syncthreads();           // every wave is done with its ring: reuse it
    for (int rl = threadIdx.x; rl < RW; rl += 64 * WAVES) {
        float M = kNegInf;
#pragma unroll
        for (int u = 0; u < WAVES; ++u) M = fmaxf(M, s_ml[u][rl][0]);
        const float ref = (M == kNegInf) ? 0.0f : M;
        float Ls = 0.0f;
#pragma unroll
        for (int u = 0; u < WAVES; ++u) {
            const float f = exp2_fast(s_ml[u][rl][0] - ref);
            s_f[u][rl] = f;
            Ls += s_ml[u][rl][1] * f;
        }
        s_M[rl] = M;
        s_L[rl] = Ls;
    }
    __syncthreads();
    // two rounds into NB = WAVES/2 buffers (upper half of the waves writes,
    // lower half adds), then one pass sums the buffers and emits: fixed
    // order, two barriers whatever the wave count.  The buffers are
    // transposed, [dimension][row] with rows padded to TS: a lane's four
    // rows 16 rb + 4 q4 .. +3 of dimension 16 dt + n16 are one 16-byte access.
    constexpr int NB = WAVES / 2;
    constexpr int TS = RW + 4;                 // 4 mod 8 words: 16-byte accesses of 8 consecutive
                                               // dimensions hit distinct banks
    constexpr int BUF = D * TS;
    static_assert(NB * BUF * 4 <= WAVES * STAGES * STAGE, "merge buffers reuse the tile ring");
    float* s_o = (float*)smem;
#pragma unroll
    for (int round = 0; round < 2; ++round) {
        const bool mine = round == 0 ? wave >= NB : wave < NB;
        if (mine) {
            float* buf = s_o + (wave % NB) * BUF;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const f32x4 f = *(const f32x4*)&s_f[wave][16 * rb + 4 * q4];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    f32x4* dst = (f32x4*)(buf + (16 * dt + n16) * TS + 16 * rb + 4 * q4);
                    const f32x4 v = acc[rb][dt] * f;
                    *dst = (round == 0) ? v : *dst + v;
                }
            }
        }
        __syncthreads();
    }
    // element e = (row quad r4, dimension d): lanes take consecutive
    // dimensions, so each row's stores are contiguous
    const size_t rs = (size_t)p.R * partial_stride<D>();
    float* split_base = p.partials + ((size_t)w.b * p.H + w.kh) * p.n_splits * rs + w.split * rs;
    for (int e = threadIdx.x; e < D * (RW / 4); e += 64 * WAVES) {
        const int d = e % D, r4 = e / D;
        f32x4 O = *(const f32x4*)(s_o + d * TS + 4 * r4);
#pragma unroll
        for (int bb = 1; bb < NB; ++bb) O += *(const f32x4*)(s_o + bb * BUF + d * TS + 4 * r4);
        const float ov[4] = {O.x, O.y, O.z, O.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int rl = 4 * r4 + k, r = r0 + rl;
            if (r >= p.R) continue;
            const float Ls = s_L[rl];
            if (p.direct) {
                const float inv = (Ls > 0.0f) ? 1.0f / Ls : 0.0f;
                p.out[out_index(p, w.b, w.kh, r, D) + d] = ov[k] * inv;
                continue;
            }
            float* rec = split_base + (size_t)r * partial_stride<D>();
            if (d == 0) *(float2*)rec = float2{s_M[rl], Ls};
            rec[4 + d] = ov[k];
        }
    }
    fused_tail<D, RW>(p, w, r0, smem, WAVES * STAGES * STAGE);
}

template <int D, int RB, int WAVES, int STAGES, bool QBF16, bool AFF>
__global__ __launch_bounds__(64 * WAVES) void attn_rows_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[WAVES * STAGES * ring_stage_bytes<D, AFF>()];
    // the shared query operands (RB x 3 KiB per 64 dimensions) where the LDS
    // budget allows them
    constexpr bool SQ = WAVES * STAGES * ring_stage_bytes<D, AFF>() + RB * (D / 64) * 3072 + 8192 <= 163840;
    rows_body<D, RB, WAVES, STAGES, QBF16, AFF, SQ>(p, s_stage, (int)blockIdx.x);
}

// Fused pass of the shared-prefix cascade: blocks [0, pre_blocks) run the
// prefix pass (row-block body, 32 rows per workgroup, over the shared pages),
// the rest the suffix pass (replicated-row body, one session's G rows), with
// one tile ring per workgroup.  Both are four-wave, two-stage rings, so a
// compute-bound prefix workgroup and memory-bound suffix workgroups share
// each CU.  pre_blocks is a multiple of 8, which keeps every block's XCD.
template <int D, int R, bool QBF16, bool AFF>
__global__ __launch_bounds__(256) void attn_cascade_kernel(const AttnParams pre, const AttnParams suf, int pre_blocks) {
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[4 * 2 * ring_stage_bytes<D, AFF>()];
    if ((int)blockIdx.x < pre_blocks) rows_body<D, 2, 4, 2, QBF16, AFF>(pre, s_stage, (int)blockIdx.x);
    else dec2_body<D, R, 4, 2, QBF16, AFF>(suf, s_stage, (int)blockIdx.x - pre_blocks);
}

template <int D, int RB, int WAVES, int STAGES, bool QBF16, bool AFF>
hipError_t launch_rows_t(const AttnParams& kp, hipStream_t stream) {
    const int blocks = work_blocks(kp);
    hipLaunchKernelGGL((attn_rows_kernel<D, RB, WAVES, STAGES, QBF16, AFF>), dim3(blocks), dim3(64 * WAVES), 0, stream,
                       kp);
    return hipGetLastError();
}

template <int D, int R, int WAVES, int STAGES, bool QBF16, bool AFF>
hipError_t launch_t(const AttnParams& kp, hipStream_t stream) {
    const int blocks = work_blocks(kp);
    hipLaunchKernelGGL((attn_dec2_kernel<D, R, WAVES, STAGES, QBF16, AFF>), dim3(blocks), dim3(64 * WAVES), 0, stream,
                       kp);
    return hipGetLastError();
}

using LaunchFn = hipError_t (*)(const AttnParams&, hipStream_t);

// Symmetric caches: every shape; affine caches: the two-stage 4- and 8-wave
// shapes (the defaults), which bounds the number of kernel instances.
template <int D, int R, bool QBF16, bool AFF>
LaunchFn pick_shape(int waves, int stages) {
    if (AFF) {
        if (waves == 4 && stages == 2) return &launch_t<D, R, 4, 2, QBF16, AFF>;
        if (waves == 8 && stages == 2) return &launch_t<D, R, 8, 2, QBF16, AFF>;
        return nullptr;
    }
    if (waves == 2 && stages == 2) return &launch_t<D, R, 2, 2, QBF16, AFF>;
    if (waves == 2 && stages == 3) return &launch_t<D, R, 2, 3, QBF16, AFF>;
    if (waves == 4 && stages == 2) return &launch_t<D, R, 4, 2, QBF16, AFF>;
    if (waves == 4 && stages == 3) return &launch_t<D, R, 4, 3, QBF16, AFF>;
    if (waves == 8 && stages == 2) return &launch_t<D, R, 8, 2, QBF16, AFF>;
    if (waves == 8 && stages == 3) return &launch_t<D, R, 8, 3, QBF16, AFF>;
    return nullptr;
}

template <int D, bool QBF16, bool AFF>
LaunchFn pick(int rows, int waves, int stages) {
    switch (rows) {
        case 1: return pick_shape<D, 1, QBF16, AFF>(waves, stages);
        case 2: return pick_shape<D, 2, QBF16, AFF>(waves, stages);
        case 4: return pick_shape<D, 4, QBF16, AFF>(waves, stages);
        case 8: return pick_shape<D, 8, QBF16, AFF>(waves, stages);
        case 16: return pick_shape<D, 16, QBF16, AFF>(waves, stages);
        default: return nullptr;
    }
}

template <int D, bool QBF16, bool AFF>
LaunchFn pick_rows(int rows_per_wg, int waves, int stages) {
#define Q8K4V_CASE(RB_, W_, S_) \
    if (rows_per_wg == 16 * RB_ && waves == W_ && stages == S_) return &launch_rows_t<D, RB_, W_, S_, QBF16, AFF>;
    if (AFF) {
        Q8K4V_CASE(1, 4, 2) Q8K4V_CASE(2, 4, 2) Q8K4V_CASE(1, 8, 2) Q8K4V_CASE(2, 8, 2)
        return nullptr;
    }
    Q8K4V_CASE(1, 2, 2) Q8K4V_CASE(1, 2, 3) Q8K4V_CASE(1, 4, 2) Q8K4V_CASE(1, 4, 3)
    Q8K4V_CASE(2, 2, 2) Q8K4V_CASE(2, 2, 3) Q8K4V_CASE(2, 4, 2) Q8K4V_CASE(2, 4, 3)
    Q8K4V_CASE(1, 8, 2) Q8K4V_CASE(2, 8, 2) Q8K4V_CASE(1, 8, 3) Q8K4V_CASE(2, 8, 3)
#undef Q8K4V_CASE
    return nullptr;
}

template <int D, int R, bool QBF16, bool AFF>
hipError_t launch_cascade_t(const AttnParams& pre, const AttnParams& suf, hipStream_t stream) {
    const int pre_blocks = work_blocks(pre);   // a multiple of 8: every block keeps its XCD
    const int suf_blocks = work_blocks(suf);
    hipLaunchKernelGGL((attn_cascade_kernel<D, R, QBF16, AFF>), dim3(pre_blocks + suf_blocks), dim3(256), 0, stream,
                       pre, suf, pre_blocks);
    return hipGetLastError();
}

template <int D, bool QBF16, bool AFF>
hipError_t pick_cascade(int rows, const AttnParams& pre, const AttnParams& suf, hipStream_t stream) {
    switch (rows) {
        case 4: return launch_cascade_t<D, 4, QBF16, AFF>(pre, suf, stream);
        case 8: return launch_cascade_t<D, 8, QBF16, AFF>(pre, suf, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D, int R, bool QBF16, bool AFF>
hipError_t launch_append_t(const AttnParams& kp, hipStream_t stream) {
    const int blocks = work_blocks(kp);
    hipLaunchKernelGGL((attn_dec2_append_kernel<D, R, QBF16, AFF>), dim3(blocks), dim3(256), 0, stream, kp);
    return hipGetLastError();
}

template <int D, bool QBF16, bool AFF>
LaunchFn pick_append(int rows) {
    switch (rows) {
        case 1: return &launch_append_t<D, 1, QBF16, AFF>;
        case 2: return &launch_append_t<D, 2, QBF16, AFF>;
        case 4: return &launch_append_t<D, 4, QBF16, AFF>;
        case 8: return &launch_append_t<D, 8, QBF16, AFF>;
        case 16: return &launch_append_t<D, 16, QBF16, AFF>;
        default: return nullptr;
    }
}

}  // namespace

// Decode with the step's token appended in the same launch: replicated-row
// plan with four waves and two stages (either codec).
bool decode_append_fusable(const Plan& plan, const q8k4v_cache& c) {
    (void)c;
    return plan.kernel == kDec2 && plan.waves == 4 && plan.stages == 2;
}

int32_t launch_dec2_append(const AttnParams& kp, const Plan& plan, int head_dim, bool qbf16, hipStream_t stream) {
    LaunchFn fn;
    if (kp.affine) {
        if (head_dim == 128) fn = qbf16 ? pick_append<128, true, true>(plan.rows) : pick_append<128, false, true>(plan.rows);
        else fn = qbf16 ? pick_append<64, true, true>(plan.rows) : pick_append<64, false, true>(plan.rows);
    } else {
        if (head_dim == 128) fn = qbf16 ? pick_append<128, true, false>(plan.rows) : pick_append<128, false, false>(plan.rows);
        else fn = qbf16 ? pick_append<64, true, false>(plan.rows) : pick_append<64, false, false>(plan.rows);
    }
    if (!fn) return fail(Q8K4V_EUNSUPPORTED, "attention: no appending decode kernel for this row count");
    const hipError_t e = fn(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return Q8K4V_OK;
}

// One launch of both cascade passes (prefix plan: 32-row blocks, 4 waves, 2
// stages; suffix plan: replicated rows, 4 or 8 rows, 4 waves, 2 stages).
bool cascade_fusable(const Plan& pre, const Plan& suf) {
    return pre.kernel == kRows && pre.rows_per_wg == 32 && pre.waves == 4 && pre.stages == 2 &&
           suf.kernel == kDec2 && (suf.rows == 4 || suf.rows == 8) && suf.waves == 4 && suf.stages == 2;
}

int32_t launch_cascade_fused(const AttnParams& pre, const AttnParams& suf, int head_dim, bool qbf16, int rows,
                             hipStream_t stream) {
    hipError_t e;
    if (pre.affine) {
        if (head_dim == 128) e = qbf16 ? pick_cascade<128, true, true>(rows, pre, suf, stream) : pick_cascade<128, false, true>(rows, pre, suf, stream);
        else e = qbf16 ? pick_cascade<64, true, true>(rows, pre, suf, stream) : pick_cascade<64, false, true>(rows, pre, suf, stream);
    } else {
        if (head_dim == 128) e = qbf16 ? pick_cascade<128, true, false>(rows, pre, suf, stream) : pick_cascade<128, false, false>(rows, pre, suf, stream);
        else e = qbf16 ? pick_cascade<64, true, false>(rows, pre, suf, stream) : pick_cascade<64, false, false>(rows, pre, suf, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "cascade kernel launch");
    return Q8K4V_OK;
}

int32_t launch_rows(const AttnParams& kp, const Plan& plan, int head_dim, bool qbf16, hipStream_t stream) {
    LaunchFn fn = nullptr;
    const int rw = plan.rows_per_wg, wv = plan.waves, st = plan.stages;
    if (kp.affine) {
        if (head_dim == 128) fn = qbf16 ? pick_rows<128, true, true>(rw, wv, st) : pick_rows<128, false, true>(rw, wv, st);
        else fn = qbf16 ? pick_rows<64, true, true>(rw, wv, st) : pick_rows<64, false, true>(rw, wv, st);
    } else {
        if (head_dim == 128) fn = qbf16 ? pick_rows<128, true, false>(rw, wv, st) : pick_rows<128, false, false>(rw, wv, st);
        else fn = qbf16 ? pick_rows<64, true, false>(rw, wv, st) : pick_rows<64, false, false>(rw, wv, st);
    }
    if (!fn) return fail(Q8K4V_EUNSUPPORTED, "attention: no row-block kernel for this rows/waves/stages combination");
    const hipError_t e = fn(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return Q8K4V_OK;
}

int32_t launch_dec2(const AttnParams& kp, const Plan& plan, int head_dim, bool qbf16, hipStream_t stream) {
    LaunchFn fn = nullptr;
    const int r = plan.rows, wv = plan.waves, st = plan.stages;
    if (kp.affine) {
        if (head_dim == 128) fn = qbf16 ? pick<128, true, true>(r, wv, st) : pick<128, false, true>(r, wv, st);
        else fn = qbf16 ? pick<64, true, true>(r, wv, st) : pick<64, false, true>(r, wv, st);
    } else {
        if (head_dim == 128) fn = qbf16 ? pick<128, true, false>(r, wv, st) : pick<128, false, false>(r, wv, st);
        else fn = qbf16 ? pick<64, true, false>(r, wv, st) : pick<64, false, false>(r, wv, st);
    }
    if (!fn) return fail(Q8K4V_EUNSUPPORTED, "attention: no paged-MFMA kernel for this rows/waves/stages combination");
    const hipError_t e = fn(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return Q8K4V_OK;
}

}  // namespace q8k4v
