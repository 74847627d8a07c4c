// Split-K ("flash-decoding") attention over the paged k8v4 cache on the
// vector ALUs of gfx950, for query blocks of up to 8 rows per kv head
// (decode: the GQA group; small verify blocks: drafts x group).
//
// What it computes: exact softmax attention over the dequantized cache
// (blog.123qwe.co.kr/?p=3927, section 5: the decode unit reads the k8v4
// cache; decode is bound by memory traffic).  Row r = (draft j, query head g
// of the group) of sequence b sees positions 0 .. L_b - W + j.
//
// Structure (per workgroup = one (sequence, kv head, split of pages)):
//  * each wavefront streams its own tiles of `TP` pages: the key codes, value
//    codes and scales of a tile are copied straight from HBM into the wave's
//    LDS stage (global_load_lds_dwordx4, 16 B per lane, fully coalesced);
//    when a tile is consumed its bytes move to registers and the copy of the
//    next tile is issued into the same stage, so one tile is in flight while
//    the current one is computed;
//  * keys: 8 (D=128) or 4 (D=64) lanes share a token, 16 dimensions each;
//    int8 codes become fp16 (1152 + code) with one byte permute per pair and
//    meet fp16 queries in v_dot2_f32_f16; the per-row bias 1152*sum(q) and
//    the key scale are applied once per token;
//  * partial dot products are summed through LDS by "softmax lanes" (row,
//    token); the tile maximum per row is a 16-lane DPP reduction; the running
//    max / sum follow the online softmax in the log2 domain;
//  * values: each lane owns D/64 dimension rows; eight int4 codes of a row
//    become four exact fp16 pairs (token t, t+4) and meet fp16 probabilities
//    already multiplied by the (token, group) value scale in v_dot2_f32_f16
//    with fp32 accumulation;
//  * the waves of a workgroup merge their (max, sum, output) in LDS; a
//    workgroup writes either the normalised output (single split) or its
//    split partial, which the combine kernel merges by log-sum-exp.
#include "attn_common.h"
#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

template <int D, int R, int WAVES, int TP, bool QBF16>
__global__ __launch_bounds__(64 * WAVES) void attn_valu_kernel(const AttnParams p) {
    constexpr int LPT = D / 16;            // key-phase lanes per token
    constexpr int TPL = D / 64;            // key-phase tokens per lane per page
    constexpr int NG = D / 32;             // value scale groups
    constexpr int DPL = D / 64;            // value-phase dimensions per lane
    constexpr int RPL = (R + 3) / 4;       // softmax rows per lane
    constexpr int KB = 16 * D;             // key code bytes per page
    constexpr int VB = 8 * D;              // value code bytes per page
    constexpr int SCH = 2 + 2 * NG;        // 16-byte scale chunks per page
    constexpr int SB = 16 * SCH;
    constexpr int STAGE = TP * (KB + VB + SB);
    constexpr int KPS = LPT * R + 4;       // padded floats per token of partial sums
    static_assert(TP * SCH <= 64, "scale chunks of a tile must fit one wavefront");

    __shared__ __attribute__((aligned(16))) uint8_t s_stage[WAVES][STAGE];
    __shared__ __attribute__((aligned(16))) float s_kpart[WAVES][TP * 16 * KPS];
    __shared__ __attribute__((aligned(16))) uint32_t s_p[WAVES][TP * NG * 8 * R];
    __shared__ float s_alpha[WAVES][R];
    __shared__ float s_ml[WAVES][R][2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    WorkItem w;
    if (!work_item(p, w)) return;
    const int kh = w.kh, b = w.b, L = w.L, pend = w.pend;
    const int G = p.G, W = p.W;
    if (w.pbeg >= pend) {
        if (w.split == 0 && !p.cascade) write_zero_rows<D>(p, w, 0, R);
        return;
    }

    // ---- queries: fp16 pairs of the lane's 16 dimensions, per row, pre-scaled
    // by a power of two so the row maximum lies in [1, 2)
    const int jc = lane % LPT;
    uint32_t qh[R][8];
    float bias_r[R], coef_r[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = r / G, g = r % G;
        const size_t qoff = (((size_t)b * W + j) * p.Hq + kh * G + g) * D + 16 * jc;
        float x[16];
        if (QBF16) {
            const u32x4* src = (const u32x4*)((const uint16_t*)p.q + qoff);
            const u32x4 a0 = src[0], a1 = src[1];
            const uint32_t w[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
                x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
            }
        } else {
            const f32x4* src = (const f32x4*)((const float*)p.q + qoff);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = src[i];
                x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
            }
        }
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(x[i]));
        mx = group_max<LPT>(mx);
        int e = 1;
        if (mx > 0.0f) (void)frexpf(mx, &e);
        e = min(max(e, -120), 120);
        const float sc = ldexpf(1.0f, 1 - e);
        float qsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 h0 = (_Float16)(x[2 * i] * sc);
            const _Float16 h1 = (_Float16)(x[2 * i + 1] * sc);
            qsum += (float)h0 + (float)h1;
            f16x2 hv = {h0, h1};
            qh[r][i] = as_u32(hv);
        }
        qsum = group_sum<LPT>(qsum);
        bias_r[r] = 1152.0f * qsum;
        coef_r[r] = p.scale_log2 * ldexpf(1.0f, e - 1);
    }

    // ---- softmax-lane view: lane = (row group rg, token t)
    const int rg = lane >> 4;
    const int tok = lane & 15;
    float m_l[RPL], l_l[RPL], bias_l[RPL], coef_l[RPL];
    int lim_l[RPL];     // visible positions of the lane's rows: pos < lim
#pragma unroll
    for (int k = 0; k < RPL; ++k) {
        m_l[k] = kNegInf;
        l_l[k] = 0.0f;
        bias_l[k] = 0.0f;
        coef_l[k] = 0.0f;
        const int r = rg + 4 * k;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            if (rr == r) { bias_l[k] = bias_r[rr]; coef_l[k] = coef_r[rr]; }
        }
        lim_l[k] = (r < R) ? (L - W + 1 + r / G) : 0;
    }
    float acc[R][DPL];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[r][e] = 0.0f;

    uint8_t* stage = s_stage[wave];
    const uint32_t stage_lds = lds_addr(stage);
    const int32_t* ptab = p.page_table + (size_t)b * p.max_pages;

    // issue the LDS copies of the tile starting at logical page pg
    auto issue_tile = [&](int pg) {
        int phys[TP];
#pragma unroll
        for (int i = 0; i < TP; ++i) phys[i] = (pg + i < pend) ? ptab[pg + i] : 0;
#pragma unroll
        for (int i = 0; i < TP; ++i) {
            if (pg + i < pend) {
                const size_t blk = (size_t)phys[i] * p.H + kh;
                const int8_t* kg = p.k_codes + blk * KB;
#pragma unroll
                for (int c = 0; c < KB / 1024; ++c)
                    lds_dma16(kg + c * 1024, lane * 16, stage_lds + i * KB + c * 1024);
                const uint8_t* vg = p.v_codes + blk * VB;
                if (VB >= 1024) {
#pragma unroll
                    for (int c = 0; c < VB / 1024; ++c)
                        lds_dma16(vg + c * 1024, lane * 16, stage_lds + TP * KB + i * VB + c * 1024);
                } else if (lane < VB / 16) {
                    lds_dma16(vg, lane * 16, stage_lds + TP * KB + i * VB);
                }
            }
        }
        // scales: lane -> (page i, chunk c); chunks 0-1 key scales, 2.. value scales
        const int si = lane / SCH, sc = lane % SCH;
        int sphys = 0;
#pragma unroll
        for (int i = 0; i < TP; ++i) sphys = (si == i) ? phys[i] : sphys;
        if (lane < TP * SCH && pg + si < pend) {
            const size_t blk = (size_t)sphys * p.H + kh;
            const uint8_t* src = (sc < 2) ? (const uint8_t*)(p.k_scales + blk * 16) + sc * 16
                                          : (const uint8_t*)(p.v_scales + blk * 16 * NG) + (sc - 2) * 16;
            lds_dma16_vaddr(src, stage_lds + TP * (KB + VB));
        }
    };

    const int step = WAVES * TP;
    int pg = w.pbeg + wave * TP;
    if (pg < pend) issue_tile(pg);

    for (; pg < pend; pg += step) {
        // ---- tile pg .. pg+TP-1 is (being) staged: wait, move to registers
        wait_vmem_all();
        u32x4 kreg[TP][TPL];
        uint32_t vreg[TP][2 * DPL];
        float ks_l[TP];
        uint16_t vs_l[TP][NG];
#pragma unroll
        for (int i = 0; i < TP; ++i) {
#pragma unroll
            for (int tt = 0; tt < TPL; ++tt)
                kreg[i][tt] = *(const u32x4*)(stage + i * KB + tt * 1024 + lane * 16);
            if (DPL == 2) {
                const u32x4 v = *(const u32x4*)(stage + TP * KB + i * VB + lane * 16);
                vreg[i][0] = v.x; vreg[i][1] = v.y; vreg[i][2 % (2 * DPL)] = v.z; vreg[i][3 % (2 * DPL)] = v.w;
            } else {
                const u32x2 v = *(const u32x2*)(stage + TP * KB + i * VB + lane * 8);
                vreg[i][0] = v.x; vreg[i][1] = v.y;
            }
            const uint8_t* sb = stage + TP * (KB + VB) + i * SB;
            ks_l[i] = h2f(*(const uint16_t*)(sb + 2 * tok));
#pragma unroll
            for (int g = 0; g < NG; ++g) vs_l[i][g] = *(const uint16_t*)(sb + 32 + 2 * (tok * NG + g));
        }
        wait_lds_all();
        if (pg + step < pend) issue_tile(pg + step);

        // ---- keys: partial dot products of the lane's 16 dimensions
        float* kpart = s_kpart[wave];
#pragma unroll
        for (int i = 0; i < TP; ++i) {
#pragma unroll
            for (int tt = 0; tt < TPL; ++tt) {
                const int t = lane / LPT + tt * (64 / LPT);
                float part[R];
#pragma unroll
                for (int r = 0; r < R; ++r) part[r] = 0.0f;
                const uint32_t kw[4] = {kreg[i][tt].x, kreg[i][tt].y, kreg[i][tt].z, kreg[i][tt].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t lo, hi;
                    k_codes_to_f16(kw[w], lo, hi);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        part[r] = dot2(lo, qh[r][2 * w], part[r]);
                        part[r] = dot2(hi, qh[r][2 * w + 1], part[r]);
                    }
                }
                float* dst = kpart + (i * 16 + t) * KPS + jc * R;
#pragma unroll
                for (int r = 0; r < R; ++r) dst[r] = part[r];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- softmax lanes: scores of (row, token) for the tile
        float sco[TP][RPL];
#pragma unroll
        for (int i = 0; i < TP; ++i) {
            const int pos = (pg + i) * 16 + tok;
#pragma unroll
            for (int k = 0; k < RPL; ++k) {
                const int r = rg + 4 * k;
                float sum = 0.0f;
                if (r < R) {
                    const float* src = kpart + (i * 16 + tok) * KPS + r;
#pragma unroll
                    for (int c = 0; c < LPT; ++c) sum += src[c * R];
                }
                const float s = (sum - bias_l[k]) * ks_l[i] * coef_l[k];
                sco[i][k] = (pos < lim_l[k] && pg + i < pend) ? s : kNegInf;
            }
        }
        float alpha_l[RPL];
#pragma unroll
        for (int k = 0; k < RPL; ++k) {
            float tmax = sco[0][k];
#pragma unroll
            for (int i = 1; i < TP; ++i) tmax = fmaxf(tmax, sco[i][k]);
            tmax = row16_max(tmax);
            const float m_new = fmaxf(m_l[k], tmax);
            const float ref = (m_new == kNegInf) ? 0.0f : m_new;
            alpha_l[k] = exp2_fast(m_l[k] - ref);
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < TP; ++i) {
                const float pr = exp2_fast(sco[i][k] - ref);
                sco[i][k] = pr;
                psum += pr;
            }
            l_l[k] = l_l[k] * alpha_l[k] + psum;
            m_l[k] = m_new;
        }
        // probabilities folded with the value scales, fp16, into the pair layout
        uint16_t* p16 = (uint16_t*)s_p[wave];
        const int kpair = (tok & 3) + 4 * (tok >> 3);
        const int half = (tok >> 2) & 1;
#pragma unroll
        for (int k = 0; k < RPL; ++k) {
            const int r = rg + 4 * k;
            if (r < R) {
                if (tok == 0) s_alpha[wave][r] = alpha_l[k];
#pragma unroll
                for (int i = 0; i < TP; ++i) {
                    const float pr = sco[i][k];
#pragma unroll
                    for (int g = 0; g < NG; ++g) {
                        const float pv = (pr > 0.0f) ? pr * h2f(vs_l[i][g]) : 0.0f;
                        const _Float16 h = (_Float16)pv;
                        p16[2 * (((i * NG + g) * 8 + kpair) * R + r) + half] = __builtin_bit_cast(uint16_t, h);
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- values: rescale the running outputs, then accumulate the tile
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float a = s_alpha[wave][r];
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[r][e] *= a;
        }
        const int g_v = (DPL * lane) / 32;
#pragma unroll
        for (int i = 0; i < TP; ++i) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                uint32_t cv[DPL][4];
#pragma unroll
                for (int e = 0; e < DPL; ++e) v_codes_to_f16(vreg[i][2 * e + hh], cv[e]);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const uint32_t* pw = s_p[wave] + ((i * NG + g_v) * 8 + 4 * hh + kk) * R;
                    uint32_t pr[R];
#pragma unroll
                    for (int r = 0; r < R; ++r) pr[r] = pw[r];
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int e = 0; e < DPL; ++e) acc[r][e] = dot2(cv[e][kk], pr[r], acc[r][e]);
                }
            }
        }
    }

    // ---- per-wave state to LDS, merge
#pragma unroll
    for (int k = 0; k < RPL; ++k) {
        const float lsum = row16_sum(l_l[k]);
        const int r = rg + 4 * k;
        if (r < R && tok == 0) {
            s_ml[wave][r][0] = m_l[k];
            s_ml[wave][r][1] = lsum;
        }
    }
    __syncthreads();        // every wave is done with its partial sums: reuse them for O
    float* s_o = &s_kpart[0][0];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < DPL; ++e) s_o[(wave * R + r) * D + DPL * lane + e] = acc[r][e];
    finish_workgroup<D, R, WAVES>(p, w, 0, s_ml, s_o, &s_stage[0][0], (int)sizeof(s_stage));
}

template <int D, int R, int WAVES, int TP, bool QBF16>
hipError_t launch_valu_t(const AttnParams& kp, hipStream_t stream) {
    const int total = kp.n_seqs * kp.H * kp.n_splits * kp.row_chunks;
    const int blocks = 8 * ((total + 7) / 8);
    hipLaunchKernelGGL((attn_valu_kernel<D, R, WAVES, TP, QBF16>), dim3(blocks), dim3(64 * WAVES), 0, stream, kp);
    return hipGetLastError();
}

using LaunchFn = hipError_t (*)(const AttnParams&, hipStream_t);

template <int D, int R, bool QBF16>
LaunchFn pick_shape(int waves, int tp) {
#define Q8K4V_CASE(WW, TT) if (waves == WW && tp == TT) return &launch_valu_t<D, R, WW, TT, QBF16>;
    Q8K4V_CASE(4, 2)
    Q8K4V_CASE(4, 1)
    Q8K4V_CASE(2, 2)
    Q8K4V_CASE(2, 4)
    Q8K4V_CASE(1, 4)
    Q8K4V_CASE(1, 2)
    Q8K4V_CASE(2, 1)
    Q8K4V_CASE(1, 1)
#undef Q8K4V_CASE
    return nullptr;
}

template <int D, bool QBF16>
LaunchFn pick_rows(int rows, int waves, int tp) {
    switch (rows) {
        case 1: return pick_shape<D, 1, QBF16>(waves, tp);
        case 2: return pick_shape<D, 2, QBF16>(waves, tp);
        case 4: return pick_shape<D, 4, QBF16>(waves, tp);
        case 8: return pick_shape<D, 8, QBF16>(waves, tp);
        default: return nullptr;
    }
}

template <int D>
hipError_t launch_combine_t(const AttnParams& kp, hipStream_t stream) {
    const int blocks = kp.n_seqs * kp.H * kp.R;
    hipLaunchKernelGGL((combine_kernel<D>), dim3(blocks), dim3(256), 0, stream, kp);
    return hipGetLastError();
}

template <int D>
hipError_t launch_combine_cascade_t(const AttnParams& kp, hipStream_t stream) {
    const int blocks = kp.n_seqs * kp.H * kp.R;
    hipLaunchKernelGGL((combine_cascade_kernel<D>), dim3(blocks), dim3(256), 0, stream, kp);
    return hipGetLastError();
}

}  // namespace

int32_t launch_valu(const AttnParams& kp, const Plan& plan, int head_dim, bool qbf16, hipStream_t stream) {
    LaunchFn fn = nullptr;
    if (head_dim == 128) fn = qbf16 ? pick_rows<128, true>(plan.rows, plan.waves, plan.tile_pages)
                                    : pick_rows<128, false>(plan.rows, plan.waves, plan.tile_pages);
    else fn = qbf16 ? pick_rows<64, true>(plan.rows, plan.waves, plan.tile_pages)
                    : pick_rows<64, false>(plan.rows, plan.waves, plan.tile_pages);
    if (!fn) return fail(Q8K4V_EUNSUPPORTED, "attention: no vector kernel for this rows/waves/tile combination");
    const hipError_t e = fn(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return Q8K4V_OK;
}

// Separate log-sum-exp combine of the split partials (when the fused combine
// is off).
int32_t launch_combine(const AttnParams& kp, int head_dim, int rows_per_wg, hipStream_t stream) {
    (void)rows_per_wg;
    const hipError_t e = head_dim == 128 ? launch_combine_t<128>(kp, stream) : launch_combine_t<64>(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
    return Q8K4V_OK;
}

// Combine of the shared-prefix cascade (prefix-pass and suffix-pass records).
int32_t launch_combine_cascade(const AttnParams& kp, int head_dim, hipStream_t stream) {
    const hipError_t e = head_dim == 128 ? launch_combine_cascade_t<128>(kp, stream) : launch_combine_cascade_t<64>(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "cascade combine kernel launch");
    return Q8K4V_OK;
}

}  // namespace q8k4v
