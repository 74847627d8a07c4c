// Split-K verify attention over the paged k8v4 cache for query blocks whose
// row count per kv head (n_draft drafts x GQA group) is not 1, 2, 4 or 8 --
// typically 12 to 128 rows -- on gfx950's 16x16 MFMAs, padded to 16 or 32
// rows per workgroup.  With many rows the query block is a dense contraction.
//
// What it computes: exact softmax attention over the dequantized cache;
// verifying several drafted tokens in the pass that one decode step costs
// (blog.123qwe.co.kr/?p=3927, section 5).  Row r = (draft j, group member g)
// of sequence b sees positions 0 .. L_b - W + j (causal among the drafts,
// whose keys/values are already appended).
//
// Per wavefront, tiles of 2 pages = 32 tokens, staged in LDS like the decode
// kernels (global_load_lds_dwordx4, key rows swizzled, next tile in flight
// while the current one is computed).  For each row block of 16 query rows:
//  * S^T = K Q^T on v_mfma_i32_16x16x64_i8: the 16 tokens of a page are the
//    rows, 16 query rows the columns, 64 dimensions per instruction; a lane's
//    operand is 16 stored int8 key codes of one token.  Queries are 15-bit
//    fixed point split into two int8 parts (two instructions per k-step),
//    exact int32 accumulation.  The token feeding row m of the instruction is
//    permuted (pi) so that the 4 scores a lane receives are the tokens one
//    32-bit word of a value row unpacks into;
//  * online softmax per query row in the log2 domain; the scores never leave
//    registers: the probabilities, times the (token, value group) scale and
//    rounded once to fp16, are directly the A operand of
//  * O = P V on v_mfma_f32_16x16x32_f16: 16 rows x 16 dimensions, k = the 32
//    tokens of the tile, values as exact fp16 codes, fp32 accumulation.
#include "attn_common.h"
#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int RW>
Q8K4V_DEV float m_l_row(const float (*s_ml)[RW][2], int wave, int rl) { return s_ml[wave][rl][0]; }

Q8K4V_DEV int pi_slot(int q, int i) {
    const int a = 2 * (q & 1) + 8 * (q >> 1);
    return a + ((i & 1) ? 4 : 0) + (i >> 1);      // i: 0->a, 1->a+4, 2->a+1, 3->a+5
}

template <int D, int RB, int WAVES, bool QBF16>
__global__ __launch_bounds__(64 * WAVES) void attn_mfma_kernel(const AttnParams p) {
    constexpr int RW = 16 * RB;            // query rows per workgroup (row chunk)
    constexpr int TP = 2;                  // pages per tile (32 tokens)
    constexpr int KB = 16 * D, VB = 8 * D;
    constexpr int NG = D / 32;
    constexpr int SB = 32 + 32 * NG;
    constexpr int CPR = D / 16;            // 16-byte chunks per key row
    constexpr int KS = D / 64;             // 64-dimension k-steps
    constexpr int NDT = D / 16;            // 16-dimension output tiles
    constexpr int STAGE = TP * (KB + VB + SB);

    __shared__ __attribute__((aligned(16))) uint8_t s_stage[WAVES][STAGE];
    __shared__ __attribute__((aligned(16))) float s_merge[RW * D];
    __shared__ __attribute__((aligned(16))) int8_t s_q[RB][16][2][D];     // [row block][row][hi/lo][dim]
    __shared__ float s_qc[RW];
    __shared__ __attribute__((aligned(16))) float s_alpha[WAVES][RB][16];
    __shared__ float s_ml[WAVES][RW][2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WorkItem w;
    if (!work_item(p, w)) return;
    const int r0 = w.rchunk * RW;
    if (w.pbeg >= w.pend) {
        if (w.split == 0 && !p.cascade) write_zero_rows<D>(p, w, r0, RW);
        return;
    }
    const int n16 = lane & 15;             // MFMA column (query row) / output dimension
    const int q4 = lane >> 4;              // MFMA lane group
    const int kh = w.kh;
    const int pend = w.pend;
    uint8_t* stage = s_stage[wave];
    const uint32_t stage_lds = lds_addr(stage);
    const int32_t* ptab = p.page_table + (size_t)w.b * p.max_pages;

    uint32_t kdma_off[KB / 1024];
#pragma unroll
    for (int c = 0; c < KB / 1024; ++c) {
        const int s = 64 * c + lane;
        const int t = s / CPR, cc = (s % CPR) ^ (t % CPR);
        kdma_off[c] = (uint32_t)(t * D + 16 * cc);
    }
    auto issue_tile = [&](int pg, const int (&ids)[TP]) {
#pragma unroll
        for (int i = 0; i < TP; ++i) {
            if (pg + i < pend) {
                const size_t blk_id = (size_t)sgpr((uint32_t)ids[i]) * p.H + kh;
                const int8_t* kg = p.k_codes + blk_id * KB;
#pragma unroll
                for (int c = 0; c < KB / 1024; ++c) lds_dma16(kg, kdma_off[c], stage_lds + i * KB + c * 1024);
                const uint8_t* vg = p.v_codes + blk_id * VB;
                if (VB >= 1024) {
#pragma unroll
                    for (int c = 0; c < VB / 1024; ++c)
                        lds_dma16(vg + c * 1024, lane * 16, stage_lds + TP * KB + i * VB + c * 1024);
                } else if (lane < VB / 16) {
                    lds_dma16(vg, lane * 16, stage_lds + TP * KB + i * VB);
                }
                const uint32_t sl = stage_lds + TP * (KB + VB) + i * SB;
                if (lane < 2) lds_dma16(p.k_scales + blk_id * 16, lane * 16, sl);
                if (lane < 2 * NG) lds_dma16(p.v_scales + blk_id * 16 * NG, lane * 16, sl + 32);
            }
        }
    };
    auto load_ids = [&](int pg, int (&ids)[TP]) {
#pragma unroll
        for (int i = 0; i < TP; ++i) ids[i] = (pg + i < pend) ? ptab[pg + i] : 0;
    };

    const int step = WAVES * TP;
    int pg = w.pbeg + wave * TP;
    int ids_next[TP];
    {
        int ids0[TP];
        load_ids(pg, ids0);
        if (pg < pend) issue_tile(pg, ids0);
        load_ids(pg + step, ids_next);
    }

    // ---- queries: 15-bit fixed point per row, int8 hi/lo parts in LDS;
    // every wave prepares a share of the rows, 16 lanes per row
    {
        constexpr int DPLQ = D / 16;
        const int part = lane & 15;
        for (int rl = wave * 4 + (lane >> 4); rl < RW; rl += 4 * WAVES) {
            const int r = r0 + rl;
            float x[DPLQ];
            if (r < p.R) {
                const size_t qoff = out_index(p, w.b, w.kh, r, D) + DPLQ * part;
#pragma unroll
                for (int d = 0; d < DPLQ; ++d)
                    x[d] = QBF16 ? bf16_to_f32(((const uint16_t*)p.q)[qoff + d]) : ((const float*)p.q)[qoff + d];
            } else {
#pragma unroll
                for (int d = 0; d < DPLQ; ++d) x[d] = 0.0f;
            }
            float mx = 0.0f;
#pragma unroll
            for (int d = 0; d < DPLQ; ++d) mx = fmaxf(mx, fabsf(x[d]));
            mx = row16_max(mx);
            int e = 0;
            if (mx > 0.0f) (void)frexpf(mx, &e);
            e = min(max(e, -110), 110);
            const float sc = ldexpf(1.0f, 14 - e);
#pragma unroll
            for (int d = 0; d < DPLQ; ++d) {
                const int Q = (int)rintf(x[d] * sc);
                const int hi = (Q + 128) >> 8;
                s_q[rl >> 4][rl & 15][0][DPLQ * part + d] = (int8_t)hi;
                s_q[rl >> 4][rl & 15][1][DPLQ * part + d] = (int8_t)(Q - 256 * hi);
            }
            if (part == 0) s_qc[rl] = p.scale_log2 * ldexpf(1.0f, e - 14);
        }
    }
    __syncthreads();
    // B operands of S^T: lane (n, q) holds dims 64ks + 16q .. +15 of row n
    u32x4 qb[RB][KS][2];
    float coef_l[RB];
    int lim_l[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) qb[rb][ks][hl] = *(const u32x4*)&s_q[rb][n16][hl][64 * ks + 16 * q4];
        const int r = r0 + 16 * rb + n16;
        coef_l[rb] = s_qc[16 * rb + n16];
        lim_l[rb] = (r < p.R) ? (w.L - p.W + 1 + r / p.G) : 0;
    }

    float m_l[RB], l_l[RB];                // running max / partial sum of row n16 of block rb
    f32x4 acc[RB][NDT];                    // O: lane (n, q) holds rows 4q+i of dim 16dt + n
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_l[rb] = kNegInf;
        l_l[rb] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[rb][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // A operand of S^T: lane (m, q) holds token slot pi(m) of the page, dims 64ks + 16q
    const int kslot = pi_slot(n16 >> 2, n16 & 3);
    const int sa = 2 * (q4 & 1) + 8 * (q4 >> 1);   // first slot of the lane's score tokens

    for (; pg < pend; pg += step) {
        wait_vmem_all();
        u32x4 krow[TP][KS];
        uint32_t vw[TP][NDT];
        uint32_t ks01[TP], ks45[TP];
        uint32_t vsw[TP][4][(NG + 1) / 2];
#pragma unroll
        for (int i = 0; i < TP; ++i) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = 4 * ks + q4;
                krow[i][ks] = *(const u32x4*)(stage + i * KB + (kslot * CPR + (c ^ (kslot % CPR))) * 16);
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                vw[i][dt] = *(const uint32_t*)(stage + TP * KB + i * VB + (16 * dt + n16) * 8 + 4 * (q4 >> 1));
            const uint8_t* sbase = stage + TP * (KB + VB) + i * SB;
            ks01[i] = *(const uint32_t*)(sbase + 2 * sa);
            ks45[i] = *(const uint32_t*)(sbase + 2 * (sa + 4));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int slot = pi_slot(q4, k);
                if (NG == 4) {
                    const u32x2 v = *(const u32x2*)(sbase + 32 + 8 * slot);
                    vsw[i][k][0] = v.x;
                    vsw[i][k][(NG + 1) / 2 - 1] = v.y;
                } else {
                    vsw[i][k][0] = *(const uint32_t*)(sbase + 32 + 4 * slot);
                }
            }
        }
        wait_lds_all();
        const int pg_next = pg + step;
        if (pg_next < pend) {
            issue_tile(pg_next, ids_next);
            load_ids(pg_next + step, ids_next);
        }

        // ---- scores S^T (lane (n, q): tokens pi(q, k) of each page, query row n)
        float sc[RB][TP][4];
#pragma unroll
        for (int i = 0; i < TP; ++i) {
            const float ksf[4] = {h2f((uint16_t)ks01[i]), h2f((uint16_t)ks45[i]), h2f((uint16_t)(ks01[i] >> 16)),
                                  h2f((uint16_t)(ks45[i] >> 16))};
            const bool page_ok = (pg + i < pend);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                i32x4_t chi = {0, 0, 0, 0}, clo = {0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const i32x4_t a = __builtin_bit_cast(i32x4_t, krow[i][ks]);
                    chi = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, __builtin_bit_cast(i32x4_t, qb[rb][ks][0]), chi, 0, 0, 0);
                    clo = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, __builtin_bit_cast(i32x4_t, qb[rb][ks][1]), clo, 0, 0, 0);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int pos = (pg + i) * 16 + pi_slot(q4, k);
                    const float v = (float)(256 * chi[k] + clo[k]) * (ksf[k] * coef_l[rb]);
                    sc[rb][i][k] = (page_ok && pos < lim_l[rb]) ? v : kNegInf;
                }
            }
        }
        // ---- online softmax per query row
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float tmax = kNegInf;
#pragma unroll
            for (int i = 0; i < TP; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k) tmax = fmaxf(tmax, sc[rb][i][k]);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_l[rb], tmax);
            const float ref = (m_new == kNegInf) ? 0.0f : m_new;
            const float alpha = exp2_fast(m_l[rb] - ref);
            m_l[rb] = m_new;
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < TP; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    sc[rb][i][k] = exp2_fast(sc[rb][i][k] - ref);
                    psum += sc[rb][i][k];
                }
            l_l[rb] = l_l[rb] * alpha + psum;
            if (__builtin_amdgcn_ballot_w64(alpha < 1.0f) != 0) {
                // output rows 4q+i of this lane need the alphas of rows 4q..4q+3
                if (q4 == 0) s_alpha[wave][rb][n16] = alpha;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const f32x4 a4 = *(const f32x4*)&s_alpha[wave][rb][4 * q4];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) acc[rb][dt] *= a4;
            }
        }
        // ---- O += P V, k = the tile's 32 tokens in the order of the scores
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            f16x8_t A[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < TP; ++i)
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint16_t sb = (uint16_t)(vsw[i][k][g >> 1] >> (16 * (g & 1)));
                        const float pv = (sc[rb][i][k] > 0.0f) ? sc[rb][i][k] * h2f(sb) : 0.0f;
                        A[rb][4 * i + k] = (_Float16)pv;
                    }
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) {
                const int dt = 2 * g + dd;
                uint32_t bw[4];
#pragma unroll
                for (int i = 0; i < TP; ++i) {
                    uint32_t cv[4];
                    v_codes_to_f16(vw[i][dt] >> (8 * (q4 & 1)), cv);
                    bw[2 * i] = cv[0];
                    bw[2 * i + 1] = cv[1];
                }
                const f16x8_t B = __builtin_bit_cast(f16x8_t, u32x4{bw[0], bw[1], bw[2], bw[3]});
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[rb], B, acc[rb][dt], 0, 0, 0);
            }
        }
    }

    // ---- merge the waves: per-row reference, then each wave adds its scaled
    // output into one shared buffer in wave order (deterministic)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float l = l_l[rb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (q4 == 0) {
            s_ml[wave][16 * rb + n16][0] = m_l[rb];
            s_ml[wave][16 * rb + n16][1] = l;
        }
    }
    __syncthreads();
    float* s_o = (float*)&s_merge[0];
#pragma unroll
    for (int wv = 0; wv < WAVES; ++wv) {
        if (wave == wv) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rl = 16 * rb + 4 * q4 + i;
                    float M = kNegInf;
#pragma unroll
                    for (int u = 0; u < WAVES; ++u) M = fmaxf(M, s_ml[u][rl][0]);
                    const float f = exp2_fast(m_l_row(s_ml, wave, rl) - ((M == kNegInf) ? 0.0f : M));
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        float* dst = s_o + rl * D + 16 * dt + n16;
                        const float v = acc[rb][dt][i] * f;
                        *dst = (wv == 0) ? v : *dst + v;
                    }
                }
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < RW * D; e += 64 * WAVES) {
        const int rl = e / D, d = e % D;
        const int r = r0 + rl;
        if (r >= p.R) continue;
        float M = kNegInf;
#pragma unroll
        for (int u = 0; u < WAVES; ++u) M = fmaxf(M, s_ml[u][rl][0]);
        const float ref = (M == kNegInf) ? 0.0f : M;
        float Ls = 0.0f;
#pragma unroll
        for (int u = 0; u < WAVES; ++u) Ls += s_ml[u][rl][1] * exp2_fast(s_ml[u][rl][0] - ref);
        emit_element<D>(p, w, r, d, M, Ls, s_o[rl * D + d]);
    }
    if (p.fused && !p.direct) __syncthreads();   // s_merge is read above; the merge reuses the ring
    fused_tail<D, RW>(p, w, r0, &s_stage[0][0], (int)sizeof(s_stage));
}

template <int D, int RB, int WAVES, bool QBF16>
hipError_t launch_t(const AttnParams& kp, hipStream_t stream) {
    const int total = kp.n_seqs * kp.H * kp.n_splits * kp.row_chunks;
    const int blocks = 8 * ((total + 7) / 8);
    hipLaunchKernelGGL((attn_mfma_kernel<D, RB, WAVES, QBF16>), dim3(blocks), dim3(64 * WAVES), 0, stream, kp);
    return hipGetLastError();
}

using LaunchFn = hipError_t (*)(const AttnParams&, hipStream_t);

template <int D, bool QBF16>
LaunchFn pick(int rows_per_wg, int waves) {
#define Q8K4V_CASE(RR, WW) if (rows_per_wg == 16 * RR && waves == WW) return &launch_t<D, RR, WW, QBF16>;
    Q8K4V_CASE(1, 1) Q8K4V_CASE(1, 2) Q8K4V_CASE(1, 4)
    Q8K4V_CASE(2, 1) Q8K4V_CASE(2, 2) Q8K4V_CASE(2, 4)
#undef Q8K4V_CASE
    return nullptr;
}

}  // namespace

int32_t launch_mfma(const AttnParams& kp, const Plan& plan, int head_dim, bool qbf16, hipStream_t stream) {
    LaunchFn fn = nullptr;
    if (head_dim == 128) fn = qbf16 ? pick<128, true>(plan.rows_per_wg, plan.waves) : pick<128, false>(plan.rows_per_wg, plan.waves);
    else fn = qbf16 ? pick<64, true>(plan.rows_per_wg, plan.waves) : pick<64, false>(plan.rows_per_wg, plan.waves);
    if (!fn) return fail(Q8K4V_EUNSUPPORTED, "attention: no MFMA kernel for this rows/waves combination");
    const hipError_t e = fn(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return Q8K4V_OK;
}

}  // namespace q8k4v
