// Split-K decode attention over the paged k8v4 cache for query blocks of 4 or
// 8 rows per kv head (a GQA group of 4 or 8, or drafts x group), with both
// contractions on gfx950's 4x4x4 block MFMAs.
//
// What it computes: exact softmax attention over the dequantized cache (the
// decode unit of blog.123qwe.co.kr/?p=3927, section 5); row r = (draft j,
// group member g) of sequence b sees positions 0 .. L_b - W + j.
//
// Why these MFMAs: v_mfma_*_4x4x4_16b_* hold 16 independent 4x4x4 blocks.
// With the 4 query rows of a group as one block side every multiply-add is
// useful -- a dense 4-row contraction, not a padded 16- or 32-row tile -- and
// the multiply-adds leave the vector ALUs, which then only unpack values.
//
// Per wavefront, tiles of 4 pages = 64 tokens:
//  * the tile's key codes (row-swizzled in LDS), value codes and scales are
//    copied from HBM into the wave's LDS stage with global_load_lds_dwordx4;
//    at the top of a tile they move to registers and the copy of the next
//    tile is issued into the same stage, so one tile is in flight while the
//    current one is computed; the page ids of the tile after next are
//    fetched during the compute so no table lookup sits on the critical path;
//  * S^T = K Q^T on v_mfma_i32_4x4x4_16b_i8: block b takes 4 tokens (rows)
//    and the 4 query rows (columns), 4 dimensions per instruction.  The int8
//    key codes are the operand as stored.  Each query row is held as a
//    15-bit fixed-point number split into two int8 parts (q ~ (256*hi + lo) *
//    2^(e-14)), two instructions per k-step, exact int32 accumulation;
//  * online softmax per row in the log2 domain; the probabilities times each
//    token's value-group scale, rounded once to fp16, go to LDS in the token
//    order of the value unpacking;
//  * O = P V on v_mfma_f32_4x4x4_16b_f16: block b covers 4 output dimensions,
//    k = 4 tokens; values enter as exact fp16 codes (nibble masked under the
//    fp16 exponent, offset removed by a packed add), fp32 accumulation.
// Token order: within a page, k-step q (0..3) takes slots
// pi(q) = {a, a+4, a+1, a+5} with a = 2(q&1) + 8(q>>1), the pairs that one
// 32-bit word of a value row unpacks into.
#include "attn_common.h"
#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

Q8K4V_DEV int pi_slot(int q, int i) {
    const int a = 2 * (q & 1) + 8 * (q >> 1);
    return a + ((i & 1) ? 4 : 0) + (i >> 1);      // i: 0->a, 1->a+4, 2->a+1, 3->a+5
}

template <int D, int RB4, int WAVES, bool QBF16>
__global__ __launch_bounds__(64 * WAVES) void attn_bmfma_kernel(const AttnParams p) {
    constexpr int R = 4 * RB4;             // query rows per kv head
    constexpr int TP = 4;                  // pages per tile (64 tokens)
    constexpr int KB = 16 * D, VB = 8 * D;
    constexpr int NG = D / 32;
    constexpr int SB = 32 + 32 * NG;       // scale bytes per page: keys 32, values 32*NG
    constexpr int CPR = D / 16;            // 16-byte chunks per key row
    constexpr int KSTEP = D / 4;           // 4-dimension k-steps
    constexpr int DH = D / 64;             // 64-dimension halves of the output
    constexpr int STAGE = TP * (KB + VB + SB);

    __shared__ __attribute__((aligned(16))) uint8_t s_stage[WAVES][STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t s_p[WAVES][NG][R][TP][16];
    __shared__ float s_ml[WAVES][R][2];
    __shared__ __attribute__((aligned(16))) uint32_t s_q[RB4][4][KSTEP][2];   // int8x4 hi, lo
    __shared__ float s_qc[R];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WorkItem w;
    if (!work_item(p, w)) return;
    if (w.pbeg >= w.pend) {
        if (w.split == 0 && !p.cascade) write_zero_rows<D>(p, w, 0, R);
        return;
    }
    const int blk = lane >> 2;             // MFMA block
    const int j4 = lane & 3;               // row / column inside the block
    const int kh = w.kh;
    const int pend = w.pend;
    uint8_t* stage = s_stage[wave];
    const uint32_t stage_lds = lds_addr(stage);
    const int32_t* ptab = p.page_table + (size_t)w.b * p.max_pages;

    // key rows are staged with chunk c of slot t at position t*CPR + (c ^ (t % CPR))
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

    // the first tile's copy goes out before the query prologue
    const int step = WAVES * TP;
    int pg = w.pbeg + wave * TP;
    int ids_next[TP];
    {
        int ids0[TP];
        load_ids(pg, ids0);
        if (pg < pend) issue_tile(pg, ids0);
        load_ids(pg + step, ids_next);
    }

    // ---- queries (B operand), once per workgroup in LDS: row r as a 15-bit
    // fixed-point number Q = rne(q * 2^(14-e)) (2^(e-1) <= max|q| < 2^e),
    // stored as int8 parts hi = (Q + 128) >> 8, lo = Q - 256 hi
    if (wave == 0) {
        constexpr int DPLQ = D / 16;
        const int rr = lane >> 4, part = lane & 15;
#pragma unroll
        for (int s = 0; s < RB4; ++s) {
            const int r = 4 * s + rr;
            const size_t qoff = out_index(p, w.b, w.kh, r, D) + DPLQ * part;
            float x[DPLQ];
#pragma unroll
            for (int d = 0; d < DPLQ; ++d)
                x[d] = QBF16 ? bf16_to_f32(((const uint16_t*)p.q)[qoff + d]) : ((const float*)p.q)[qoff + d];
            float mx = 0.0f;
#pragma unroll
            for (int d = 0; d < DPLQ; ++d) mx = fmaxf(mx, fabsf(x[d]));
            mx = row16_max(mx);
            int e = 0;
            if (mx > 0.0f) (void)frexpf(mx, &e);
            e = min(max(e, -110), 110);
            const float sc = ldexpf(1.0f, 14 - e);
#pragma unroll
            for (int d = 0; d < DPLQ; d += 4) {
                uint32_t hi4 = 0, lo4 = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int Q = (int)rintf(x[d + t] * sc);
                    const int hi = (Q + 128) >> 8;
                    const int lo = Q - 256 * hi;
                    hi4 |= (uint32_t)(hi & 0xFF) << (8 * t);
                    lo4 |= (uint32_t)(lo & 0xFF) << (8 * t);
                }
                const int k = (DPLQ * part + d) / 4;
                s_q[s][rr][k][0] = hi4;
                s_q[s][rr][k][1] = lo4;
            }
            if (part == 0) s_qc[r] = p.scale_log2 * ldexpf(1.0f, e - 14);
        }
    }
    __syncthreads();
    float coef_l[RB4];
    int lim_l[RB4];
#pragma unroll
    for (int s = 0; s < RB4; ++s) {
        const int r = 4 * s + j4;
        coef_l[s] = s_qc[r];
        lim_l[s] = w.L - p.W + 1 + r / p.G;
    }

    float m_l[RB4], l_l[RB4];              // running max / partial sum of row j4 (+4s)
    f32x4 acc[RB4][DH];                    // O: lane (b, n) holds rows 0..3 (+4s) of dim 64h + 4b + n
#pragma unroll
    for (int s = 0; s < RB4; ++s) {
        m_l[s] = kNegInf;
        l_l[s] = 0.0f;
#pragma unroll
        for (int h = 0; h < DH; ++h) acc[s][h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // lane (b, i) holds the key row of token (page b>>2, slot pi(b&3, i))
    const int kpage = blk >> 2;
    const int kq = blk & 3;
    const int kslot = pi_slot(kq, j4);
    const int sa = 2 * (kq & 1) + 8 * (kq >> 1);      // first slot of the lane's k-step
    // lane (b, n) in P V: output dimension 64h + 4b + n
    const int vdim = 4 * blk + j4;

    for (; pg < pend; pg += step) {
        wait_vmem_all();
        // ---- move the staged tile to registers
        u32x4 krow[CPR];
#pragma unroll
        for (int c = 0; c < CPR; ++c)
            krow[c] = *(const u32x4*)(stage + kpage * KB + (kslot * CPR + (c ^ (kslot % CPR))) * 16);
        u32x2 vrow[TP][DH];
#pragma unroll
        for (int i = 0; i < TP; ++i)
#pragma unroll
            for (int h = 0; h < DH; ++h)
                vrow[i][h] = *(const u32x2*)(stage + TP * KB + i * VB + (64 * h + vdim) * 8);
        const uint8_t* sbase = stage + TP * (KB + VB) + kpage * SB;
        const uint32_t ks01 = *(const uint32_t*)(sbase + 2 * sa);          // slots a, a+1
        const uint32_t ks45 = *(const uint32_t*)(sbase + 2 * (sa + 4));    // slots a+4, a+5
        uint32_t vsw[4][(NG + 1) / 2];                                      // value scales of the 4 slots
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int slot = pi_slot(kq, i);
            if (NG == 4) {
                const u32x2 v = *(const u32x2*)(sbase + 32 + 8 * slot);
                vsw[i][0] = v.x;
                vsw[i][(NG + 1) / 2 - 1] = v.y;
            } else {
                vsw[i][0] = *(const uint32_t*)(sbase + 32 + 4 * slot);
            }
        }
        wait_lds_all();
        const int pg_next = pg + step;
        if (pg_next < pend) {
            issue_tile(pg_next, ids_next);
            load_ids(pg_next + step, ids_next);
        }

        // ---- S^T = K Q^T, int8 x int8 -> int32 (two accumulators per part
        // so consecutive instructions do not wait on each other)
        i32x4_t shi[RB4][2], slo[RB4][2];
#pragma unroll
        for (int s = 0; s < RB4; ++s)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                shi[s][u] = i32x4_t{0, 0, 0, 0};
                slo[s][u] = i32x4_t{0, 0, 0, 0};
            }
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            const uint32_t kw[4] = {krow[c].x, krow[c].y, krow[c].z, krow[c].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int s = 0; s < RB4; ++s) {
                    const u32x2 qv = *(const u32x2*)&s_q[s][j4][4 * c + t][0];
                    shi[s][t & 1] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)kw[t], (int)qv.x, shi[s][t & 1], 0, 0, 0);
                    slo[s][t & 1] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)kw[t], (int)qv.y, slo[s][t & 1], 0, 0, 0);
                }
            }
        }
        // ---- scores of tokens (page kpage, slots pi(kq, i)) for row j4 (+4s)
        const float ksf[4] = {h2f((uint16_t)ks01), h2f((uint16_t)ks45), h2f((uint16_t)(ks01 >> 16)),
                              h2f((uint16_t)(ks45 >> 16))};
        const bool page_ok = (pg + kpage < pend);
#pragma unroll
        for (int s = 0; s < RB4; ++s) {
            float sc4[4];
            float tmax = kNegInf;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pos = (pg + kpage) * 16 + pi_slot(kq, i);
                const int dot = 256 * (shi[s][0][i] + shi[s][1][i]) + (slo[s][0][i] + slo[s][1][i]);
                const float v = (float)dot * (ksf[i] * coef_l[s]);
                sc4[i] = (page_ok && pos < lim_l[s]) ? v : kNegInf;
                tmax = fmaxf(tmax, sc4[i]);
            }
            // row max over the 16 lanes holding row j4: same j4, all blocks
            tmax = fmaxf(tmax, dpp<0x124>(tmax));       // row_ror:4
            tmax = fmaxf(tmax, dpp<0x128>(tmax));       // row_ror:8
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_l[s], tmax);
            const float ref = (m_new == kNegInf) ? 0.0f : m_new;
            const float alpha = exp2_fast(m_l[s] - ref);
            m_l[s] = m_new;
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc4[i] = exp2_fast(sc4[i] - ref);
                psum += sc4[i];
            }
            l_l[s] = l_l[s] * alpha + psum;
            // rescale O rows 0..3 (+4s): alpha of row m sits in the lanes with j4 == m
            if (__builtin_amdgcn_ballot_w64(alpha < 1.0f) != 0) {
                const int ai = __builtin_bit_cast(int, alpha);
                const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(ai, 0x00, 0xF, 0xF, false));
                const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(ai, 0x55, 0xF, 0xF, false));
                const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(ai, 0xAA, 0xF, 0xF, false));
                const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(ai, 0xFF, 0xF, 0xF, false));
#pragma unroll
                for (int h = 0; h < DH; ++h) {
                    acc[s][h][0] *= a0; acc[s][h][1] *= a1; acc[s][h][2] *= a2; acc[s][h][3] *= a3;
                }
            }
            // probabilities x value scale, fp16, into s_p[g][row][page][pi order]
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                _Float16 hv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint16_t sb = (uint16_t)(vsw[i][g >> 1] >> (16 * (g & 1)));
                    const float pv = (sc4[i] > 0.0f) ? sc4[i] * h2f(sb) : 0.0f;
                    hv[i] = (_Float16)pv;
                }
                const f16x4_t v4 = {hv[0], hv[1], hv[2], hv[3]};
                *(f16x4_t*)&s_p[wave][g][4 * s + j4][kpage][4 * kq] = v4;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- O += P V
#pragma unroll
        for (int i = 0; i < TP; ++i) {
#pragma unroll
            for (int h = 0; h < DH; ++h) {
                const int g = (64 * h + 4 * blk) / 32;
#pragma unroll
                for (int wd = 0; wd < 2; ++wd) {
                    uint32_t cv[4];
                    v_codes_to_f16(wd == 0 ? vrow[i][h].x : vrow[i][h].y, cv);
#pragma unroll
                    for (int hq = 0; hq < 2; ++hq) {
                        const int q = 2 * wd + hq;
                        const f16x4_t B = __builtin_bit_cast(f16x4_t, u32x2{cv[2 * hq], cv[2 * hq + 1]});
#pragma unroll
                        for (int s = 0; s < RB4; ++s) {
                            const f16x4_t A = *(const f16x4_t*)&s_p[wave][g][4 * s + j4][i][4 * q];
                            acc[s][h] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, B, acc[s][h], 0, 0, 0);
                        }
                    }
                }
            }
        }
    }

    // ---- per-wave state to LDS, merge
#pragma unroll
    for (int s = 0; s < RB4; ++s) {
        float l = l_l[s];
        l += dpp<0x124>(l);
        l += dpp<0x128>(l);
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (blk == 0) {
            s_ml[wave][4 * s + j4][0] = m_l[s];
            s_ml[wave][4 * s + j4][1] = l;
        }
    }
    __syncthreads();        // every wave is done with its stage: reuse it for O
    float* s_o = (float*)&s_stage[0][0];
#pragma unroll
    for (int s = 0; s < RB4; ++s)
#pragma unroll
        for (int h = 0; h < DH; ++h)
#pragma unroll
            for (int m = 0; m < 4; ++m) s_o[(wave * R + 4 * s + m) * D + 64 * h + vdim] = acc[s][h][m];
    finish_workgroup<D, R, WAVES>(p, w, 0, s_ml, s_o, &s_stage[0][0], (int)sizeof(s_stage));
}

template <int D, int RB4, int WAVES, bool QBF16>
hipError_t launch_t(const AttnParams& kp, hipStream_t stream) {
    const int total = kp.n_seqs * kp.H * kp.n_splits * kp.row_chunks;
    const int blocks = 8 * ((total + 7) / 8);
    hipLaunchKernelGGL((attn_bmfma_kernel<D, RB4, WAVES, QBF16>), dim3(blocks), dim3(64 * WAVES), 0, stream, kp);
    return hipGetLastError();
}

using LaunchFn = hipError_t (*)(const AttnParams&, hipStream_t);

template <int D, bool QBF16>
LaunchFn pick(int rows, int waves) {
#define Q8K4V_CASE(RR, WW) if (rows == 4 * RR && waves == WW) return &launch_t<D, RR, WW, QBF16>;
    Q8K4V_CASE(1, 1) Q8K4V_CASE(1, 2) Q8K4V_CASE(1, 4)
    Q8K4V_CASE(2, 1) Q8K4V_CASE(2, 2) Q8K4V_CASE(2, 4)
#undef Q8K4V_CASE
    return nullptr;
}

}  // namespace

int32_t launch_bmfma(const AttnParams& kp, const Plan& plan, int head_dim, bool qbf16, hipStream_t stream) {
    LaunchFn fn = nullptr;
    if (head_dim == 128) fn = qbf16 ? pick<128, true>(plan.rows, plan.waves) : pick<128, false>(plan.rows, plan.waves);
    else fn = qbf16 ? pick<64, true>(plan.rows, plan.waves) : pick<64, false>(plan.rows, plan.waves);
    if (!fn) return fail(Q8K4V_EUNSUPPORTED, "attention: no block-MFMA kernel for this rows/waves combination");
    const hipError_t e = fn(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return Q8K4V_OK;
}

}  // namespace q8k4v
