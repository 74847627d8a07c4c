// Pieces shared by the attention kernels (the replicated-row and row-block
// tile-ring kernels of attn_paged.hip) and the combine kernels: launch parameters,
// the XCD-aware work-item mapping, the merge of a workgroup's waves, the
// split partials and the log-sum-exp combine of the splits (by the
// last-arriving workgroup or by a separate kernel, and the two-source combine
// of the shared-prefix cascade).
#pragma once

#include "q8k4v_device.h"

namespace q8k4v {

struct AttnParams {
    const int8_t* __restrict__ k_codes;
    const uint16_t* __restrict__ k_scales;
    const uint8_t* __restrict__ v_codes;
    const uint16_t* __restrict__ v_scales;
    const void* __restrict__ q;
    float* __restrict__ out;
    float* __restrict__ partials;      // [n_seqs][H][n_splits][R][D + 4]
    uint32_t* __restrict__ counters;   // [n_seqs][H] arrivals (fused combine)
    const int32_t* __restrict__ seq_lens;
    const int32_t* __restrict__ page_table;
    int32_t H, max_pages, n_seqs, Hq, G, W, R;
    int32_t split_pages, n_splits, row_chunks;
    float scale_log2;                  // softmax scale * log2(e)
    int32_t direct;                    // one split: write normalised output
    int32_t fused;                     // last workgroup merges the splits
    // Page ranges of the shared-prefix cascade (0 for a plain launch):
    // page_lo is the first logical page of every split range; page_cap > 0
    // makes every sequence exactly page_cap pages long with no causal edge
    // inside them (the prefix pass over pages all sessions share).
    int32_t page_lo, page_cap;
    int32_t cascade;                   // pass of a cascade: partials only
    // prefix-pass partials, read by the cascade combine:
    // [H][pre_splits][pre_R][D + 4], row b * G + g of session b; the first
    // pre_eff splits hold pages
    const float* __restrict__ pre_partials;
    int32_t pre_splits, pre_eff, pre_R;
    // affine codec: per-token key zero points (z XOR 0x80) [P][H][16] and
    // per-(token, group) value zero points [P][H][16][D/32]
    int32_t affine;
    const int8_t* __restrict__ k_zeros;
    const uint8_t* __restrict__ v_zeros;
    // decode that appends the step's token itself: K and V rows [n_seqs][H][D]
    // of the token at position seq_lens[b] - 1 (bf16 bit patterns or fp32)
    const void* __restrict__ k_new;
    const void* __restrict__ v_new;
    int32_t new_bf16;
};

constexpr float kNegInf = -__builtin_inff();

// Online softmax reference (log2 units): a row's reference moves only when a
// score passes it and is then set this far above the new maximum.  Every
// p = 2^(s - ref) stays <= 1 (so p times an fp16 value scale stays finite in
// fp16), the largest p of a row is >= 2^-kRefHeadroom, and the accumulators
// are rescaled only when a score passes the reference rather than on every
// new maximum.  Partial results carry the reference as their m, which is all
// the log-sum-exp merge needs.
constexpr float kRefHeadroom = 2.0f;

template <int D>
constexpr int partial_stride() { return D + 4; }   // m, l, pad, pad, o[D]

struct WorkItem {
    int b, kh, split, rchunk, L, npages, pbeg, pend;
};

// Work items are (sequence, split, kv head, row chunk); the dispatcher hands
// workgroup i to XCD i % 8.  The (sequence, split) pairs are taken split by
// split -- every sequence's split 0, then every split 1, ... -- with the
// sequences of split round s rotated by s, and dealt round robin over the 8
// XCDs; the kv heads and row chunks of a pair (which share the lines of the
// key-scale pool) stay together on its XCD.  So pair (s, b) sits at slot
// q = s n + (b + s) mod n: a sequence's consecutive splits visit different
// XCDs, every XCD gets an even share of the pairs with no slot left empty
// but in the last round, and the workgroups that hold pages come first in
// dispatch order -- in a batch of ragged lengths the empty splits of the
// short sequences are the late ones -- so the workgroups with pages spread
// over the CUs instead of pairing up on some of them.
Q8K4V_DEV bool work_item(const AttnParams& p, WorkItem& w, int bid) {
    const int C = p.H * p.row_chunks;          // items per (sequence, split)
    const int n = p.n_seqs;
    const int x = bid & 7, j = bid >> 3;
    const int inner = j % C;
    const int q = 8 * (j / C) + x;             // pair slot, split-major
    if (q >= n * p.n_splits) return false;
    w.split = q / n;
    w.b = (q % n - w.split % n + n) % n;
    w.rchunk = inner % p.row_chunks;
    w.kh = inner / p.row_chunks;
    if (p.page_cap > 0) {
        w.npages = p.page_cap;
        w.L = 16 * p.page_cap + p.W - 1;       // row j's causal limit 16 page_cap + j: no edge inside
    } else {
        w.L = p.seq_lens[w.b];
        w.npages = (w.L + 15) >> 4;
    }
    w.pbeg = p.page_lo + w.split * p.split_pages;
    w.pend = min(w.npages, w.pbeg + p.split_pages);
    return true;
}
Q8K4V_DEV bool work_item(const AttnParams& p, WorkItem& w) { return work_item(p, w, (int)blockIdx.x); }

// Workgroups of a launch under that mapping: 8 XCDs x rounds of pair slots x items per pair.
inline int work_blocks(const AttnParams& p) {
    const int slots = p.n_seqs * p.n_splits;
    return 8 * ((slots + 7) / 8) * p.H * p.row_chunks;
}

Q8K4V_DEV size_t out_index(const AttnParams& p, int b, int kh, int r, int D) {
    const int j = r / p.G, g = r % p.G;
    return (((size_t)b * p.W + j) * p.Hq + kh * p.G + g) * D;
}

// Empty split of a single-split launch: the sequence has no tokens, its
// output rows are zero.
template <int D>
Q8K4V_DEV void write_zero_rows(const AttnParams& p, const WorkItem& w, int r0, int nrows) {
    for (int e = threadIdx.x; e < nrows * D; e += blockDim.x) {
        const int r = r0 + e / D;
        if (r < p.R) p.out[out_index(p, w.b, w.kh, r, D) + e % D] = 0.0f;
    }
}

// Log-sum-exp merge of the n_eff split partials of (b, kh) for rows
// [r0, r0 + NR), by the threads of the last workgroup to finish.  The split
// records were written by workgroups on any XCD and released by their
// arrivals (fused_tail); an agent-scope acquire (which drops this XCD's stale
// L2 lines) lets plain, vectorised loads see them.  Thread t takes (row, float4 column) pairs and
// a split group, loads the records of its splits in batches of CH with all
// loads of a batch in flight, merges them online, and the split groups are
// merged through LDS.  Every load of a batch is unconditional (split index
// clamped, the extra records masked afterwards): a load under a branch gets
// its own wait, one memory round trip per split.
constexpr int kCombineMaxSplits = 1024;

template <int D, int NR>
Q8K4V_DEV void combine_splits(const AttnParams& p, int b, int kh, int r0, int n_eff, void* scratch,
                              int scratch_bytes) {
    constexpr int NQ = D / 4;
    constexpr int NP = NR * NQ;               // (row, column) pairs
    constexpr int CH = 16;
    constexpr int REC = 24;                   // LDS bytes per pair and group: m, l, o
    const int nt = blockDim.x;
    const int sg_n = max(1, min(nt / NP, scratch_bytes / (REC * NP)));   // split groups
    const int chunk = min(NP, max(1, scratch_bytes / (REC * sg_n)));    // pairs per pass
    float* s_m = (float*)scratch;             // [sg_n][chunk]
    float* s_l = s_m + sg_n * chunk;
    f32x4* s_o = (f32x4*)(s_l + sg_n * chunk + ((4 - (2 * sg_n * chunk) % 4) % 4));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const size_t rs = (size_t)p.R * partial_stride<D>();
    const float* base = p.partials + ((size_t)b * p.H + kh) * p.n_splits * rs;
    for (int pc0 = 0; pc0 < NP; pc0 += chunk) {
        const int npc = min(chunk, NP - pc0);
        for (int t = threadIdx.x; t < npc * sg_n; t += nt) {
            const int pl = t % npc, sg = t / npc;
            const int pr = pc0 + pl;
            const int rl = pr / NQ, qc = pr % NQ;
            const int r = min(r0 + rl, p.R - 1);
            const float* rbase = base + (size_t)r * partial_stride<D>();
            float M = kNegInf, Ls = 0.0f;
            f32x4 O = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int s0 = sg; s0 < n_eff; s0 += sg_n * CH) {
                float m[CH], l[CH];
                f32x4 o[CH];
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const int sp = s0 + c * sg_n;
                    const float* rec = rbase + (size_t)min(sp, n_eff - 1) * rs;
                    const float2 ml = *(const float2*)rec;
                    const f32x4 ov = *((const f32x4*)(rec + 4) + qc);
                    const bool in = sp < n_eff;
                    m[c] = in ? ml.x : kNegInf;
                    l[c] = in ? ml.y : 0.0f;
                    o[c] = in ? ov : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
                float Mn = M;
#pragma unroll
                for (int c = 0; c < CH; ++c) Mn = fmaxf(Mn, m[c]);
                // branch-free (a branch here lets the compiler sink the batch's
                // loads below it): with every maximum -inf, ref 0 gives weights 0
                const float ref = (Mn == kNegInf) ? 0.0f : Mn;
                const float a = exp2_fast(M - ref);        // M = -inf gives 0
                O *= a;
                Ls *= a;
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const float wgt = exp2_fast(m[c] - ref);
                    O += o[c] * wgt;
                    Ls += l[c] * wgt;
                }
                M = Mn;
            }
            s_m[sg * chunk + pl] = M;
            s_l[sg * chunk + pl] = Ls;
            s_o[sg * chunk + pl] = O;
        }
        __syncthreads();
        for (int pl = threadIdx.x; pl < npc; pl += nt) {
            const int pr = pc0 + pl;
            const int rl = pr / NQ, qc = pr % NQ;
            const int r = r0 + rl;
            if (r >= p.R) continue;
            float Mg = kNegInf;
            for (int g = 0; g < sg_n; ++g) Mg = fmaxf(Mg, s_m[g * chunk + pl]);
            const float ref = (Mg == kNegInf) ? 0.0f : Mg;
            f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
            float Lt = 0.0f;
            for (int g = 0; g < sg_n; ++g) {
                const float wgt = exp2_fast(s_m[g * chunk + pl] - ref);
                sum += s_o[g * chunk + pl] * wgt;
                Lt += s_l[g * chunk + pl] * wgt;
            }
            const float inv = (Lt > 0.0f) ? 1.0f / Lt : 0.0f;
            *((f32x4*)(p.out + out_index(p, b, kh, r, D)) + qc) = sum * inv;
        }
        __syncthreads();
    }
}

// Write one merged (row, dimension) element of a workgroup: the normalised
// output when there is a single split, else the split partial.
template <int D>
Q8K4V_DEV void emit_element(const AttnParams& p, const WorkItem& w, int r, int d, float M, float Ls, float O) {
    if (p.direct) {
        p.out[out_index(p, w.b, w.kh, r, D) + d] = (Ls > 0.0f) ? O / Ls : 0.0f;
    } else {
        const size_t rs = (size_t)p.R * partial_stride<D>();
        float* rec = p.partials + ((size_t)w.b * p.H + w.kh) * p.n_splits * rs + w.split * rs +
                     (size_t)r * partial_stride<D>();
        if (d == 0) *(float2*)rec = float2{M, Ls};
        rec[4 + d] = O;
    }
}

// With the fused combine, the last workgroup of (b, kh, row chunk) to finish
// merges all splits.  Called by every thread after its record stores.  The
// records cross XCDs (each XCD has its own L2): every wave waits for its
// stores, the barrier orders them before thread 0's arrival, and the
// arrival is an agent-scope acquire-release read-modify-write -- its release
// writes this XCD's dirty L2 lines back, its acquire (and the merging
// threads' acquire fence) drops stale lines -- so the merge's plain loads
// see every record.  The last arrival resets the counter to zero: between
// completed calls every counter of the workspace header is zero.
template <int D, int RW>
Q8K4V_DEV void fused_tail(const AttnParams& p, const WorkItem& w, int r0, void* scratch, int scratch_bytes) {
    if (p.direct || !p.fused) return;
    __shared__ int s_last;
    const int n_eff = (max(0, w.npages - p.page_lo) + p.split_pages - 1) / p.split_pages;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t* ctr = p.counters + ((size_t)w.b * p.H + w.kh) * p.row_chunks + w.rchunk;
        const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old + 1 == (uint32_t)n_eff);
        if (s_last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    combine_splits<D, RW>(p, w.b, w.kh, r0, n_eff, scratch, scratch_bytes);
}

// Emit the merged rows [r0, r0 + RW) of a workgroup, four dimensions per
// thread: s_M / s_L hold each row's max and sum, s_o [RW][SO_STRIDE] its unnormalised
// output (already on the row's reference).  One split: the normalised output.
// Several: the split record (m, l, o); a separate combine kernel reads it
// after the kernel boundary, the in-launch merge after fused_tail's
// acquire-release arrival.
template <int D, int RW, int SO_STRIDE = D>
Q8K4V_DEV void emit_rows(const AttnParams& p, const WorkItem& w, int r0, const float* s_M, const float* s_L,
                         const float* s_o) {
    constexpr int NQ = D / 4;
    const size_t rs = (size_t)p.R * partial_stride<D>();
    float* split_base = p.partials + ((size_t)w.b * p.H + w.kh) * p.n_splits * rs + w.split * rs;
    for (int e = threadIdx.x; e < RW * NQ; e += blockDim.x) {
        const int rl = e / NQ, qc = e % NQ;
        const int r = r0 + rl;
        if (r >= p.R) continue;
        const f32x4 O = *((const f32x4*)(s_o + rl * SO_STRIDE) + qc);
        const float Ls = s_L[rl];
        if (p.direct) {
            const float inv = (Ls > 0.0f) ? 1.0f / Ls : 0.0f;
            *((f32x4*)(p.out + out_index(p, w.b, w.kh, r, D)) + qc) = O * inv;
            continue;
        }
        float* rec = split_base + (size_t)r * partial_stride<D>();
        if (qc == 0) *(float2*)rec = float2{s_M[rl], Ls};
        *((f32x4*)(rec + 4) + qc) = O;
    }
}

// Merge the waves of a workgroup (each wave left its running max m, sum l
// and unnormalised output o in LDS), then emit the rows.
// `scratch` (scratch_bytes of LDS, 16-byte aligned, s_o may lie in it) is
// free for the fused combine once the rows are emitted.
template <int D, int RW, int WAVES>
Q8K4V_DEV void finish_workgroup(const AttnParams& p, const WorkItem& w, int r0,
                                const float (*s_ml)[RW][2], float* s_o /* [WAVES][RW][D] */,
                                void* scratch, int scratch_bytes) {
    __shared__ float s_M[RW], s_L[RW], s_f[WAVES][RW];
    __syncthreads();
    for (int rl = threadIdx.x; rl < RW; rl += 64 * WAVES) {
        float M = kNegInf;
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) M = fmaxf(M, s_ml[wv][rl][0]);
        const float ref = (M == kNegInf) ? 0.0f : M;
        float Ls = 0.0f;
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) {
            const float f = exp2_fast(s_ml[wv][rl][0] - ref);
            s_f[wv][rl] = f;
            Ls += s_ml[wv][rl][1] * f;
        }
        s_M[rl] = M;
        s_L[rl] = Ls;
    }
    __syncthreads();
    // waves' outputs on the common reference, summed into wave 0's slot
    constexpr int NQ = D / 4;
    for (int e = threadIdx.x; e < RW * NQ; e += 64 * WAVES) {
        const int rl = e / NQ;
        f32x4 O = *((const f32x4*)s_o + e) * s_f[0][rl];
#pragma unroll
        for (int wv = 1; wv < WAVES; ++wv) O += *((const f32x4*)(s_o + wv * RW * D) + e) * s_f[wv][rl];
        *((f32x4*)s_o + e) = O;
    }
    __syncthreads();
    emit_rows<D, RW>(p, w, r0, s_M, s_L, s_o);
    fused_tail<D, RW>(p, w, r0, scratch, scratch_bytes);
}

// Separate combine kernel: one 256-thread workgroup per (b, kh, row).
// Thread (split group sg, float4 column qc) loads the records of splits sg,
// sg + SG, ... in chunks of 8 -- maxima, sums and its output column, all
// loads of a chunk issued together -- and merges them online; the SG group
// states are then merged through LDS.  The partials come from the previous
// kernel on the stream, so plain loads see them.  Records are loaded for
// every split of the launch (all in bounds) and those past the sequence's
// last split are masked afterwards, so the loads do not wait for seq_lens.
// The split index of a batch's loads is clamped rather than branched on, so
// the loads of a batch go out together.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const AttnParams p) {
    constexpr int NQ = D / 4;                 // float4 columns of a row
    constexpr int SG = 256 / NQ;              // split groups
    constexpr int CH = 8;                     // splits per load batch
    __shared__ float s_m[SG], s_l[SG];
    __shared__ f32x4 s_o[SG][NQ];
    const int t = threadIdx.x;
    const int qc = t % NQ, sg = t / NQ;
    const int r = blockIdx.x % p.R;
    const int kh = (blockIdx.x / p.R) % p.H;
    const int b = blockIdx.x / (p.R * p.H);
    // The sequence length comes in through a vector (buffer) load and is first
    // used after a batch's record loads are out: a scalar load of it would be
    // waited for before them, one more memory round trip.  Buffer resource
    // word 3 of gfx9-family targets: 32-bit data format.
    const int L = (int)__builtin_amdgcn_raw_buffer_load_b32(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(p.seq_lens + b), 0, 4, 0x00020000), 0, 0, 0);
    const size_t rs = (size_t)p.R * partial_stride<D>();
    const float* base = p.partials + ((size_t)b * p.H + kh) * p.n_splits * rs + (size_t)r * partial_stride<D>();
    float M = kNegInf, Ls = 0.0f;
    f32x4 O = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = sg; s0 < p.n_splits; s0 += SG * CH) {
        float m[CH], l[CH];
        f32x4 o[CH];
        float2 ml[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float* rec = base + (size_t)min(s0 + c * SG, p.n_splits - 1) * rs;
            ml[c] = *(const float2*)rec;
            o[c] = *((const f32x4*)(rec + 4) + qc);
        }
        int Lv = L;
        asm volatile("" : "+v"(Lv));   // keeps the length's wait below the loads
        const int npages = (Lv + 15) >> 4;
        const int n_eff = min(p.n_splits, (max(0, npages - p.page_lo) + p.split_pages - 1) / p.split_pages);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = s0 + c * SG < n_eff;     // selects, not a branch the loads could sink into
            m[c] = in ? ml[c].x : kNegInf;
            l[c] = in ? ml[c].y : 0.0f;
            if (!in) o[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        float Mn = M;
#pragma unroll
        for (int c = 0; c < CH; ++c) Mn = fmaxf(Mn, m[c]);
        // branch-free (a branch here lets the compiler sink the batch's
        // loads below it): with every maximum -inf, ref 0 gives weights 0
        const float ref = (Mn == kNegInf) ? 0.0f : Mn;
        const float a = exp2_fast(M - ref);        // M = -inf gives 0
        O *= a;
        Ls *= a;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float wgt = exp2_fast(m[c] - ref);
            O += o[c] * wgt;
            Ls += l[c] * wgt;
        }
        M = Mn;
    }
    if (qc == 0) {
        s_m[sg] = M;
        s_l[sg] = Ls;
    }
    s_o[sg][qc] = O;
    __syncthreads();
    if (t < NQ) {
        float Mg = kNegInf;
#pragma unroll
        for (int g = 0; g < SG; ++g) Mg = fmaxf(Mg, s_m[g]);
        const float ref = (Mg == kNegInf) ? 0.0f : Mg;
        f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
        float Lt = 0.0f;
#pragma unroll
        for (int g = 0; g < SG; ++g) {
            const float wgt = exp2_fast(s_m[g] - ref);
            sum += s_o[g][t] * wgt;
            Lt += s_l[g] * wgt;
        }
        const float inv = (Lt > 0.0f) ? 1.0f / Lt : 0.0f;
        f32x4* dst = (f32x4*)(p.out + out_index(p, b, kh, r, D)) + t;
        *dst = sum * inv;
    }
}

// Combine of the shared-prefix cascade: one 256-thread workgroup per
// (b, kh, g) of a decode launch.  Row (b, g) has two record sets: the prefix
// pass's first pre_eff records (row b * G + g of each [pre_R] block) and the
// suffix pass's splits of sequence b, of which those past its last page are
// masked.  Both sets are walked as one list of pre_eff + n_splits records,
// merged online as in combine_kernel.
template <int D>
__global__ __launch_bounds__(256) void combine_cascade_kernel(const AttnParams p) {
    constexpr int NQ = D / 4;
    constexpr int SG = 256 / NQ;
    constexpr int CH = 8;
    constexpr int RS = partial_stride<D>();
    __shared__ float s_m[SG], s_l[SG];
    __shared__ f32x4 s_o[SG][NQ];
    const int t = threadIdx.x;
    const int qc = t % NQ, sg = t / NQ;
    const int g = blockIdx.x % p.R;
    const int kh = (blockIdx.x / p.R) % p.H;
    const int b = blockIdx.x / (p.R * p.H);
    // the sequence length as in combine_kernel: a vector load, waited for
    // after a batch's record loads
    const int L = (int)__builtin_amdgcn_raw_buffer_load_b32(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(p.seq_lens + b), 0, 4, 0x00020000), 0, 0, 0);
    const float* pre = p.pre_partials + ((size_t)kh * p.pre_splits * p.pre_R + (size_t)b * p.R + g) * RS;
    const size_t pre_step = (size_t)p.pre_R * RS;
    const float* suf = p.partials + (((size_t)b * p.H + kh) * p.n_splits * p.R + g) * RS;
    const size_t suf_step = (size_t)p.R * RS;
    const int total = p.pre_eff + p.n_splits;
    float M = kNegInf, Ls = 0.0f;
    f32x4 O = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int u0 = sg; u0 < total; u0 += SG * CH) {
        float m[CH], l[CH];
        f32x4 o[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int u = min(u0 + c * SG, total - 1);    // clamped: no branch around the loads
            const float* rec = u < p.pre_eff ? pre + (size_t)u * pre_step : suf + (size_t)(u - p.pre_eff) * suf_step;
            const float2 ml = *(const float2*)rec;
            m[c] = ml.x;
            l[c] = ml.y;
            o[c] = *((const f32x4*)(rec + 4) + qc);
        }
        int Lv = L;
        asm volatile("" : "+v"(Lv));   // keeps the length's wait below the loads
        const int npages = (Lv + 15) >> 4;
        const int n_suf = min(p.n_splits, (max(0, npages - p.page_lo) + p.split_pages - 1) / p.split_pages);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int u = u0 + c * SG;
            const bool in = u < total && (u < p.pre_eff || u - p.pre_eff < n_suf);   // selects
            m[c] = in ? m[c] : kNegInf;
            l[c] = in ? l[c] : 0.0f;
            if (!in) o[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        float Mn = M;
#pragma unroll
        for (int c = 0; c < CH; ++c) Mn = fmaxf(Mn, m[c]);
        // branch-free (a branch here lets the compiler sink the batch's
        // loads below it): with every maximum -inf, ref 0 gives weights 0
        const float ref = (Mn == kNegInf) ? 0.0f : Mn;
        const float a = exp2_fast(M - ref);        // M = -inf gives 0
        O *= a;
        Ls *= a;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float wgt = exp2_fast(m[c] - ref);
            O += o[c] * wgt;
            Ls += l[c] * wgt;
        }
        M = Mn;
    }
    if (qc == 0) {
        s_m[sg] = M;
        s_l[sg] = Ls;
    }
    s_o[sg][qc] = O;
    __syncthreads();
    if (t < NQ) {
        float Mg = kNegInf;
#pragma unroll
        for (int k = 0; k < SG; ++k) Mg = fmaxf(Mg, s_m[k]);
        const float ref = (Mg == kNegInf) ? 0.0f : Mg;
        f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
        float Lt = 0.0f;
#pragma unroll
        for (int k = 0; k < SG; ++k) {
            const float wgt = exp2_fast(s_m[k] - ref);
            sum += s_o[k][t] * wgt;
            Lt += s_l[k] * wgt;
        }
        const float inv = (Lt > 0.0f) ? 1.0f / Lt : 0.0f;
        *((f32x4*)(p.out + out_index(p, b, kh, g, D)) + t) = sum * inv;
    }
}

}  // namespace q8k4v
