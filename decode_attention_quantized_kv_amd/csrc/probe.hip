// Streaming probes: the HBM reference of the attention kernels' roofline.
//
// q8k4v_hbm_probe reads exactly the bytes a decode launch reads -- every
// (page, kv head) block of key codes, value codes, key scales and value
// scales of each sequence's pages, through the page table, with the decode
// plan's split of pages over workgroups, its XCD-aware work mapping and its
// 2-page tiles copied HBM -> LDS by global_load_lds_dwordx4 -- and computes
// nothing.  Its time is what the memory system gives this access pattern
// (random 3,232-byte page-head blocks at D = 128) at a given ring depth;
// the attention kernel cannot stream faster.  q8k4v_stream_probe does the
// same for one contiguous buffer (the sequential reference).
#include <algorithm>

#include "attn_common.h"
#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

template <int N>
Q8K4V_DEV void probe_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One wave's ring of STAGES 2-page tiles (the decode kernel's tile layout).
// With HPW > 1 a workgroup streams HPW kv heads of its pages (head group
// p.kh of work_item, whose p.H counts head groups; p.Hq is the cache's head
// count): wave w takes head w % HPW and every (WAVES / HPW)-th tile, so the
// HPW heads' blocks of a page -- contiguous in every pool -- are read by one
// compute unit together.
template <int D, int WAVES, int STAGES, int HPW>
__global__ __launch_bounds__(64 * WAVES) void paged_probe_kernel(const AttnParams p) {
    constexpr int TP = 2;
    constexpr int KB = 16 * D, VB = 8 * D, NG = D / 32;
    constexpr int KSB = 32, VSB = 32 * NG;
    constexpr int OFF_V = TP * KB, OFF_KS = OFF_V + TP * VB, OFF_VS = OFF_KS + TP * KSB;
    constexpr int STAGE = OFF_VS + TP * VSB;
    constexpr int KI = KB / 1024;
    constexpr int IPT = TP * (KI + 3);          // copy instructions per tile
    __shared__ __attribute__((aligned(16))) uint8_t s_ring[WAVES * STAGES * STAGE];
    static_assert(WAVES % HPW == 0, "whole waves per head");
    constexpr int TW = WAVES / HPW;             // waves per head
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WorkItem w;
    if (!work_item(p, w) || w.pbeg >= w.pend) return;
    const int head = w.kh * HPW + wave % HPW;
    const int tw = wave / HPW;                  // this wave's tile phase
    const int H = p.Hq;
    const int ntile_all = (w.pend - w.pbeg + TP - 1) / TP;
    const int nt = ntile_all > tw ? (ntile_all - tw + TW - 1) / TW : 0;
    int my_id = 0;
    {
        const int pg = w.pbeg + TP * (tw + TW * (lane >> 1)) + (lane & 1);
        if (lane < TP * nt) my_id = p.page_table[(size_t)w.b * p.max_pages + min(pg, w.pend - 1)];
    }
    asm volatile("" ::"v"(my_id));
    const uint32_t lds0 = lds_addr(s_ring + wave * STAGES * STAGE);
    auto issue = [&](int t, int slot) {
        const uint32_t base = lds0 + slot * STAGE;
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const int id = __builtin_amdgcn_readlane(my_id, TP * t + u);
            const size_t blk = (size_t)id * H + head;
#pragma unroll
            for (int c = 0; c < KI; ++c) lds_dma16(p.k_codes + blk * KB, 1024 * c + 16 * lane, base + u * KB + c * 1024);
            if (VB >= 1024 || lane < VB / 16) lds_dma16(p.v_codes + blk * VB, lane * 16, base + OFF_V + u * VB);
            if (lane < 2) lds_dma16(p.k_scales + blk * 16, lane * 16, base + OFF_KS + u * KSB);
            if (lane < 2 * NG) lds_dma16(p.v_scales + blk * 16 * NG, lane * 16, base + OFF_VS + u * VSB);
        }
    };
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nt) issue(s, s);
    for (int t = 0; t < nt; ++t) {
        if (t + STAGES - 1 < nt) issue(t + STAGES - 1, (t + STAGES - 1) % STAGES);
        const int after = min(STAGES - 1, nt - 1 - t);   // tiles issued after this one
        if (STAGES >= 4 && after >= 3) probe_wait<3 * IPT>();
        else if (STAGES >= 3 && after >= 2) probe_wait<2 * IPT>();
        else if (after >= 1) probe_wait<IPT>();
        else probe_wait<0>();
    }
}

// Contiguous stream: workgroup i reads chunk i of `bytes` (16-byte aligned)
// in 1 KiB wave copies, STAGES copies of 4 KiB per wave in flight.
template <int WAVES, int STAGES>
__global__ __launch_bounds__(64 * WAVES) void stream_probe_kernel(const uint8_t* buf, size_t bytes, size_t chunk) {
    constexpr int CP = 4;                       // 1 KiB copies per step
    __shared__ __attribute__((aligned(16))) uint8_t s_ring[WAVES * STAGES * CP * 1024];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t beg = (size_t)blockIdx.x * chunk;
    const size_t end = min(bytes, beg + chunk);
    if (beg >= end) return;
    const size_t step = (size_t)CP * 1024;
    const int nsteps = (int)((end - beg + step - 1) / step);
    const int nt = nsteps > wave ? (nsteps - wave + WAVES - 1) / WAVES : 0;
    const uint32_t lds0 = lds_addr(s_ring + wave * STAGES * CP * 1024);
    auto issue = [&](int t, int slot) {
        const size_t off = beg + (size_t)(wave + WAVES * t) * step;
#pragma unroll
        for (int c = 0; c < CP; ++c) {
            const size_t o = min(off + 1024 * c, end - 1024);   // the tail re-reads its last KiB
            lds_dma16(buf + o, 16 * lane, lds0 + (slot * CP + c) * 1024);
        }
    };
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nt) issue(s, s);
    for (int t = 0; t < nt; ++t) {
        if (t + STAGES - 1 < nt) issue(t + STAGES - 1, (t + STAGES - 1) % STAGES);
        const int after = min(STAGES - 1, nt - 1 - t);
        if (STAGES >= 4 && after >= 3) probe_wait<3 * CP>();
        else if (STAGES >= 3 && after >= 2) probe_wait<2 * CP>();
        else if (after >= 1) probe_wait<CP>();
        else probe_wait<0>();
    }
}

template <int D, int WAVES, int STAGES, int HPW>
hipError_t launch_paged_probe_t(const AttnParams& kp, hipStream_t stream) {
    hipLaunchKernelGGL((paged_probe_kernel<D, WAVES, STAGES, HPW>), dim3(work_blocks(kp)), dim3(64 * WAVES),
                       0, stream, kp);
    return hipGetLastError();
}

template <int D, int HPW>
hipError_t launch_paged_probe_h(const AttnParams& kp, int waves, int stages, hipStream_t stream) {
#define Q8K4V_PROBE(W_, S_) \
    if (waves == W_ && stages == S_) return launch_paged_probe_t<D, W_, S_, HPW>(kp, stream);
    if constexpr (HPW <= 4) {
        Q8K4V_PROBE(4, 2) Q8K4V_PROBE(4, 3) Q8K4V_PROBE(4, 4)
    }
    Q8K4V_PROBE(8, 2) Q8K4V_PROBE(8, 3)
#undef Q8K4V_PROBE
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_paged_probe(const AttnParams& kp, int waves, int stages, int hpw, hipStream_t stream) {
    switch (hpw) {
        case 1: return launch_paged_probe_h<D, 1>(kp, waves, stages, stream);
        case 2: return launch_paged_probe_h<D, 2>(kp, waves, stages, stream);
        case 4: return launch_paged_probe_h<D, 4>(kp, waves, stages, stream);
        default: return waves == 8 ? launch_paged_probe_h<D, 8>(kp, waves, stages, stream) : hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace q8k4v

using namespace q8k4v;

extern "C" int32_t q8k4v_hbm_probe(const q8k4v_cache* cache, int32_t n_seqs, const int32_t* seq_lens,
                                   int32_t max_seq_len, const int32_t* page_table, int32_t max_pages,
                                   int32_t waves_per_wg, int32_t stages, int32_t heads_per_wg,
                                   hipStream_t stream) {
    if (!cache || cache->codec != Q8K4V_CODEC_SYMMETRIC)
        return fail(Q8K4V_EINVAL, "q8k4v_hbm_probe: needs a symmetric-codec cache");
    if (!((waves_per_wg == 4 && (stages == 2 || stages == 3 || stages == 4)) ||
          (waves_per_wg == 8 && (stages == 2 || stages == 3))))
        return fail(Q8K4V_EINVAL, "q8k4v_hbm_probe: (waves, stages) must be (4, 2..4) or (8, 2..3)");
    const int hpw = heads_per_wg;
    if (!(hpw == 1 || hpw == 2 || hpw == 4 || (hpw == 8 && waves_per_wg == 8)) || cache->num_kv_heads % hpw)
        return fail(Q8K4V_EINVAL, "q8k4v_hbm_probe: heads_per_wg must be 1, 2, 4 or 8 (8 with 8 waves) and divide "
                                  "the kv heads");
    // the decode plan of the same launch shape: same splits, same mapping
    static const uint16_t fake_q = 0;
    static float fake_out = 0.0f;
    AttnArgs a{cache, &fake_q, Q8K4V_BF16, &fake_out, n_seqs, cache->num_kv_heads, 1, seq_lens, max_seq_len,
               page_table, max_pages, 1.0f};
    q8k4v_config cfg = default_config(1);
    cfg.variant = 4;
    cfg.waves_per_wg = waves_per_wg;
    cfg.stages = stages == 4 ? 3 : stages;   // the plan checks 2 or 3; the split does not depend on it
    Plan plan;
    int32_t rc = make_plan(a, &cfg, &plan);
    if (rc != Q8K4V_OK) return rc;
    // heads_per_wg > 1: the same number of workgroups, each over hpw heads
    // and 1/hpw of the pages (at least a tile per wave)
    int32_t split_pages = plan.split_pages, n_splits = plan.n_splits;
    if (hpw > 1) {
        const int32_t max_np = std::max(1, (max_seq_len + 15) / 16);
        const int32_t unit = 2 * (waves_per_wg / hpw);
        split_pages = std::max(unit, (plan.split_pages / hpw + unit - 1) / unit * unit);
        n_splits = (max_np + split_pages - 1) / split_pages;
        if (split_pages > 64 * (waves_per_wg / hpw)) return fail(Q8K4V_EUNSUPPORTED, "q8k4v_hbm_probe: too long");
    }
    AttnParams kp{};
    kp.k_codes = cache->k_codes;
    kp.k_scales = cache->k_scales;
    kp.v_codes = cache->v_codes;
    kp.v_scales = cache->v_scales;
    kp.seq_lens = seq_lens;
    kp.page_table = page_table;
    kp.H = cache->num_kv_heads / hpw;           // head groups (the work items' kh)
    kp.Hq = cache->num_kv_heads;                // the pools' head count
    kp.max_pages = max_pages;
    kp.n_seqs = n_seqs;
    kp.W = 1;
    kp.split_pages = split_pages;
    kp.n_splits = n_splits;
    kp.row_chunks = 1;
    const hipError_t e = cache->head_dim == 128 ? launch_paged_probe<128>(kp, waves_per_wg, stages, hpw, stream)
                                                : launch_paged_probe<64>(kp, waves_per_wg, stages, hpw, stream);
    if (e != hipSuccess) return hip_fail(e, "q8k4v_hbm_probe launch");
    return Q8K4V_OK;
}

extern "C" int32_t q8k4v_stream_probe(const void* buf, size_t bytes, int32_t waves_per_wg, int32_t stages,
                                      hipStream_t stream) {
    if (!buf || bytes < 1024 || (bytes & 15) || ((uintptr_t)buf & 15))
        return fail(Q8K4V_EINVAL, "q8k4v_stream_probe: buf must be 16-byte aligned, bytes >= 1024 and a multiple of 16");
    if (waves_per_wg != 4 && waves_per_wg != 8) return fail(Q8K4V_EINVAL, "q8k4v_stream_probe: waves_per_wg must be 4 or 8");
    if (stages < 2 || stages > 4) return fail(Q8K4V_EINVAL, "q8k4v_stream_probe: stages must be 2..4");
    const size_t wgs = (size_t)device_cu_count();
    const size_t chunk = ((bytes + wgs - 1) / wgs + 4095) / 4096 * 4096;
    const int blocks = (int)((bytes + chunk - 1) / chunk);
    const uint8_t* b = (const uint8_t*)buf;
    if (waves_per_wg == 4) {
        if (stages == 2) hipLaunchKernelGGL((stream_probe_kernel<4, 2>), dim3(blocks), dim3(256), 0, stream, b, bytes, chunk);
        else if (stages == 3) hipLaunchKernelGGL((stream_probe_kernel<4, 3>), dim3(blocks), dim3(256), 0, stream, b, bytes, chunk);
        else hipLaunchKernelGGL((stream_probe_kernel<4, 4>), dim3(blocks), dim3(256), 0, stream, b, bytes, chunk);
    } else {
        if (stages == 2) hipLaunchKernelGGL((stream_probe_kernel<8, 2>), dim3(blocks), dim3(512), 0, stream, b, bytes, chunk);
        else if (stages == 3) hipLaunchKernelGGL((stream_probe_kernel<8, 3>), dim3(blocks), dim3(512), 0, stream, b, bytes, chunk);
        else hipLaunchKernelGGL((stream_probe_kernel<8, 4>), dim3(blocks), dim3(512), 0, stream, b, bytes, chunk);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "q8k4v_stream_probe launch");
    return Q8K4V_OK;
}
