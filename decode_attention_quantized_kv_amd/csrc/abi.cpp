// C ABI of the k8v4 attention library: argument validation, launch planning
// and dispatch.  See include/q8k4v.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "attn_common.h"
#include "q8k4v_internal.h"

#ifndef Q8K4V_BUILD_ID
#define Q8K4V_BUILD_ID "dev"
#endif

namespace q8k4v {

int32_t launch_dec2(const AttnParams& kp, const Plan& plan, int head_dim, bool qbf16, hipStream_t stream);
int32_t launch_rows(const AttnParams& kp, const Plan& plan, int head_dim, bool qbf16, hipStream_t stream);
int32_t launch_combine(const AttnParams& kp, int head_dim, int rows_per_wg, hipStream_t stream);
int32_t launch_combine_cascade(const AttnParams& kp, int head_dim, hipStream_t stream);
bool cascade_fusable(const Plan& pre, const Plan& suf);
bool decode_append_fusable(const Plan& plan, const q8k4v_cache& c);
int32_t launch_dec2_append(const AttnParams& kp, const Plan& plan, int head_dim, bool qbf16, hipStream_t stream);
int32_t launch_cascade_fused(const AttnParams& pre, const AttnParams& suf, int head_dim, bool qbf16, int rows,
                             hipStream_t stream);

namespace {
thread_local std::string g_last_error;

struct TunedEntry {          // keyed by device and shape; n_draft 1 is the decode unit
    int32_t device, n_draft, hq, hkv, d;
    q8k4v_config cfg;
};
std::mutex g_tuned_mu;
std::vector<TunedEntry> g_tuned;

bool valid_cache(const q8k4v_cache* c, std::string* why) {
    if (!c) { *why = "cache is NULL"; return false; }
    if (c->head_dim != 64 && c->head_dim != 128) { *why = "head_dim must be 64 or 128"; return false; }
    if (c->page_size != Q8K4V_PAGE_SIZE) { *why = "page_size must be 16"; return false; }
    if (c->num_kv_heads < 1 || c->num_pages < 1) { *why = "num_kv_heads and num_pages must be >= 1"; return false; }
    if (!c->k_codes || !c->k_scales || !c->v_codes || !c->v_scales) { *why = "a cache pool pointer is NULL"; return false; }
    if (c->codec != Q8K4V_CODEC_SYMMETRIC && c->codec != Q8K4V_CODEC_AFFINE) { *why = "codec must be 0 (symmetric) or 1 (affine)"; return false; }
    if (c->codec == Q8K4V_CODEC_AFFINE && (!c->k_zeros || !c->v_zeros)) { *why = "an affine cache needs k_zeros and v_zeros"; return false; }
    return true;
}

int32_t round_up(int32_t x, int32_t m) { return (x + m - 1) / m * m; }
}  // namespace

int32_t fail(int32_t code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

int32_t hip_fail(hipError_t e, const char* what) {
    return fail(Q8K4V_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

int32_t device_cu_count() {
    // compute units of the current device, looked up once per device
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

namespace {
bool dec2_rows(int32_t rows) { return rows == 1 || rows == 2 || rows == 4 || rows == 8 || rows == 16; }

// launch shape defaults per kernel; the row-block kernel takes 8 waves once
// two row blocks share the page stream (more than 16 rows per kv head)
void kernel_defaults(int32_t kernel, int32_t rows, q8k4v_config* c) {
    c->wgs_per_cu = 1;
    c->stages = 2;
    c->tile_pages = 2;
    c->waves_per_wg = (kernel == kRows && rows > 16) ? 8 : 4;
}

int32_t auto_kernel(int32_t rows) { return dec2_rows(rows) ? kDec2 : kRows; }
}  // namespace

q8k4v_config default_config(int32_t rows) {
    q8k4v_config c;
    std::memset(&c, 0, sizeof(c));
    kernel_defaults(auto_kernel(rows), rows, &c);
    c.split_pages = 0;
    c.fused_combine = 0;
    c.qualified = 0;
    c.variant = 0;
    return c;
}

static int current_device() {
    int dev = 0;
    return hipGetDevice(&dev) == hipSuccess ? dev : 0;
}

bool tuned_lookup(int32_t n_draft, int32_t hq, int32_t hkv, int32_t d, q8k4v_config* cfg) {
    const int dev = current_device();
    std::lock_guard<std::mutex> lk(g_tuned_mu);
    for (const auto& e : g_tuned)
        if (e.device == dev && e.n_draft == n_draft && e.hq == hq && e.hkv == hkv && e.d == d) {
            *cfg = e.cfg;
            return true;
        }
    return false;
}

void tuned_install(int32_t n_draft, int32_t hq, int32_t hkv, int32_t d, const q8k4v_config& cfg) {
    const int dev = current_device();
    std::lock_guard<std::mutex> lk(g_tuned_mu);
    for (auto& e : g_tuned)
        if (e.device == dev && e.n_draft == n_draft && e.hq == hq && e.hkv == hkv && e.d == d) {
            e.cfg = cfg;
            return;
        }
    g_tuned.push_back({dev, n_draft, hq, hkv, d, cfg});
}

int32_t make_plan(const AttnArgs& a, const q8k4v_config* cfg_in, Plan* plan) {
    std::string why;
    if (!valid_cache(a.cache, &why)) return fail(Q8K4V_EINVAL, "attention: " + why);
    const int32_t H = a.cache->num_kv_heads;
    const int32_t D = a.cache->head_dim;
    if (a.n_seqs < 1) return fail(Q8K4V_EINVAL, "attention: n_seqs must be >= 1");
    if (a.num_q_heads < 1 || a.num_q_heads % H) return fail(Q8K4V_EINVAL, "attention: num_q_heads must be a positive multiple of num_kv_heads");
    const int32_t G = a.num_q_heads / H;
    if (G != 1 && G != 2 && G != 4 && G != 8) return fail(Q8K4V_EUNSUPPORTED, "attention: group size num_q_heads/num_kv_heads must be 1, 2, 4 or 8");
    if (a.n_draft < 1 || a.n_draft > Q8K4V_MAX_CHUNK) return fail(Q8K4V_EINVAL, "attention: n_draft must be in 1..1024");
    if (a.max_seq_len < 0) return fail(Q8K4V_EINVAL, "attention: max_seq_len must be >= 0");
    if (a.max_pages < 1 || (int64_t)a.max_pages * Q8K4V_PAGE_SIZE < a.max_seq_len)
        return fail(Q8K4V_EINVAL, "attention: max_pages * 16 must cover max_seq_len");
    if (a.q_dtype != Q8K4V_F32 && a.q_dtype != Q8K4V_BF16) return fail(Q8K4V_EINVAL, "attention: q_dtype must be F32 or BF16");
    if (!a.q || !a.out || !a.seq_lens || !a.page_table) return fail(Q8K4V_EINVAL, "attention: NULL q/out/seq_lens/page_table");
    (void)D;

    const int32_t rows = a.n_draft * G;
    q8k4v_config cfg;
    if (cfg_in) cfg = *cfg_in;
    else if (!tuned_lookup(a.n_draft, a.num_q_heads, H, D, &cfg)) cfg = default_config(rows);

    int32_t kernel;
    switch (cfg.variant) {
        case 0: kernel = auto_kernel(rows); break;
        case 4:
            if (!dec2_rows(rows)) return fail(Q8K4V_EINVAL, "attention: variant 4 needs 1, 2, 4, 8 or 16 rows per kv head");
            kernel = kDec2;
            break;
        case 5: kernel = kRows; break;
        default: return fail(Q8K4V_EINVAL, "attention: variant must be 0 (automatic), 4 or 5");
    }
    q8k4v_config kd;
    std::memset(&kd, 0, sizeof(kd));
    kernel_defaults(kernel, rows, &kd);
    if (cfg.wgs_per_cu <= 0) cfg.wgs_per_cu = kd.wgs_per_cu;
    if (cfg.stages <= 0) cfg.stages = kd.stages;
    if (cfg.waves_per_wg <= 0) cfg.waves_per_wg = kd.waves_per_wg;
    if (cfg.waves_per_wg != 2 && cfg.waves_per_wg != 4 && cfg.waves_per_wg != 8)
        return fail(Q8K4V_EINVAL, "attention: waves_per_wg must be 2, 4 or 8");
    if (cfg.stages != 2 && cfg.stages != 3) return fail(Q8K4V_EINVAL, "attention: stages must be 2 or 3");
    if (cfg.tile_pages != 0 && cfg.tile_pages != 2)
        return fail(Q8K4V_EINVAL, "attention: tile_pages must be 0 or 2 (both kernels stage 2-page tiles)");
    cfg.tile_pages = 2;

    plan->rows = rows;
    plan->kernel = kernel;
    plan->tile_pages = cfg.tile_pages;
    plan->waves = cfg.waves_per_wg;
    plan->stages = cfg.stages;
    plan->rows_per_wg = kernel == kRows ? (rows > 16 ? 32 : 16) : rows;
    plan->row_chunks = (rows + plan->rows_per_wg - 1) / plan->rows_per_wg;
    const int32_t max_np = std::max(1, (a.max_seq_len + Q8K4V_PAGE_SIZE - 1) / Q8K4V_PAGE_SIZE);
    const int32_t unit = cfg.tile_pages * cfg.waves_per_wg;      // pages per workgroup step
    int32_t sp;
    if (cfg.split_pages > 0) {
        sp = round_up(cfg.split_pages, unit);
    } else if (max_np <= unit * cfg.stages) {
        // one workgroup has every page of the sequence in flight at once (each
        // wave's ring holds its share): splitting cannot shorten that one
        // round trip and would add the merge
        sp = round_up(max_np, unit);
    } else {
        const int64_t target = (int64_t)cfg.wgs_per_cu * device_cu_count();
        const int64_t per = (int64_t)a.n_seqs * H * plan->row_chunks;
        const int64_t splits = std::max<int64_t>(1, (target + per - 1) / per);
        sp = round_up((int32_t)((max_np + splits - 1) / splits), unit);
    }
    sp = std::max(sp, unit);
    if (sp > 64 * cfg.waves_per_wg) {
        // a wave's page ids sit one per lane: at most 64 pages per wave.  With
        // the automatic split of a one-chunk query block (decode, small
        // verify), the extra splits this forces are made even: a multiple of
        // 8 (splits are dealt round robin over the 8 XCDs, so every XCD gets
        // the same pages), then at least the next whole number of workgroups
        // per CU (not just over one).  Blocks of many row chunks (prefill)
        // keep the capped split: their workgroups are many already, and
        // doubling them costs more in per-workgroup set-up than the uneven
        // last split (measured)
        const int32_t cap = 64 * cfg.waves_per_wg;
        if (cfg.split_pages > 0 || plan->row_chunks > 1) {
            sp = cap;
        } else {
            const int64_t cus = device_cu_count();
            const int64_t per = (int64_t)a.n_seqs * H * plan->row_chunks;
            int64_t splits = round_up((int32_t)((max_np + cap - 1) / cap), 8);   // splits at the cap, even over XCDs
            const int64_t k = (splits * per + cus - 1) / cus;                       // workgroups per CU
            splits = round_up((int32_t)std::max<int64_t>(splits, (k * cus + per - 1) / per), 8);
            sp = round_up((int32_t)((max_np + splits - 1) / splits), unit);   // <= cap: unit divides cap
        }
    }
    plan->split_pages = sp;
    plan->n_splits = (max_np + sp - 1) / sp;
    if (plan->n_splits > kCombineMaxSplits) {   // the combine holds one weight per split in LDS
        sp = round_up((max_np + kCombineMaxSplits - 1) / kCombineMaxSplits, unit);
        plan->split_pages = sp;
        plan->n_splits = (max_np + sp - 1) / sp;
    }
    if (plan->split_pages > 64 * cfg.waves_per_wg)
        return fail(Q8K4V_EUNSUPPORTED, "attention: sequence too long (more than 1024 splits of 64 pages per wave)");
    // the in-launch merge keeps one arrival counter per (sequence, kv head,
    // row chunk) in the workspace header; a launch with more items than the
    // header holds merges with the separate combine kernel instead
    const int64_t n_ctr = (int64_t)a.n_seqs * H * plan->row_chunks;
    plan->fused_combine = (plan->n_splits > 1 && cfg.fused_combine && n_ctr <= kMaxCounters) ? 1 : 0;
    const size_t rec = (size_t)(a.cache->head_dim + 4) * sizeof(float);
    plan->partial_bytes = plan->n_splits > 1 ? (size_t)a.n_seqs * H * plan->n_splits * rows * rec : 0;
    plan->partial_bytes = (plan->partial_bytes + 255) / 256 * 256;
    plan->counter_bytes = plan->fused_combine ? (size_t)n_ctr * sizeof(uint32_t) : 0;
    if ((int64_t)a.n_seqs * H * plan->n_splits * plan->row_chunks + 8 > 0x7FFFFFFFLL)
        return fail(Q8K4V_EINVAL, "attention: launch too large");
    return Q8K4V_OK;
}

// Every plan that writes split records puts them behind the header, fused
// or not, so the header's counters are never overwritten by another plan's
// records; a single-split plan writes nothing to the workspace.
size_t plan_workspace(const Plan& p) { return p.partial_bytes ? Q8K4V_WS_HEADER_BYTES + p.partial_bytes : 0; }

namespace {
// Kernel parameters of one plain launch (no page offsets, no cascade).
AttnParams launch_params(const AttnArgs& a, const Plan& plan, void* workspace) {
    const q8k4v_cache& c = *a.cache;
    AttnParams kp{};
    kp.k_codes = c.k_codes;
    kp.k_scales = c.k_scales;
    kp.v_codes = c.v_codes;
    kp.v_scales = c.v_scales;
    kp.q = a.q;
    kp.out = a.out;
    kp.partials = plan.partial_bytes ? (float*)((char*)workspace + Q8K4V_WS_HEADER_BYTES) : nullptr;
    kp.counters = plan.counter_bytes ? (uint32_t*)workspace : nullptr;
    kp.seq_lens = a.seq_lens;
    kp.page_table = a.page_table;
    kp.H = c.num_kv_heads;
    kp.max_pages = a.max_pages;
    kp.n_seqs = a.n_seqs;
    kp.Hq = a.num_q_heads;
    kp.G = a.num_q_heads / c.num_kv_heads;
    kp.W = a.n_draft;
    kp.R = plan.rows;
    kp.split_pages = plan.split_pages;
    kp.n_splits = plan.n_splits;
    kp.row_chunks = plan.row_chunks;
    kp.scale_log2 = a.softmax_scale * kLog2e;
    kp.direct = plan.n_splits == 1;
    kp.fused = plan.fused_combine;
    kp.affine = c.codec == Q8K4V_CODEC_AFFINE;
    kp.k_zeros = c.k_zeros;
    kp.v_zeros = c.v_zeros;
    return kp;
}

int32_t launch_kernel(const AttnParams& kp, const Plan& plan, int head_dim, bool bf, hipStream_t stream) {
    return plan.kernel == kDec2 ? launch_dec2(kp, plan, head_dim, bf, stream) : launch_rows(kp, plan, head_dim, bf, stream);
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

int32_t launch_attention(const AttnArgs& a, const Plan& plan, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    const size_t need = plan_workspace(plan);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(Q8K4V_EWORKSPACE, "attention: workspace needs " + std::to_string(need) + " bytes");
    const AttnParams kp = launch_params(a, plan, workspace);
    const int D = a.cache->head_dim;
    const int32_t rc = launch_kernel(kp, plan, D, a.q_dtype == Q8K4V_BF16, stream);
    if (rc != Q8K4V_OK) return rc;
    if (!kp.direct && !kp.fused) return launch_combine(kp, D, plan.rows_per_wg, stream);
    return Q8K4V_OK;
}

// ---- shared-prefix cascade ------------------------------------------------
// Sessions whose first n_prefix_pages logical pages are the same physical
// pages (a shared prompt prefix, blog.123qwe.co.kr/?p=3927, section 5) are
// decoded in two passes and a combine: a prefix pass of the row-block kernel
// over one virtual sequence -- the shared pages, read once for all sessions
// -- whose query rows are every session's rows (session j as "draft" j, no
// causal edge inside the prefix); a suffix pass, the plain decode plan over
// each session's pages from n_prefix_pages on; and a combine that merges both
// record sets per (session, q head) by log-sum-exp.  When the suffix plan is
// the four-wave, two-stage replicated-row kernel and the prefix block has more
// than 16 rows, both passes run in one launch (the prefix pass then takes
// four waves too): the compute-bound prefix workgroups and the memory-bound
// suffix workgroups share the CUs.
int32_t make_cascade_plan(const AttnArgs& a, int32_t n_pref, const q8k4v_config* cfg, CascadePlan* cp) {
    if (n_pref < 1 || n_pref > a.max_pages || (int64_t)n_pref * Q8K4V_PAGE_SIZE > a.max_seq_len)
        return fail(Q8K4V_EINVAL, "attention: n_prefix_pages must be in 1 .. min(max_pages, max_seq_len / 16)");
    AttnArgs as = a;
    as.max_seq_len = a.max_seq_len - n_pref * Q8K4V_PAGE_SIZE;
    int32_t rc = make_plan(as, cfg, &cp->suf);
    if (rc != Q8K4V_OK) return rc;
    const int32_t H = a.cache->num_kv_heads;
    const int32_t G = a.num_q_heads / H;
    const size_t rec = (size_t)(a.cache->head_dim + 4) * sizeof(float);
    Plan& sp = cp->suf;
    sp.fused_combine = 0;
    sp.counter_bytes = 0;
    sp.partial_bytes = round256((size_t)a.n_seqs * H * sp.n_splits * sp.rows * rec);

    Plan& pp = cp->pre;
    const int64_t rows = (int64_t)a.n_seqs * G;
    if (rows > kMaxPrefixRows)
        return fail(Q8K4V_EUNSUPPORTED, "attention: the prefix pass takes at most " + std::to_string(kMaxPrefixRows) +
                                            " query rows per kv head (n_seqs * group)");
    pp = Plan{};
    pp.rows = (int32_t)rows;
    pp.kernel = kRows;
    pp.tile_pages = 2;
    // 8 waves for a large prefix block on its own; 4 when it shares the
    // launch with a four-wave, two-stage replicated-row suffix pass
    const bool fuse = rows > 16 && sp.kernel == kDec2 && (sp.rows == 4 || sp.rows == 8) && sp.waves == 4 &&
                      sp.stages == 2;
    pp.waves = (rows > 16 && !fuse) ? 8 : 4;
    pp.stages = 2;
    pp.rows_per_wg = rows > 16 ? 32 : 16;
    pp.row_chunks = (pp.rows + pp.rows_per_wg - 1) / pp.rows_per_wg;
    const int32_t unit = pp.tile_pages * pp.waves;
    const int64_t per = (int64_t)H * pp.row_chunks;
    // one prefix workgroup per CU on its own; one per two CUs in the fused
    // launch, which leaves room for the suffix workgroups (measured)
    const int64_t target = fuse ? device_cu_count() / 2 : device_cu_count();
    const int64_t splits = std::max<int64_t>(1, (target + per - 1) / per);
    int32_t spp = round_up((int32_t)((n_pref + splits - 1) / splits), unit);
    spp = std::min(std::max(spp, unit), 64 * pp.waves);
    pp.split_pages = spp;
    pp.n_splits = (n_pref + spp - 1) / spp;
    pp.fused_combine = 0;
    pp.counter_bytes = 0;
    pp.partial_bytes = round256((size_t)H * pp.n_splits * pp.rows * rec);
    if (per * pp.n_splits + 8 > 0x7FFFFFFFLL) return fail(Q8K4V_EINVAL, "attention: launch too large");
    return Q8K4V_OK;
}

// The cascade's records sit behind the workspace header too (it keeps no
// counters), so one workspace serves every entry point.
size_t cascade_workspace(const CascadePlan& cp) {
    return Q8K4V_WS_HEADER_BYTES + cp.pre.partial_bytes + cp.suf.partial_bytes;
}

int32_t launch_cascade(const AttnArgs& a, int32_t n_pref, const CascadePlan& cp, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    const size_t need = cascade_workspace(cp);
    if (!workspace || workspace_bytes < need)
        return fail(Q8K4V_EWORKSPACE, "attention: workspace needs " + std::to_string(need) + " bytes");
    const int D = a.cache->head_dim;
    const bool bf = a.q_dtype == Q8K4V_BF16;
    float* pre_part = (float*)((char*)workspace + Q8K4V_WS_HEADER_BYTES);
    float* suf_part = (float*)((char*)workspace + Q8K4V_WS_HEADER_BYTES + cp.pre.partial_bytes);

    AttnParams pre = launch_params(a, cp.pre, pre_part);
    pre.partials = pre_part;
    pre.n_seqs = 1;                 // page table row 0 holds the shared pages
    pre.W = a.n_seqs;               // session j's rows are "draft" j
    pre.R = cp.pre.rows;
    pre.page_cap = n_pref;
    pre.cascade = 1;
    pre.direct = 0;
    pre.fused = 0;

    AttnParams suf = launch_params(a, cp.suf, suf_part);
    suf.partials = suf_part;
    suf.page_lo = n_pref;
    suf.cascade = 1;
    suf.direct = 0;
    suf.fused = 0;

    int32_t rc;
    if (cascade_fusable(cp.pre, cp.suf)) {
        rc = launch_cascade_fused(pre, suf, D, bf, cp.suf.rows, stream);
        if (rc != Q8K4V_OK) return rc;
    } else {
        rc = launch_rows(pre, cp.pre, D, bf, stream);
        if (rc != Q8K4V_OK) return rc;
        rc = launch_kernel(suf, cp.suf, D, bf, stream);
        if (rc != Q8K4V_OK) return rc;
    }

    suf.pre_partials = pre_part;
    suf.pre_splits = cp.pre.n_splits;
    suf.pre_eff = (n_pref + cp.pre.split_pages - 1) / cp.pre.split_pages;
    suf.pre_R = cp.pre.rows;
    return launch_combine_cascade(suf, D, stream);
}

q8k4v_config cascade_default_config(int32_t group) {
    q8k4v_config c = default_config(std::max(1, group));
    c.wgs_per_cu = kCascadeSuffixWgsPerCu;
    return c;
}

// Suffix-pass configuration of the cascade: the caller's, else the one
// tune_select installed for this device and head shape, else the decode
// defaults with more, shorter splits (ragged suffixes balance better).
static const q8k4v_config* cascade_config(const q8k4v_config* cfg, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, q8k4v_config* dflt) {
    if (cfg || num_kv_heads <= 0) return cfg;
    if (tuned_lookup(kTunedCascadeKey, num_q_heads, num_kv_heads, head_dim, dflt)) return dflt;
    *dflt = cascade_default_config(num_q_heads / num_kv_heads);
    return dflt;
}

}  // namespace q8k4v

using namespace q8k4v;

extern "C" {

const char* q8k4v_last_error(void) { return g_last_error.c_str(); }

const char* q8k4v_version(void) { return "q8k4v 1 gfx950 " Q8K4V_BUILD_ID; }

int32_t kv_quant_append(const q8k4v_cache* cache, const void* k_new, const void* v_new, int32_t dtype,
                        const int32_t* cu_new, const int32_t* start_pos, const int32_t* page_table,
                        int32_t max_pages, int32_t n_seqs, int32_t total_new, hipStream_t stream) {
    std::string why;
    if (!valid_cache(cache, &why)) return fail(Q8K4V_EINVAL, "kv_quant_append: " + why);
    if (dtype != Q8K4V_F32 && dtype != Q8K4V_BF16) return fail(Q8K4V_EINVAL, "kv_quant_append: dtype must be F32 or BF16");
    if (n_seqs < 1) return fail(Q8K4V_EINVAL, "kv_quant_append: n_seqs must be >= 1");
    if (total_new < 0) return fail(Q8K4V_EINVAL, "kv_quant_append: total_new must be >= 0");
    if (max_pages < 1) return fail(Q8K4V_EINVAL, "kv_quant_append: max_pages must be >= 1");
    if (total_new == 0) return Q8K4V_OK;
    if (!k_new || !v_new || !cu_new || !start_pos || !page_table)
        return fail(Q8K4V_EINVAL, "kv_quant_append: NULL input pointer");
    AppendArgs a{cache, k_new, v_new, dtype, cu_new, start_pos, page_table, max_pages, n_seqs, total_new, nullptr};
    return launch_append(a, stream);
}

// Launch arguments with placeholder pointers, for workspace queries.
static AttnArgs shape_args(q8k4v_cache* fake, int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t max_seq_len, int32_t n_draft) {
    fake->num_pages = 1;
    fake->num_kv_heads = num_kv_heads;
    fake->head_dim = head_dim;
    fake->page_size = Q8K4V_PAGE_SIZE;
    fake->k_codes = (int8_t*)1;
    fake->k_scales = (uint16_t*)1;
    fake->v_codes = (uint8_t*)1;
    fake->v_scales = (uint16_t*)1;
    fake->codec = Q8K4V_CODEC_SYMMETRIC;
    fake->k_zeros = nullptr;
    fake->v_zeros = nullptr;
    AttnArgs a{};
    a.cache = fake;
    a.q = (const void*)1;
    a.q_dtype = Q8K4V_BF16;
    a.out = (float*)1;
    a.n_seqs = n_seqs;
    a.num_q_heads = num_q_heads;
    a.n_draft = n_draft <= 0 ? 1 : n_draft;
    a.seq_lens = (const int32_t*)1;
    a.max_seq_len = max_seq_len;
    a.page_table = (const int32_t*)1;
    a.max_pages = std::max(1, (max_seq_len + 15) / 16);
    a.softmax_scale = 1.0f;
    return a;
}

size_t q8k4v_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_seq_len, int32_t n_draft, const q8k4v_config* cfg) {
    q8k4v_cache fake;
    const AttnArgs a = shape_args(&fake, n_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, n_draft);
    Plan p;
    std::string saved = g_last_error;
    if (make_plan(a, cfg, &p) != Q8K4V_OK) { g_last_error = saved; return 0; }
    return plan_workspace(p);
}


size_t q8k4v_prefix_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_seq_len, int32_t n_prefix_pages, const q8k4v_config* cfg) {
    if (n_prefix_pages == 0)
        return q8k4v_workspace_bytes(n_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, 0, cfg);
    q8k4v_config dflt;
    cfg = cascade_config(cfg, num_q_heads, num_kv_heads, head_dim, &dflt);
    // the larger need of the codecs the configuration supports (a plan
    // unavailable for one codec does not count)
    size_t need = 0;
    const std::string saved = g_last_error;
    for (int32_t codec : {Q8K4V_CODEC_SYMMETRIC, Q8K4V_CODEC_AFFINE}) {
        q8k4v_cache fake;
        const AttnArgs a = shape_args(&fake, n_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, 1);
        fake.codec = codec;
        fake.k_zeros = (int8_t*)1;
        fake.v_zeros = (uint8_t*)1;
        CascadePlan cp;
        if (make_plan(a, cfg, &cp.suf) == Q8K4V_OK && make_cascade_plan(a, n_prefix_pages, cfg, &cp) == Q8K4V_OK)
            need = std::max(need, cascade_workspace(cp));
    }
    g_last_error = saved;
    return need;
}

static int32_t attention_entry(const char* name, const q8k4v_cache* cache, const void* q, int32_t q_dtype,
                               float* out, int32_t n_seqs, int32_t num_q_heads, int32_t n_draft,
                               const int32_t* seq_lens, int32_t max_seq_len, const int32_t* page_table,
                               int32_t max_pages, float softmax_scale, const q8k4v_config* cfg,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    AttnArgs a{cache, q, q_dtype, out, n_seqs, num_q_heads, n_draft, seq_lens, max_seq_len,
               page_table, max_pages, softmax_scale};
    Plan plan;
    int32_t rc = make_plan(a, cfg, &plan);
    if (rc != Q8K4V_OK) {
        g_last_error = std::string(name) + ": " + g_last_error;
        return rc;
    }
    return launch_attention(a, plan, workspace, workspace_bytes, stream);
}

int32_t attn_decode_q8k4v(const q8k4v_cache* cache, const void* q, int32_t q_dtype, float* out, int32_t n_seqs,
                          int32_t num_q_heads, const int32_t* seq_lens, int32_t max_seq_len,
                          const int32_t* page_table, int32_t max_pages, float softmax_scale,
                          const q8k4v_config* cfg, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return attention_entry("attn_decode_q8k4v", cache, q, q_dtype, out, n_seqs, num_q_heads, 1, seq_lens,
                           max_seq_len, page_table, max_pages, softmax_scale, cfg, workspace, workspace_bytes,
                           stream);
}

int32_t attn_decode_prefix_q8k4v(const q8k4v_cache* cache, const void* q, int32_t q_dtype, float* out,
                                 int32_t n_seqs, int32_t num_q_heads, const int32_t* seq_lens, int32_t max_seq_len,
                                 const int32_t* page_table, int32_t max_pages, int32_t n_prefix_pages,
                                 float softmax_scale, const q8k4v_config* cfg, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    const char* name = "attn_decode_prefix_q8k4v";
    if (n_prefix_pages < 0) return fail(Q8K4V_EINVAL, std::string(name) + ": n_prefix_pages must be >= 0");
    if (n_prefix_pages == 0)
        return attention_entry(name, cache, q, q_dtype, out, n_seqs, num_q_heads, 1, seq_lens, max_seq_len,
                               page_table, max_pages, softmax_scale, cfg, workspace, workspace_bytes, stream);
    AttnArgs a{cache, q, q_dtype, out, n_seqs, num_q_heads, 1, seq_lens, max_seq_len,
               page_table, max_pages, softmax_scale};
    q8k4v_config dflt;
    cfg = cascade_config(cfg, num_q_heads, cache ? cache->num_kv_heads : 0, cache ? cache->head_dim : 0, &dflt);
    CascadePlan cp;
    int32_t rc = make_plan(a, cfg, &cp.suf);        // validates the shape as a decode launch
    if (rc == Q8K4V_OK) rc = make_cascade_plan(a, n_prefix_pages, cfg, &cp);
    if (rc != Q8K4V_OK) {
        g_last_error = std::string(name) + ": " + g_last_error;
        return rc;
    }
    return launch_cascade(a, n_prefix_pages, cp, workspace, workspace_bytes, stream);
}

int32_t attn_decode_append_q8k4v(const q8k4v_cache* cache, const void* k_new, const void* v_new, int32_t new_dtype,
                                 const void* q, int32_t q_dtype, float* out, int32_t n_seqs, int32_t num_q_heads,
                                 const int32_t* seq_lens, int32_t max_seq_len, const int32_t* page_table,
                                 int32_t max_pages, float softmax_scale, const q8k4v_config* cfg, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    const char* name = "attn_decode_append_q8k4v";
    if (!k_new || !v_new) return fail(Q8K4V_EINVAL, std::string(name) + ": NULL k_new / v_new");
    if (new_dtype != Q8K4V_F32 && new_dtype != Q8K4V_BF16) return fail(Q8K4V_EINVAL, std::string(name) + ": new_dtype must be F32 or BF16");
    if (max_seq_len < 1) return fail(Q8K4V_EINVAL, std::string(name) + ": max_seq_len must count the new token");
    AttnArgs a{cache, q, q_dtype, out, n_seqs, num_q_heads, 1, seq_lens, max_seq_len, page_table, max_pages,
               softmax_scale};
    Plan plan;
    int32_t rc = make_plan(a, cfg, &plan);
    if (rc != Q8K4V_OK) {
        g_last_error = std::string(name) + ": " + g_last_error;
        return rc;
    }
    const size_t need = plan_workspace(plan);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(Q8K4V_EWORKSPACE, std::string(name) + ": workspace needs " + std::to_string(need) + " bytes");
    if (decode_append_fusable(plan, *cache)) {
        AttnParams kp = launch_params(a, plan, workspace);
        kp.k_new = k_new;
        kp.v_new = v_new;
        kp.new_bf16 = new_dtype == Q8K4V_BF16;
        const int D = cache->head_dim;
        rc = launch_dec2_append(kp, plan, D, q_dtype == Q8K4V_BF16, stream);
        if (rc != Q8K4V_OK) return rc;
        if (!kp.direct && !kp.fused) return launch_combine(kp, D, plan.rows_per_wg, stream);
        return Q8K4V_OK;
    }
    // other plans: the append kernel (one token per sequence), then the decode
    AppendArgs ap{cache, k_new, v_new, new_dtype, nullptr, nullptr, page_table, max_pages, n_seqs, n_seqs, seq_lens};
    rc = launch_append(ap, stream);
    if (rc != Q8K4V_OK) return rc;
    return launch_attention(a, plan, workspace, workspace_bytes, stream);
}

int32_t attn_prefill_q8k4v(const q8k4v_cache* cache, const void* q, int32_t q_dtype, float* out, int32_t n_seqs,
                           int32_t num_q_heads, int32_t n_new, const int32_t* seq_lens, int32_t max_seq_len,
                           const int32_t* page_table, int32_t max_pages, float softmax_scale,
                           const q8k4v_config* cfg, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (n_new < 1 || n_new > Q8K4V_MAX_CHUNK) return fail(Q8K4V_EINVAL, "attn_prefill_q8k4v: n_new must be in 1..1024");
    if (max_seq_len < n_new) return fail(Q8K4V_EINVAL, "attn_prefill_q8k4v: max_seq_len must hold the new tokens");
    return attention_entry("attn_prefill_q8k4v", cache, q, q_dtype, out, n_seqs, num_q_heads, n_new, seq_lens,
                           max_seq_len, page_table, max_pages, softmax_scale, cfg, workspace, workspace_bytes,
                           stream);
}

int32_t attn_verify_q8k4v(const q8k4v_cache* cache, const void* q, int32_t q_dtype, float* out, int32_t n_seqs,
                          int32_t num_q_heads, int32_t n_draft, const int32_t* seq_lens, int32_t max_seq_len,
                          const int32_t* page_table, int32_t max_pages, float softmax_scale,
                          const q8k4v_config* cfg, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (n_draft < 1 || n_draft > Q8K4V_MAX_DRAFT) return fail(Q8K4V_EINVAL, "attn_verify_q8k4v: n_draft must be in 1..16");
    if (max_seq_len < n_draft) return fail(Q8K4V_EINVAL, "attn_verify_q8k4v: max_seq_len must hold the drafts");
    return attention_entry("attn_verify_q8k4v", cache, q, q_dtype, out, n_seqs, num_q_heads, n_draft, seq_lens,
                           max_seq_len, page_table, max_pages, softmax_scale, cfg, workspace, workspace_bytes,
                           stream);
}

}  // extern "C"
