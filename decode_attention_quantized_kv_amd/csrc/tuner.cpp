// On-device tuner of the attention launch configuration (the first-load
// tuner of blog.123qwe.co.kr/?p=3927, section 3, with the admission rule of
// section 4).  Contract: tune_select in include/q8k4v.h.
//
// Everything below runs inside one wall-clock budget (<= 60 s): memory
// admission, synthesis of the timing caches on the device, the defaults'
// measurements and outputs, the storage-resolution noise, the candidates and
// their gate.  Per unit (decode: one query row block per kv head; verify:
// n_draft drafts; with n_sessions, multi-session: the shared-prefix entry
// point's suffix pass, ns sessions over a ctx / 2 token shared prefix with
// private suffixes of about (i + 1) / ns x ctx / 2 tokens) the service cost
// of a configuration c is
//     cost(c) = sum over the unit's two shapes p of median(c, p) / median(default, p)
// with shapes at ctx_small and ctx_large, term weights 1, one launch per
// layer-step.  Times are per launch within a replayed graph of launches on
// the tuner's own stream (medians over replays, bracketed by HIP events);
// the launches rotate over distinct cache copies (and, for the small
// context, over disjoint page sets) whose total exceeds four times the
// 256 MiB last-level cache, so every launch streams from HBM.
//
// Order: each unit's default first; then one candidate at a time from the
// unit with the earliest virtual completion time
//     (effort + price) / (share x opportunity)
// (section 3 of the same page): effort = wall time already spent on the unit,
// price = wall time of its last measurement, share = the unit's part of the
// default service time, opportunity = the fraction of its generated
// candidates still unmeasured.  Within a unit, the structural variants (which
// kernel) come first, then a refinement of the launch shape (stages, waves
// per workgroup, workgroups per CU, fused combine) around the best structural
// choice.  A candidate that is not fully measured and checked before the
// deadline is "unknown" and is never admitted.
//
// Records: with a record path, the choice is stored per device identity
// (architecture, device name and CU count, HIP runtime and driver versions,
// library build) and request shape; a later call with the same identity and
// shape uses the stored choice without measuring, and a changed identity
// (new driver, toolchain or library) searches again.  Admission: on each of
// the unit's two shapes, the candidate's output may differ from the default
// configuration's output by at most alpha = 8 times the storage-resolution
// noise -- the change of the default output when every stored code moves by
// one quantisation step -- and, on every term for which the caller passes a
// reference output (decode, verify and multi-session at both contexts, e.g.
// computed by a CPU oracle on the caller's inputs), the sigma-normalised deviation from it
// may not exceed ref_tol.  A deviation that was not measured is reported as
// unknown (null), never as 0.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <sstream>
#include <string>
#include <vector>

#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

using Clock = std::chrono::steady_clock;

constexpr double kAlpha = 8.0;
constexpr size_t kLlcBytes = size_t(256) << 20;
constexpr int kMaxBudgetMs = 60000;

// ---- device-side synthesis (counter-based hash, no state) -----------------

__device__ __forceinline__ uint32_t mix32(uint64_t x) {
    x ^= x >> 33;
    x *= 0xff51afd7ed558ccdULL;
    x ^= x >> 33;
    x *= 0xc4ceb9fe1a85ec53ULL;
    x ^= x >> 33;
    return (uint32_t)x;
}

__device__ __forceinline__ float unit_float(uint32_t h) { return (float)(h >> 8) * (1.0f / 16777216.0f); }

// Random cache contents: key codes in -127..127, value codes in -7..7 (two
// per byte), key scales 0.01..0.03, value scales 0.2..0.6 (the magnitudes of
// N(0,1) data quantised per row / per 32-dim group).
__global__ void fill_cache_kernel(int8_t* kc, uint16_t* ks, uint8_t* vc, uint16_t* vs, size_t nk, size_t nks,
                                  size_t nv, size_t nvs, uint64_t seed) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (size_t i = i0; i < nk; i += stride) kc[i] = (int8_t)((int)(mix32(seed ^ (i * 4 + 0)) % 255u) - 127);
    for (size_t i = i0; i < nv; i += stride) {
        const uint32_t h = mix32(seed ^ (i * 4 + 1));
        const int lo = (int)(h % 15u) - 7, hi = (int)((h >> 16) % 15u) - 7;
        vc[i] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
    }
    for (size_t i = i0; i < nks; i += stride)
        ks[i] = __builtin_bit_cast(uint16_t, (_Float16)(0.01f + 0.02f * unit_float(mix32(seed ^ (i * 4 + 2)))));
    for (size_t i = i0; i < nvs; i += stride)
        vs[i] = __builtin_bit_cast(uint16_t, (_Float16)(0.2f + 0.4f * unit_float(mix32(seed ^ (i * 4 + 3)))));
}

// dst = src with every code moved one step up or down (seeded sign, kept in
// range); scales copied unchanged.
__global__ void perturb_cache_kernel(const int8_t* kc, const uint16_t* ks, const uint8_t* vc, const uint16_t* vs,
                                     int8_t* dkc, uint16_t* dks, uint8_t* dvc, uint16_t* dvs, size_t nk, size_t nks,
                                     size_t nv, size_t nvs, uint64_t seed) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (size_t i = i0; i < nk; i += stride) {
        int c = kc[i] + ((mix32(seed ^ (i * 2)) & 1u) ? 1 : -1);
        if (c > 127) c = 126;
        if (c < -127) c = -126;
        dkc[i] = (int8_t)c;
    }
    for (size_t i = i0; i < nv; i += stride) {
        const uint32_t h = mix32(seed ^ (i * 2 + 1));
        const uint8_t b = vc[i];
        int lo = (int)(b & 0xF), hi = (int)(b >> 4);
        lo = lo >= 8 ? lo - 16 : lo;
        hi = hi >= 8 ? hi - 16 : hi;
        lo += (h & 1u) ? 1 : -1;
        hi += (h & 2u) ? 1 : -1;
        lo = lo > 7 ? 6 : (lo < -7 ? -6 : lo);
        hi = hi > 7 ? 6 : (hi < -7 ? -6 : hi);
        dvc[i] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
    }
    for (size_t i = i0; i < nks; i += stride) dks[i] = ks[i];
    for (size_t i = i0; i < nvs; i += stride) dvs[i] = vs[i];
}

// bf16 queries, uniform on (-1.73, 1.73) (unit variance).
__global__ void fill_bf16_kernel(uint16_t* q, size_t n, uint64_t seed) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = (unit_float(mix32(seed ^ i)) * 2.0f - 1.0f) * 1.7320508f;
        q[i] = (uint16_t)(__float_as_uint(x) >> 16);
    }
}

// ---- host side --------------------------------------------------------------

constexpr int kUnits = 3;          // decode, verify, multi-session
constexpr int kMaxSessions = 64;

struct Shape {
    std::string name;
    int kind = 0;      // 0 decode, 1 verify, 2 sessions over a shared prefix (the cascade)
    int n_draft = 1;   // 1 for decode and the cascade
    int ctx = 0;       // cached tokens (drafts included for verify); the longest session
    bool small = false;
    int n_seqs = 1, n_pref = 0, max_pages = 0;   // the cascade's sessions, shared pages, table row length
};

constexpr double kUnmeasured = NAN;   // printed as null ("unknown")

struct Cand {
    q8k4v_config cfg;
    std::string stage;             // "default", "structural", "refine"
    std::string verdict;           // "admitted", "rejected", "invalid", "unknown"
    std::string gate;              // rejected by: "alpha" or "oracle"
    std::string why;
    double t[2] = {kUnmeasured, kUnmeasured};     // median microseconds per shape
    double dev[2] = {kUnmeasured, kUnmeasured};   // max |out - default out| per shape
    double ref_dev[2] = {kUnmeasured, kUnmeasured};   // normalised deviation from the unit's references
    double cost = kUnmeasured;
    int seq = -1;                  // position in the measurement order (all units)
    double vt[kUnits] = {-1, -1, -1};   // virtual completion times of the units when it was picked
};

// Search state of one unit: measured candidates (default first), the queue
// of generated but unmeasured ones, and the accounting of the search order.
struct UnitSearch {
    std::vector<Cand> cands;
    std::vector<Cand> queue;       // front first
    size_t best_i = 0;
    bool active = false;           // default admitted: the unit is searched
    bool refined = false;          // refinement queue generated
    int generated = 0;             // non-default candidates generated so far
    double effort_ms = 0, price_ms = 0;
};

struct Arena {
    std::vector<void*> ptrs;
    ~Arena() {
        for (void* p : ptrs) (void)hipFree(p);
    }
    void* alloc(size_t bytes) {
        void* p = nullptr;
        if (hipMalloc(&p, std::max<size_t>(bytes, 256)) != hipSuccess) return nullptr;
        ptrs.push_back(p);
        return p;
    }
};

std::string cfg_json(const q8k4v_config& c) {
    char b[256];
    std::snprintf(b, sizeof b,
                  "{\"variant\":%d,\"waves_per_wg\":%d,\"wgs_per_cu\":%d,\"split_pages\":%d,\"fused_combine\":%d,"
                  "\"stages\":%d}",
                  c.variant, c.waves_per_wg, c.wgs_per_cu, c.split_pages, c.fused_combine, c.stages);
    return b;
}

bool same_cfg(const q8k4v_config& a, const q8k4v_config& b) {
    return a.variant == b.variant && a.waves_per_wg == b.waves_per_wg && a.wgs_per_cu == b.wgs_per_cu &&
           a.split_pages == b.split_pages && a.fused_combine == b.fused_combine && a.stages == b.stages;
}

// Text safe inside a JSON string (quotes, backslashes and controls blanked).
std::string json_text(std::string w) {
    for (auto& ch : w)
        if (ch == '"' || ch == '\\' || (unsigned char)ch < 32) ch = ' ';
    return w;
}

std::string fmt(double x) {
    if (!std::isfinite(x)) return "null";     // JSON has no inf / nan
    char b[64];
    std::snprintf(b, sizeof b, "%.6g", x);
    return b;
}

class Tuner {
  public:
    Tuner(const q8k4v_tune_request& r, Clock::time_point deadline) : req_(r), deadline_(deadline) {}

    int32_t run(q8k4v_config* out_table, std::string* report);

  private:
    bool expired() const { return Clock::now() >= deadline_; }
    int rows_of(int unit) const { return (unit == 1 ? w_ : 1) * g_; }
    q8k4v_config unit_default(int unit) const {
        return unit == 2 ? cascade_default_config(g_) : default_config(rows_of(unit));
    }
    const char* unit_name(int unit) const { return unit == 0 ? "decode" : unit == 1 ? "verify" : "multi_session"; }
    int cascade_shape(Shape* s, const std::string& name, int ctx, bool small, std::vector<int32_t>* lens,
                      std::vector<int32_t>* rows) const;
    int32_t setup(std::string* why);
    int32_t launch(const q8k4v_config* cfg, const Shape& s, int copy, int set, float* out, const void* q);
    int32_t time_shape(const q8k4v_config* cfg, const Shape& s, double* median_us);
    int32_t output(const q8k4v_config* cfg, const Shape& s, int copy, std::vector<float>* host);
    int32_t ref_output(const q8k4v_config* cfg, int term, std::vector<float>* host);
    bool has_ref(int term) const { return req_.ref[term].cache != nullptr; }
    double ref_deviation(int term, const std::vector<float>& o) const;
    void start_unit(int unit, UnitSearch* u);
    void refine_queue(int unit, UnitSearch* u);
    void measure(int unit, Cand* c);

    const q8k4v_tune_request& req_;
    Clock::time_point deadline_;
    Arena arena_;
    hipStream_t stream_ = nullptr;
    std::vector<hipEvent_t> events_;
    int hq_ = 0, h_ = 0, d_ = 0, w_ = 0, g_ = 0, n_units_ = 2, ns_ = 0;
    float scale_ = 0;
    int pages_ = 0, small_pages_ = 0, n_copies_ = 0, n_sets_ = 0, reps_ = 0;
    int casc_window_ = 0, n_csets_ = 0;  // multi-session small shape: pages per set, sets
    double llc_multiple_ = 0;            // least bytes streamed per replay over the shapes, / LLC
    size_t cache_bytes_ = 0;
    std::vector<q8k4v_cache> copies_;
    int32_t* d_tables_ = nullptr;        // [n_sets][pages]: set 0 is the full permutation
    int32_t* d_lens_ = nullptr;          // [4]: decode small, decode large, verify small, verify large
    int32_t* d_ref_lens_ = nullptr;      // [4]: the caller's reference lengths of the decode / verify terms
    int32_t* d_casc_tables_ = nullptr;   // cascade page tables: [n_csets][ns][small max_pages], then [ns][large max_pages]
    int32_t* d_casc_lens_ = nullptr;     // cascade session lengths: [ns] small, [ns] large
    void* d_q_ = nullptr;                // bf16 [max(w, ns)][hq][d]
    float* d_out_ = nullptr;             // fp32 [max(w, ns)][hq][d]
    void* d_ws_ = nullptr;
    size_t ws_bytes_ = 0;
    Shape shapes_[kUnits][2];            // [unit][small/large]
    std::vector<float> def_out_[kUnits][2];   // default outputs per unit/shape on copy 0
    double noise_[kUnits][2] = {{0, 0}, {0, 0}, {0, 0}};
    double def_t_[kUnits][2] = {{0, 0}, {0, 0}, {0, 0}};
    std::string setup_note_;
    int seq_ = 0;                        // measurement order over all units
    std::string summary_, error_;

  public:
    const std::string& summary() const { return summary_; }
    const std::string& error() const { return error_; }
};

// A multi-session shape at context ctx: ns sessions share a ctx / 2 token
// prefix (whole pages); session i owns a private suffix of about
// (i + 1) / ns x ctx / 2 tokens (whole pages less i % 16 tokens: ragged
// lengths, a ragged last page), so the suffixes average about ctx / 4 tokens
// and the shortest and longest differ by ns.  The sessions' pages are
// window-relative: the prefix first, then each suffix in turn.  `rows` gets
// each session's page indices (max_pages each); returns the window's pages.
int Tuner::cascade_shape(Shape* s, const std::string& name, int ctx, bool small, std::vector<int32_t>* lens,
                         std::vector<int32_t>* rows) const {
    const int pre = std::max(1, ctx / 2 / Q8K4V_PAGE_SIZE);
    const int most = std::max(1, ctx / 2 / Q8K4V_PAGE_SIZE);    // the longest suffix, in pages
    s->name = name;
    s->kind = 2;
    s->n_draft = 1;
    s->small = small;
    s->n_seqs = ns_;
    s->n_pref = pre;
    s->max_pages = pre + most;
    lens->assign(ns_, 0);
    rows->assign((size_t)ns_ * s->max_pages, 0);
    int longest = 0, next = pre;
    for (int i = 0; i < ns_; ++i) {
        const int own = std::max(1, (int)((int64_t)most * (i + 1) / ns_));
        (*lens)[i] = Q8K4V_PAGE_SIZE * (pre + own) - i % 16;
        longest = std::max(longest, (*lens)[i]);
        for (int j = 0; j < s->max_pages; ++j)
            (*rows)[(size_t)i * s->max_pages + j] = j < pre ? j : j < pre + own ? next + (j - pre) : 0;
        next += own;
    }
    s->ctx = longest;
    return next;
}

int32_t Tuner::setup(std::string* why) {
    hq_ = req_.num_q_heads;
    h_ = req_.num_kv_heads;
    d_ = req_.head_dim;
    w_ = req_.n_draft;
    g_ = hq_ / h_;
    ns_ = req_.n_sessions >= 2 ? req_.n_sessions : 0;
    n_units_ = ns_ ? 3 : 2;
    scale_ = req_.softmax_scale > 0 ? req_.softmax_scale : 1.0f / std::sqrt((float)d_);
    const int ctx_s = req_.ctx_small, ctx_l = req_.ctx_large;
    const int dv_pages = (ctx_l + w_ + Q8K4V_PAGE_SIZE - 1) / Q8K4V_PAGE_SIZE;
    small_pages_ = (ctx_s + w_ + Q8K4V_PAGE_SIZE - 1) / Q8K4V_PAGE_SIZE;

    shapes_[0][0] = {"decode@" + std::to_string(ctx_s), 0, 1, ctx_s, true};
    shapes_[0][1] = {"decode@" + std::to_string(ctx_l), 0, 1, ctx_l, false};
    shapes_[1][0] = {"verify@" + std::to_string(ctx_s) + "+" + std::to_string(w_), 1, w_, ctx_s + w_, true};
    shapes_[1][1] = {"verify@" + std::to_string(ctx_l) + "+" + std::to_string(w_), 1, w_, ctx_l + w_, false};
    std::vector<int32_t> lens_s, rows_s, lens_l, rows_l;
    int casc_large_window = 0;
    if (ns_) {
        casc_window_ = cascade_shape(&shapes_[2][0], std::to_string(ns_) + " sessions@" + std::to_string(ctx_s / 2) +
                                     " shared", ctx_s, true, &lens_s, &rows_s);
        casc_large_window = cascade_shape(&shapes_[2][1], std::to_string(ns_) + " sessions@" +
                                          std::to_string(ctx_l / 2) + " shared", ctx_l, false, &lens_l, &rows_l);
    }
    // the pool of every copy: the large decode / verify context, or the large
    // multi-session window if that is larger
    pages_ = std::max(dv_pages, casc_large_window);
    const size_t per_th = (size_t)d_ + 2 + d_ / 2 + 2 * (d_ / 32);
    const size_t page_bytes = (size_t)h_ * Q8K4V_PAGE_SIZE * per_th;
    cache_bytes_ = (size_t)pages_ * page_bytes;
    // enough copies that every shape's replay streams 4x the LLC before a
    // copy comes round again: per copy, a large shape reads its pages, a
    // small one at most its disjoint page sets
    const size_t dv_bytes = (size_t)dv_pages * page_bytes;
    size_t per_copy = std::min(dv_bytes, (size_t)(pages_ / small_pages_) * small_pages_ * page_bytes);
    if (ns_)
        per_copy = std::min({per_copy, (size_t)casc_large_window * page_bytes,
                             (size_t)(pages_ / casc_window_) * casc_window_ * page_bytes});
    const int want = std::max(2, (int)((4 * kLlcBytes + per_copy - 1) / per_copy) + 1);

    // workspace: the largest any candidate can ask for (split count is capped
    // by the combine, so the bound is the cap times the row records)
    ws_bytes_ = 0;
    int max_len = ctx_l + w_;
    for (int k = 0; k < 4; ++k)
        if (has_ref(k)) max_len = std::max(max_len, req_.ref[k].len);
    for (int unit = 0; unit < n_units_; ++unit)
        for (int wgs : {1, 2, 3, 4, 6, 8})
            for (int waves : {2, 4, 8})
                for (int variant : {0, 4, 5}) {
                    q8k4v_config c = unit_default(unit);
                    c.wgs_per_cu = wgs;
                    c.waves_per_wg = waves;
                    c.variant = variant;
                    c.stages = 0;
                    c.fused_combine = unit == 2 ? 0 : 1;
                    if (unit < 2) {
                        ws_bytes_ = std::max(ws_bytes_, q8k4v_workspace_bytes(1, hq_, h_, d_, max_len, unit ? w_ : 1, &c));
                        continue;
                    }
                    for (int k = 0; k < 2; ++k) {
                        const Shape& sh = shapes_[2][k];
                        ws_bytes_ = std::max(ws_bytes_, q8k4v_prefix_workspace_bytes(ns_, hq_, h_, d_, sh.ctx, sh.n_pref, &c));
                        const q8k4v_tune_ref& r = req_.ref[4 + k];
                        if (r.cache)
                            ws_bytes_ = std::max(ws_bytes_, q8k4v_prefix_workspace_bytes(r.n_seqs, hq_, h_, d_, r.len,
                                                                                         r.n_prefix_pages, &c));
                    }
                }
    ws_bytes_ = std::max<size_t>(ws_bytes_, Q8K4V_WS_HEADER_BYTES);
    int qrows = std::max(w_, ns_);
    for (int k = 4; k < 6; ++k)
        if (ns_ && has_ref(k)) qrows = std::max(qrows, req_.ref[k].n_seqs);
    // page sets of the small shapes: disjoint windows of the pool, as many as
    // make a replay stream 4x the LLC over the copies (at most what fits); the
    // memory admission below assumes the most
    auto sets_for = [&](int window, int copies) {
        const size_t per = (size_t)copies * window * page_bytes;
        return std::max(1, std::min(pages_ / window, (int)((4 * kLlcBytes + per - 1) / per) + 1));
    };
    const int most_csets = ns_ ? std::max(1, pages_ / casc_window_) : 0;
    const size_t casc_table_ints = ns_ ? (size_t)most_csets * rows_s.size() + rows_l.size() : 0;
    n_sets_ = std::max(1, pages_ / small_pages_);

    size_t free_b = 0, total_b = 0;
    if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) return hip_fail(hipGetLastError(), "tune_select: hipMemGetInfo");
    const size_t cap = req_.mem_cap_bytes ? std::min(req_.mem_cap_bytes, free_b) : free_b;
    const size_t fixed = ws_bytes_ + (size_t)n_sets_ * pages_ * 4 + casc_table_ints * 4 + (size_t)qrows * hq_ * d_ * 6 +
                         (64u << 20);
    int copies = want;
    while (copies >= 2 && fixed + (size_t)copies * cache_bytes_ > cap) --copies;
    if (copies < 2) {
        *why = "memory admission: two cache copies of " + std::to_string(cache_bytes_) + " bytes do not fit in " +
               std::to_string(cap) + " bytes";
        return Q8K4V_ENOMEM;
    }
    if (copies < want) setup_note_ = "rotation limited by memory: " + std::to_string(copies) + " of " + std::to_string(want) + " copies";
    n_copies_ = copies;
    n_sets_ = sets_for(small_pages_, n_copies_);
    n_csets_ = ns_ ? sets_for(casc_window_, n_copies_) : 0;
    // bytes streamed by one replay of each shape's graph, over the LLC
    llc_multiple_ = (double)n_copies_ * n_sets_ * small_pages_ * page_bytes / (double)kLlcBytes;
    llc_multiple_ = std::min(llc_multiple_, (double)n_copies_ * dv_bytes / (double)kLlcBytes);
    if (ns_) {
        llc_multiple_ = std::min(llc_multiple_, (double)n_copies_ * n_csets_ * casc_window_ * page_bytes / (double)kLlcBytes);
        llc_multiple_ = std::min(llc_multiple_, (double)n_copies_ * casc_large_window * page_bytes / (double)kLlcBytes);
    }

    if (hipStreamCreateWithFlags(&stream_, hipStreamNonBlocking) != hipSuccess)
        return hip_fail(hipGetLastError(), "tune_select: stream");
    const size_t nk = (size_t)pages_ * h_ * 16 * d_, nks = (size_t)pages_ * h_ * 16;
    const size_t nv = (size_t)pages_ * h_ * d_ * 8, nvs = (size_t)pages_ * h_ * 16 * (d_ / 32);
    copies_.resize(n_copies_);
    for (int i = 0; i < n_copies_; ++i) {
        q8k4v_cache& c = copies_[i];
        c.num_pages = pages_;
        c.num_kv_heads = h_;
        c.head_dim = d_;
        c.page_size = Q8K4V_PAGE_SIZE;
        c.k_codes = (int8_t*)arena_.alloc(nk);
        c.k_scales = (uint16_t*)arena_.alloc(nks * 2);
        c.v_codes = (uint8_t*)arena_.alloc(nv);
        c.v_scales = (uint16_t*)arena_.alloc(nvs * 2);
        if (!c.k_codes || !c.k_scales || !c.v_codes || !c.v_scales) {
            *why = "hipMalloc of a cache copy failed";
            return Q8K4V_ENOMEM;
        }
        if (i == 1) {   // copy 1: copy 0 with every code moved one step
            hipLaunchKernelGGL(perturb_cache_kernel, dim3(2048), dim3(256), 0, stream_, copies_[0].k_codes,
                               copies_[0].k_scales, copies_[0].v_codes, copies_[0].v_scales, c.k_codes, c.k_scales,
                               c.v_codes, c.v_scales, nk, nks, nv, nvs, req_.seed ^ 0x5eedULL);
        } else {
            hipLaunchKernelGGL(fill_cache_kernel, dim3(2048), dim3(256), 0, stream_, c.k_codes, c.k_scales, c.v_codes,
                               c.v_scales, nk, nks, nv, nvs, req_.seed * 1000003ULL + (uint64_t)i);
        }
        if (hipGetLastError() != hipSuccess) return hip_fail(hipGetLastError(), "tune_select: fill");
        if (expired()) return Q8K4V_OK;
    }
    // page tables: a seeded permutation of the pool; set j of the small
    // context uses pages j*small_pages .. of it (disjoint sets)
    std::vector<int32_t> perm(pages_);
    for (int i = 0; i < pages_; ++i) perm[i] = i;
    uint64_t s = req_.seed * 6364136223846793005ULL + 1442695040888963407ULL;
    for (int i = pages_ - 1; i > 0; --i) {
        s = s * 6364136223846793005ULL + 1442695040888963407ULL;
        const int j = (int)((s >> 33) % (uint64_t)(i + 1));
        std::swap(perm[i], perm[j]);
    }
    std::vector<int32_t> tables((size_t)n_sets_ * pages_);
    for (int set = 0; set < n_sets_; ++set)
        for (int i = 0; i < pages_; ++i)
            tables[(size_t)set * pages_ + i] = perm[(i + (size_t)set * small_pages_) % pages_];
    // cascade tables: the window-relative pages through the same permutation
    // (small shape: set j's window starts at page j * window; large shape: at 0)
    std::vector<int32_t> casc_tables(ns_ ? (size_t)n_csets_ * rows_s.size() + rows_l.size() : 0);
    if (ns_) {
        for (int set = 0; set < n_csets_; ++set)
            for (size_t i = 0; i < rows_s.size(); ++i)
                casc_tables[set * rows_s.size() + i] = perm[(rows_s[i] + (size_t)set * casc_window_) % pages_];
        for (size_t i = 0; i < rows_l.size(); ++i) casc_tables[n_csets_ * rows_s.size() + i] = perm[rows_l[i]];
    }
    d_tables_ = (int32_t*)arena_.alloc(tables.size() * 4);
    d_lens_ = (int32_t*)arena_.alloc(16);
    d_ref_lens_ = (int32_t*)arena_.alloc(16);
    d_casc_tables_ = ns_ ? (int32_t*)arena_.alloc(casc_tables.size() * 4) : nullptr;
    d_casc_lens_ = ns_ ? (int32_t*)arena_.alloc((size_t)2 * ns_ * 4) : nullptr;
    d_q_ = arena_.alloc((size_t)qrows * hq_ * d_ * 2);
    d_out_ = (float*)arena_.alloc((size_t)qrows * hq_ * d_ * 4);
    d_ws_ = arena_.alloc(ws_bytes_);
    if (!d_tables_ || !d_lens_ || !d_ref_lens_ || !d_q_ || !d_out_ || !d_ws_ ||
        (ns_ && (!d_casc_tables_ || !d_casc_lens_))) {
        *why = "hipMalloc failed";
        return Q8K4V_ENOMEM;
    }
    const int32_t lens[4] = {shapes_[0][0].ctx, shapes_[0][1].ctx, shapes_[1][0].ctx, shapes_[1][1].ctx};
    const int32_t ref_lens[4] = {req_.ref[0].len, req_.ref[1].len, req_.ref[2].len, req_.ref[3].len};
    if (hipMemcpyAsync(d_tables_, tables.data(), tables.size() * 4, hipMemcpyHostToDevice, stream_) != hipSuccess ||
        hipMemcpyAsync(d_lens_, lens, sizeof lens, hipMemcpyHostToDevice, stream_) != hipSuccess ||
        hipMemcpyAsync(d_ref_lens_, ref_lens, sizeof ref_lens, hipMemcpyHostToDevice, stream_) != hipSuccess)
        return hip_fail(hipGetLastError(), "tune_select: upload");
    if (ns_) {
        std::vector<int32_t> cl(lens_s);
        cl.insert(cl.end(), lens_l.begin(), lens_l.end());
        if (hipMemcpyAsync(d_casc_tables_, casc_tables.data(), casc_tables.size() * 4, hipMemcpyHostToDevice, stream_) !=
                hipSuccess ||
            hipMemcpyAsync(d_casc_lens_, cl.data(), cl.size() * 4, hipMemcpyHostToDevice, stream_) != hipSuccess)
            return hip_fail(hipGetLastError(), "tune_select: upload");
        // the host vectors must outlive the copies
        if (hipStreamSynchronize(stream_) != hipSuccess) return hip_fail(hipGetLastError(), "tune_select: upload");
    }
    hipLaunchKernelGGL(fill_bf16_kernel, dim3(64), dim3(256), 0, stream_, (uint16_t*)d_q_, (size_t)qrows * hq_ * d_,
                       req_.seed ^ 0xA11CEULL);
    // the workspace header (the in-launch merge's counters) starts at zero;
    // every completed launch leaves it at zero, whatever its plan
    if (hipMemsetAsync(d_ws_, 0, Q8K4V_WS_HEADER_BYTES, stream_) != hipSuccess)
        return hip_fail(hipGetLastError(), "tune_select: memset");
    if (hipStreamSynchronize(stream_) != hipSuccess) return hip_fail(hipGetLastError(), "tune_select: synthesis");
    reps_ = 5;
    events_.resize(2 * reps_);
    for (auto& e : events_)
        if (hipEventCreate(&e) != hipSuccess) return hip_fail(hipGetLastError(), "tune_select: events");
    return Q8K4V_OK;
}

int32_t Tuner::launch(const q8k4v_config* cfg, const Shape& s, int copy, int set, float* out, const void* q) {
    if (s.kind == 2) {      // sessions over the shared prefix (small shape: page set `set`)
        const size_t small_rows = (size_t)ns_ * shapes_[2][0].max_pages;
        const int32_t* table = d_casc_tables_ + (s.small ? (size_t)set * small_rows : (size_t)n_csets_ * small_rows);
        const int32_t* lens = d_casc_lens_ + (s.small ? 0 : ns_);
        return attn_decode_prefix_q8k4v(&copies_[copy], q, Q8K4V_BF16, out, ns_, hq_, lens, s.ctx, table, s.max_pages,
                                        s.n_pref, scale_, cfg, d_ws_, ws_bytes_, stream_);
    }
    const int32_t* lens = d_lens_ + (s.kind == 1 ? 2 : 0) + (s.small ? 0 : 1);
    const int32_t* table = d_tables_ + (size_t)(s.small ? set : 0) * pages_;
    if (s.kind == 1)
        return attn_verify_q8k4v(&copies_[copy], q, Q8K4V_BF16, out, 1, hq_, s.n_draft, lens, s.ctx, table, pages_,
                                 scale_, cfg, d_ws_, ws_bytes_, stream_);
    return attn_decode_q8k4v(&copies_[copy], q, Q8K4V_BF16, out, 1, hq_, lens, s.ctx, table, pages_, scale_, cfg,
                             d_ws_, ws_bytes_, stream_);
}

int32_t Tuner::time_shape(const q8k4v_config* cfg, const Shape& s, double* median_us) {
    // One captured graph of launches that rotate over the cache copies (and,
    // for the small shape, over the disjoint page sets), so every replay
    // streams more than 4x the LLC from HBM and no copy is re-read within a
    // replay or across the seam between two.  Replaying a graph is how a
    // serving loop issues these launches (no host launch gap between them);
    // the time per launch is a replay's time over its launches, the median
    // over reps_ timed replays after one untimed.
    const int sets = s.kind == 2 ? n_csets_ : n_sets_;
    const int G = s.small ? n_copies_ * sets : n_copies_;
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(stream_, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return hip_fail(hipGetLastError(), "tune_select: begin capture");
    int32_t rc = Q8K4V_OK;
    for (int r = 0; r < G && rc == Q8K4V_OK; ++r)
        rc = launch(cfg, s, r % n_copies_, s.small ? (r / n_copies_) % sets : 0, d_out_, d_q_);
    const hipError_t ec = hipStreamEndCapture(stream_, &graph);
    if (rc != Q8K4V_OK || ec != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc != Q8K4V_OK ? rc : hip_fail(ec, "tune_select: capture");
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) return hip_fail(ei, "tune_select: graph instantiate");
    hipError_t e = hipGraphLaunch(exec, stream_);
    for (int r = 0; r < reps_ && e == hipSuccess; ++r) {
        e = hipEventRecord(events_[2 * r], stream_);
        if (e == hipSuccess) e = hipGraphLaunch(exec, stream_);
        if (e == hipSuccess) e = hipEventRecord(events_[2 * r + 1], stream_);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream_);
    (void)hipGraphExecDestroy(exec);
    if (e != hipSuccess) return hip_fail(e, "tune_select: timing");
    std::vector<double> t(reps_);
    for (int r = 0; r < reps_; ++r) {
        float ms = 0;
        if (hipEventElapsedTime(&ms, events_[2 * r], events_[2 * r + 1]) != hipSuccess)
            return hip_fail(hipGetLastError(), "tune_select: elapsed");
        t[r] = ms * 1e3 / G;
    }
    std::nth_element(t.begin(), t.begin() + reps_ / 2, t.end());
    *median_us = t[reps_ / 2];
    return Q8K4V_OK;
}

int32_t Tuner::output(const q8k4v_config* cfg, const Shape& s, int copy, std::vector<float>* host) {
    const size_t n = (size_t)(s.kind == 2 ? ns_ : s.n_draft) * hq_ * d_;
    if (hipMemsetAsync(d_out_, 0xFF, n * 4, stream_) != hipSuccess) return hip_fail(hipGetLastError(), "tune_select: memset");
    const int32_t rc = launch(cfg, s, copy, 0, d_out_, d_q_);
    if (rc != Q8K4V_OK) return rc;
    host->resize(n);
    if (hipMemcpyAsync(host->data(), d_out_, n * 4, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipStreamSynchronize(stream_) != hipSuccess)
        return hip_fail(hipGetLastError(), "tune_select: readback");
    return Q8K4V_OK;
}

// Output of a candidate on reference term `term` (0, 1 decode; 2, 3 verify;
// 4, 5 sessions over a shared prefix).
int32_t Tuner::ref_output(const q8k4v_config* cfg, int term, std::vector<float>* host) {
    const q8k4v_tune_ref& r = req_.ref[term];
    const int nrows = term >= 4 ? r.n_seqs : term >= 2 ? w_ : 1;
    const size_t n = (size_t)nrows * hq_ * d_;
    int32_t rc;
    if (hipMemsetAsync(d_out_, 0xFF, n * 4, stream_) != hipSuccess) return hip_fail(hipGetLastError(), "tune_select: memset");
    if (term >= 4)
        rc = attn_decode_prefix_q8k4v(r.cache, r.q, Q8K4V_BF16, d_out_, r.n_seqs, hq_, r.seq_lens, r.len, r.page_table,
                                      r.max_pages, r.n_prefix_pages, scale_, cfg, d_ws_, ws_bytes_, stream_);
    else if (term >= 2)
        rc = attn_verify_q8k4v(r.cache, r.q, Q8K4V_BF16, d_out_, 1, hq_, w_, d_ref_lens_ + term, r.len, r.page_table,
                               r.max_pages, scale_, cfg, d_ws_, ws_bytes_, stream_);
    else
        rc = attn_decode_q8k4v(r.cache, r.q, Q8K4V_BF16, d_out_, 1, hq_, d_ref_lens_ + term, r.len, r.page_table,
                               r.max_pages, scale_, cfg, d_ws_, ws_bytes_, stream_);
    if (rc != Q8K4V_OK) return rc;
    host->resize(n);
    if (hipMemcpyAsync(host->data(), d_out_, n * 4, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipStreamSynchronize(stream_) != hipSuccess)
        return hip_fail(hipGetLastError(), "tune_select: readback");
    return Q8K4V_OK;
}

// max over elements of |o - ref| / sigma (sigma per (q head, dim), 1 if not
// given); a non-finite output gives +inf.
double Tuner::ref_deviation(int term, const std::vector<float>& o) const {
    const float* ref = req_.ref[term].out;
    const float* sigma = req_.ref[term].sigma;
    const size_t hd = (size_t)hq_ * d_;
    double m = 0;
    for (size_t i = 0; i < o.size(); ++i) {
        const double sig = sigma ? (double)sigma[i % hd] : 1.0;
        const double d = std::fabs((double)o[i] - (double)ref[i]) / sig;
        if (!(d <= m)) m = std::isnan(d) ? INFINITY : d;
    }
    return m;
}

double max_abs_diff(const std::vector<float>& a, const float* b, size_t n) {
    double m = 0;
    for (size_t i = 0; i < n; ++i) {
        const double d = std::fabs((double)a[i] - (double)b[i]);
        if (!(d <= m)) m = std::isnan(d) ? INFINITY : d;
    }
    return m;
}

void Tuner::measure(int unit, Cand* c) {
    // timing on both shapes, then the alpha gate on both shapes, then the
    // oracle gate on the unit's reference terms; "unknown" if the deadline
    // passes first (what was not measured stays unknown)
    for (int k = 0; k < 2; ++k) {
        if (expired()) { c->verdict = "unknown"; c->why = "deadline"; return; }
        const int32_t rc = time_shape(&c->cfg, shapes_[unit][k], &c->t[k]);
        if (rc != Q8K4V_OK) { c->verdict = "invalid"; c->why = q8k4v_last_error(); return; }
    }
    for (int k = 0; k < 2; ++k) {
        if (expired()) { c->verdict = "unknown"; c->why = "deadline"; return; }
        std::vector<float> o;
        const int32_t rc = output(&c->cfg, shapes_[unit][k], 0, &o);
        if (rc != Q8K4V_OK) { c->verdict = "invalid"; c->why = q8k4v_last_error(); return; }
        c->dev[k] = max_abs_diff(def_out_[unit][k], o.data(), o.size());
        if (!(c->dev[k] <= kAlpha * noise_[unit][k])) {
            c->verdict = "rejected";
            c->gate = "alpha";
            c->why = shapes_[unit][k].name + ": deviation " + fmt(c->dev[k]) + " > alpha * noise " +
                     fmt(kAlpha * noise_[unit][k]);
            return;
        }
    }
    for (int k = 0; k < 2; ++k) {
        const int term = 2 * unit + k;
        if (!has_ref(term)) continue;
        if (expired()) { c->verdict = "unknown"; c->why = "deadline"; return; }
        std::vector<float> o;
        const int32_t rc = ref_output(&c->cfg, term, &o);
        if (rc != Q8K4V_OK) { c->verdict = "invalid"; c->why = q8k4v_last_error(); return; }
        c->ref_dev[k] = ref_deviation(term, o);
        if (!(c->ref_dev[k] <= req_.ref_tol)) {
            c->verdict = "rejected";
            c->gate = "oracle";
            c->why = "reference term " + std::to_string(term) + ": deviation " + fmt(c->ref_dev[k]) + " > ref_tol";
            return;
        }
    }
    c->cost = c->t[0] / def_t_[unit][0] + c->t[1] / def_t_[unit][1];
    c->verdict = "admitted";
}

// Measures the unit's default (its times normalise the cost, its outputs are
// the gate) and queues the structural variants.  Nothing is searched when the
// default itself is unmeasured, invalid or fails the caller's references.
void Tuner::start_unit(int unit, UnitSearch* u) {
    const int rows = rows_of(unit);
    const bool paged16 = rows == 1 || rows == 2 || rows == 4 || rows == 8 || rows == 16;
    const q8k4v_config dflt = unit_default(unit);
    const auto t0 = Clock::now();
    Cand d;
    d.cfg = dflt;
    d.stage = "default";
    for (int k = 0; k < 2 && d.verdict.empty(); ++k) {
        if (expired()) { d.verdict = "unknown"; d.why = "deadline"; break; }
        int32_t rc = time_shape(&dflt, shapes_[unit][k], &def_t_[unit][k]);
        std::vector<float> pert;
        if (rc == Q8K4V_OK) rc = output(&dflt, shapes_[unit][k], 0, &def_out_[unit][k]);
        if (rc == Q8K4V_OK) rc = output(&dflt, shapes_[unit][k], 1, &pert);
        if (rc != Q8K4V_OK) { d.verdict = "invalid"; d.why = q8k4v_last_error(); break; }
        double peak = 0;
        for (float x : def_out_[unit][k]) peak = std::max(peak, (double)std::fabs(x));
        noise_[unit][k] = std::max(max_abs_diff(def_out_[unit][k], pert.data(), pert.size()), 1e-6 * peak);
        d.t[k] = def_t_[unit][k];
        d.dev[k] = 0.0;                         // the default is the alpha gate's reference
    }
    for (int k = 0; k < 2 && d.verdict.empty(); ++k) {
        const int term = 2 * unit + k;
        if (!has_ref(term)) continue;
        std::vector<float> o;
        if (ref_output(&dflt, term, &o) != Q8K4V_OK) { d.verdict = "invalid"; d.why = q8k4v_last_error(); break; }
        d.ref_dev[k] = ref_deviation(term, o);
        if (!(d.ref_dev[k] <= req_.ref_tol)) {
            d.verdict = "rejected";
            d.gate = "oracle";
            d.why = "reference term " + std::to_string(term) + ": deviation " + fmt(d.ref_dev[k]) + " > ref_tol";
        }
    }
    if (d.verdict.empty()) {
        d.cost = 2.0;
        d.verdict = "admitted";
    }
    d.seq = seq_++;
    u->cands.push_back(d);
    u->best_i = 0;
    u->price_ms = std::chrono::duration<double, std::milli>(Clock::now() - t0).count();
    u->effort_ms = u->price_ms;
    u->active = d.verdict == "admitted";
    if (!u->active) return;
    // structural variant: the other kernel, where it runs the unit (the
    // row-block kernel takes any row count; the replicated-row kernel only
    // 1, 2, 4, 8 or 16 rows), with its own launch-shape defaults
    std::vector<int> variants;
    if (paged16) variants.push_back(5);
    for (int v : variants) {
        Cand c;
        c.cfg = dflt;
        c.cfg.variant = v;
        c.cfg.waves_per_wg = c.cfg.stages = 0;
        if (unit != 2) c.cfg.wgs_per_cu = 0;     // the cascade's suffix keeps its finer default split
        c.stage = "structural";
        u->queue.push_back(c);
    }
    u->generated = (int)u->queue.size();
}

// Queues the refinement of the launch shape around the best candidate so far.
void Tuner::refine_queue(int unit, UnitSearch* u) {
    u->refined = true;
    const bool paged16 = [&] { const int r = rows_of(unit); return r == 1 || r == 2 || r == 4 || r == 8 || r == 16; }();
    const q8k4v_config base = u->cands[u->best_i].cfg;
    const bool base_paged = base.variant == 4 || (base.variant == 0 && paged16);
    auto push = [&](const q8k4v_config& c) {
        Cand x;
        x.cfg = c;
        x.stage = "refine";
        u->queue.push_back(x);
        ++u->generated;
    };
    // launch shapes both kernels accept: 2, 4 or 8 waves, 2 or 3 stages; one
    // 8-wave workgroup fills a CU's LDS, so 8 waves take one or two per CU.
    // The cascade's suffix pass (unit 2) merges in the cascade's own combine
    // (no in-launch merge) and takes finer splits over ragged sessions.
    for (int fused : {0, 1})
        for (int stages : {2, 3})
            for (int waves : {4, 8, 2})
                for (int wgs : {1, 2, 3, 4, 6, 8}) {
                    if (unit == 2 && fused) continue;
                    if (unit != 2 && wgs == 8) continue;
                    if (waves == 8 && wgs > 2) continue;
                    if (!base_paged && waves == 2 && wgs > 4) continue;
                    q8k4v_config c = base;
                    c.waves_per_wg = waves;
                    c.wgs_per_cu = wgs;
                    c.stages = stages;
                    c.fused_combine = fused;
                    push(c);
                }
}

// ---- records ----------------------------------------------------------------

std::string device_identity() {
    int dev = 0, rt = 0, drv = 0;
    (void)hipGetDevice(&dev);
    hipDeviceProp_t prop;
    std::memset(&prop, 0, sizeof prop);
    (void)hipGetDeviceProperties(&prop, dev);
    (void)hipRuntimeGetVersion(&rt);
    (void)hipDriverGetVersion(&drv);
    std::string id = "arch=" + std::string(prop.gcnArchName) + ";device=" + std::string(prop.name) +
                     ";cus=" + std::to_string(prop.multiProcessorCount) + ";hip_runtime=" + std::to_string(rt) +
                     ";driver=" + std::to_string(drv) + ";library=" + q8k4v_version();
    for (auto& ch : id)
        if ((unsigned char)ch < 32 || ch == '"' || ch == '\\') ch = ' ';
    return id;
}

std::string identity_hash(const std::string& id) {   // FNV-1a, 64 bits
    uint64_t h = 1469598103934665603ull;
    for (unsigned char ch : id) {
        h ^= ch;
        h *= 1099511628211ull;
    }
    char b[24];
    std::snprintf(b, sizeof b, "%016llx", (unsigned long long)h);
    return b;
}

constexpr const char* kRecordTag = "q8k4v-tune-record";

// One stored choice: identity hash, request shape (with the session count
// of the multi-session unit), unit, qualified flag and the configuration, then
// a tab and the identity in words.
struct Record {
    std::string id_hash;
    int n_draft = 0, hq = 0, hkv = 0, d = 0, ctx_small = 0, ctx_large = 0, n_sessions = 0, unit = 0, qualified = 0;
    q8k4v_config cfg{};
};

std::string record_line(const Record& r, const std::string& identity) {
    char b[512];
    std::snprintf(b, sizeof b, "%s 2 %s %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d\t%s", kRecordTag,
                  r.id_hash.c_str(), r.n_draft, r.hq, r.hkv, r.d, r.ctx_small, r.ctx_large, r.n_sessions, r.unit,
                  r.qualified, r.cfg.variant, r.cfg.wgs_per_cu, r.cfg.split_pages, r.cfg.tile_pages,
                  r.cfg.waves_per_wg, r.cfg.fused_combine, r.cfg.stages, identity.c_str());
    return b;
}

bool parse_record(const std::string& line, Record* r) {
    char tag[32] = {0}, hash[32] = {0};
    int ver = 0;
    int v[16];
    const int n = std::sscanf(line.c_str(), "%31s %d %31s %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d %d", tag, &ver,
                              hash, &v[0], &v[1], &v[2], &v[3], &v[4], &v[5], &v[6], &v[7], &v[8], &v[9], &v[10],
                              &v[11], &v[12], &v[13], &v[14], &v[15]);
    if (n != 19 || std::strcmp(tag, kRecordTag) != 0 || ver != 2 || std::strlen(hash) != 16) return false;
    r->id_hash = hash;
    r->n_draft = v[0]; r->hq = v[1]; r->hkv = v[2]; r->d = v[3]; r->ctx_small = v[4]; r->ctx_large = v[5];
    r->n_sessions = v[6]; r->unit = v[7]; r->qualified = v[8];
    std::memset(&r->cfg, 0, sizeof r->cfg);
    r->cfg.variant = v[9]; r->cfg.wgs_per_cu = v[10]; r->cfg.split_pages = v[11]; r->cfg.tile_pages = v[12];
    r->cfg.waves_per_wg = v[13]; r->cfg.fused_combine = v[14]; r->cfg.stages = v[15];
    r->cfg.qualified = r->qualified;
    return r->unit >= 0 && r->unit < kUnits;
}

std::vector<std::string> read_lines(const char* path) {
    std::vector<std::string> lines;
    std::ifstream f(path);
    std::string line;
    while (f && std::getline(f, line)) lines.push_back(line);
    return lines;
}

int32_t Tuner::run(q8k4v_config* out_table, std::string* report) {
    const auto t0 = Clock::now();
    std::string why;
    g_ = req_.num_q_heads / req_.num_kv_heads;
    w_ = req_.n_draft;
    ns_ = req_.n_sessions >= 2 ? req_.n_sessions : 0;
    n_units_ = ns_ ? 3 : 2;
    for (int unit = 0; unit < n_units_; ++unit) out_table[unit] = unit_default(unit);
    // stored choice for this device identity and request shape
    const std::string identity = device_identity();
    const std::string id_hash = identity_hash(identity);
    const bool use_records = req_.record_path && req_.record_path[0];
    auto matches = [&](const Record& r) {
        return r.id_hash == id_hash && r.n_draft == req_.n_draft && r.hq == req_.num_q_heads &&
               r.hkv == req_.num_kv_heads && r.d == req_.head_dim && r.ctx_small == req_.ctx_small &&
               r.ctx_large == req_.ctx_large && r.n_sessions == ns_;
    };
    std::string record_action = "none";
    bool stored[kUnits] = {false, false, false};
    Record rec[kUnits];
    if (use_records) {
        for (const auto& line : read_lines(req_.record_path)) {
            Record r;
            if (parse_record(line, &r) && matches(r) && r.unit < n_units_) {
                rec[r.unit] = r;
                stored[r.unit] = true;
            }
        }
    }
    bool from_records = true;
    for (int unit = 0; unit < n_units_; ++unit) from_records = from_records && stored[unit];
    std::vector<Cand> cands[kUnits];
    q8k4v_config chosen[kUnits] = {out_table[0], out_table[1], out_table[n_units_ - 1]};
    bool qual[kUnits] = {false, false, false};
    bool searched = false;
    int32_t rc = Q8K4V_OK;
    if (from_records) {
        record_action = "loaded";
        for (int unit = 0; unit < n_units_; ++unit) {
            chosen[unit] = rec[unit].cfg;
            qual[unit] = rec[unit].qualified != 0;
        }
    } else {
        rc = setup(&why);
    }
    if (!from_records && rc == Q8K4V_OK && !expired()) {
        searched = true;
        UnitSearch us[kUnits];
        for (int unit = 0; unit < n_units_; ++unit) start_unit(unit, &us[unit]);
        const int limit = req_.max_candidates > 0 ? req_.max_candidates : (1 << 20);
        for (;;) {
            // the next candidate comes from the unit with the earliest virtual
            // completion time; a unit whose structural variants are done gets
            // its refinement queue first
            double share_den = 0;
            for (int unit = 0; unit < n_units_; ++unit)
                if (us[unit].active) share_den += def_t_[unit][0] + def_t_[unit][1];
            double vt[kUnits] = {-1, -1, -1};
            int pick = -1;
            for (int unit = 0; unit < n_units_; ++unit) {
                UnitSearch& u = us[unit];
                if (!u.active || (int)u.cands.size() >= limit) continue;
                if (u.queue.empty() && !u.refined) refine_queue(unit, &u);
                while (!u.queue.empty()) {    // already measured configurations are skipped
                    bool dup = false;
                    for (const auto& e : u.cands) dup = dup || same_cfg(e.cfg, u.queue.front().cfg);
                    if (!dup) break;
                    u.queue.erase(u.queue.begin());
                }
                if (u.queue.empty()) continue;
                const double share = (def_t_[unit][0] + def_t_[unit][1]) / share_den;
                const double opportunity = (double)u.queue.size() / std::max(1, u.generated);
                vt[unit] = (u.effort_ms + u.price_ms) / (share * opportunity);
                if (pick < 0 || vt[unit] < vt[pick]) pick = unit;
            }
            if (pick < 0) break;
            UnitSearch& u = us[pick];
            Cand x = u.queue.front();
            u.queue.erase(u.queue.begin());
            x.seq = seq_++;
            for (int unit = 0; unit < kUnits; ++unit) x.vt[unit] = vt[unit];
            const auto t0c = Clock::now();
            measure(pick, &x);
            const double dt = std::chrono::duration<double, std::milli>(Clock::now() - t0c).count();
            u.effort_ms += dt;
            u.price_ms = dt;
            u.cands.push_back(x);
            if (x.verdict == "admitted" && x.cost < u.cands[u.best_i].cost) u.best_i = u.cands.size() - 1;
            if (x.verdict == "unknown") {   // the deadline passed: the rest stays unmeasured
                for (int unit = 0; unit < n_units_; ++unit)
                    for (auto& q : us[unit].queue) {
                        q.verdict = "unknown";
                        q.why = "deadline";
                        us[unit].cands.push_back(q);
                    }
                break;
            }
        }
        for (int unit = 0; unit < n_units_; ++unit) {
            cands[unit] = us[unit].cands;
            if (us[unit].cands.empty()) continue;
            const Cand& b = us[unit].cands[us[unit].best_i];
            chosen[unit] = b.cfg;
            qual[unit] = b.verdict == "admitted";
        }
    }
    for (int unit = 0; unit < n_units_; ++unit) {
        out_table[unit] = chosen[unit];
        out_table[unit].qualified = qual[unit] ? 1 : 0;
        if (!qual[unit]) {
            out_table[unit] = unit_default(unit);
            out_table[unit].qualified = 0;
        }
    }
    bool install = false;
    if (req_.install && rc == Q8K4V_OK)
        for (int unit = 0; unit < n_units_; ++unit)
            if (qual[unit]) {
                const int key = unit == 0 ? 1 : unit == 1 ? req_.n_draft : kTunedCascadeKey;
                tuned_install(key, req_.num_q_heads, req_.num_kv_heads, req_.head_dim, out_table[unit]);
                install = true;
            }
    // store a completed search (records of other identities and shapes stay)
    if (use_records && searched) {
        std::vector<std::string> keep;
        for (const auto& line : read_lines(req_.record_path)) {
            Record r;
            if (parse_record(line, &r) && !matches(r)) keep.push_back(line);
        }
        for (int unit = 0; unit < n_units_; ++unit) {
            Record r;
            r.id_hash = id_hash;
            r.n_draft = req_.n_draft; r.hq = req_.num_q_heads; r.hkv = req_.num_kv_heads; r.d = req_.head_dim;
            r.ctx_small = req_.ctx_small; r.ctx_large = req_.ctx_large; r.n_sessions = ns_;
            r.unit = unit;
            r.qualified = qual[unit] ? 1 : 0;
            r.cfg = out_table[unit];
            keep.push_back(record_line(r, identity));
        }
        const std::string tmp = std::string(req_.record_path) + ".tmp";
        bool ok;
        {
            std::ofstream f(tmp, std::ios::trunc);
            for (const auto& line : keep) f << line << "\n";
            ok = (bool)f;
        }
        ok = ok && std::rename(tmp.c_str(), req_.record_path) == 0;
        record_action = ok ? "stored" : "unwritable";
    }
    const double elapsed = std::chrono::duration<double, std::milli>(Clock::now() - t0).count();

    std::string j = "{";
    j += "\"status\":\"" + std::string(from_records ? "stored" : (searched ? "searched" : "defaults")) + "\"";
    j += ",\"budget_ms\":" + std::to_string(std::min<int64_t>(req_.budget_ms, kMaxBudgetMs));
    j += ",\"elapsed_ms\":" + fmt(elapsed);
    j += ",\"alpha\":" + fmt(kAlpha);
    if (!why.empty()) j += ",\"error\":\"" + why + "\"";
    j += ",\"rotation\":{\"copies\":" + std::to_string(n_copies_) + ",\"copy_bytes\":" + std::to_string(cache_bytes_) +
         ",\"small_page_sets\":" + std::to_string(n_sets_) + ",\"session_page_sets\":" + std::to_string(n_csets_) +
         ",\"llc_multiple\":" + fmt(llc_multiple_) + ",\"timed_replays\":" + std::to_string(reps_) +
         ",\"launches_per_replay\":[" + std::to_string(n_copies_ * n_sets_) + "," + std::to_string(n_copies_);
    if (ns_) j += "," + std::to_string(n_copies_ * n_csets_) + "," + std::to_string(n_copies_);
    j += "]}";
    if (!setup_note_.empty()) j += ",\"note\":\"" + setup_note_ + "\"";
    j += ",\"installed\":" + std::string(install ? "true" : "false");
    j += ",\"identity\":\"" + identity + "\",\"identity_hash\":\"" + id_hash + "\"";
    j += ",\"record\":\"" + record_action + "\"";
    j += ",\"units\":[";
    std::string cand_lists;
    for (int unit = 0; unit < n_units_; ++unit) {
        if (unit) j += ",";
        int n_adm = 0, n_rej = 0, n_unk = 0, n_inv = 0, n_alpha = 0, n_oracle = 0;
        std::vector<std::string> invalid_why;
        for (const auto& c : cands[unit]) {
            n_adm += c.verdict == "admitted";
            n_rej += c.verdict == "rejected";
            n_unk += c.verdict == "unknown";
            n_inv += c.verdict == "invalid";
            n_alpha += c.gate == "alpha";
            n_oracle += c.gate == "oracle";
            if (c.verdict == "invalid" && std::find(invalid_why.begin(), invalid_why.end(), c.why) == invalid_why.end())
                invalid_why.push_back(c.why);
        }
        j += "{\"unit\":\"" + std::string(unit_name(unit)) + "\"";
        j += ",\"rows_per_kv_head\":" + std::to_string(rows_of(unit));
        if (unit == 2) j += ",\"sessions\":" + std::to_string(ns_);
        j += ",\"shapes\":[\"" + shapes_[unit][0].name + "\",\"" + shapes_[unit][1].name + "\"]";
        j += ",\"default_us\":[" + fmt(def_t_[unit][0]) + "," + fmt(def_t_[unit][1]) + "]";
        j += ",\"noise\":[" + fmt(noise_[unit][0]) + "," + fmt(noise_[unit][1]) + "]";
        j += ",\"searched\":" + std::to_string(cands[unit].size());
        j += ",\"admitted\":" + std::to_string(n_adm) + ",\"rejected\":" + std::to_string(n_rej) +
             ",\"unknown\":" + std::to_string(n_unk) + ",\"invalid\":" + std::to_string(n_inv);
        j += ",\"rejected_by\":{\"alpha\":" + std::to_string(n_alpha) + ",\"oracle\":" + std::to_string(n_oracle) + "}";
        j += ",\"oracle_gate\":[" + std::string(has_ref(2 * unit) ? "true" : "false") + "," +
             std::string(has_ref(2 * unit + 1) ? "true" : "false") + "]";
        j += ",\"invalid_why\":[";
        for (size_t i = 0; i < invalid_why.size(); ++i) j += (i ? ",\"" : "\"") + json_text(invalid_why[i]) + "\"";
        j += "]";
        j += ",\"qualified\":" + std::string(qual[unit] ? "true" : "false");
        j += ",\"chosen\":" + cfg_json(out_table[unit]);
        double best_cost = 2.0, best_t0 = def_t_[unit][0], best_t1 = def_t_[unit][1];
        for (const auto& c : cands[unit])
            if (c.verdict == "admitted" && same_cfg(c.cfg, out_table[unit])) { best_cost = c.cost; best_t0 = c.t[0]; best_t1 = c.t[1]; }
        j += ",\"chosen_cost\":" + fmt(best_cost) + ",\"chosen_us\":[" + fmt(best_t0) + "," + fmt(best_t1) + "]";
        j += "}";
        cand_lists += unit ? ",[" : "[";
        for (size_t i = 0; i < cands[unit].size(); ++i) {
            const Cand& c = cands[unit][i];
            if (i) cand_lists += ",";
            cand_lists += "{\"stage\":\"" + c.stage + "\",\"cfg\":" + cfg_json(c.cfg) + ",\"verdict\":\"" + c.verdict +
                          "\",\"us\":[" + fmt(c.t[0]) + "," + fmt(c.t[1]) + "],\"dev\":[" + fmt(c.dev[0]) + "," +
                          fmt(c.dev[1]) + "],\"cost\":" + fmt(c.cost) + ",\"seq\":" + std::to_string(c.seq) +
                          ",\"vt\":[";
            for (int k = 0; k < n_units_; ++k)
                cand_lists += (k ? "," : "") + (c.vt[k] < 0 ? std::string("null") : fmt(c.vt[k]));
            cand_lists += "]";
            cand_lists += ",\"ref_dev\":[" + fmt(c.ref_dev[0]) + "," + fmt(c.ref_dev[1]) + "]";
            if (!c.gate.empty()) cand_lists += ",\"gate\":\"" + c.gate + "\"";
            if (!c.why.empty()) cand_lists += ",\"why\":\"" + json_text(c.why) + "\"";
            cand_lists += "}";
        }
        cand_lists += "]";
    }
    j += "]";
    *report = j + ",\"candidates\":[" + cand_lists + "]}";
    summary_ = j + "}";        // for a caller buffer too small for the candidate list
    error_ = why;

    for (auto& e : events_) (void)hipEventDestroy(e);
    events_.clear();
    if (stream_) {
        (void)hipStreamSynchronize(stream_);
        (void)hipStreamDestroy(stream_);
        stream_ = nullptr;
    }
    return rc == Q8K4V_ENOMEM ? Q8K4V_ENOMEM : (rc == Q8K4V_OK ? Q8K4V_OK : rc);
}

}  // namespace
}  // namespace q8k4v

using namespace q8k4v;

extern "C" int32_t tune_select(const q8k4v_tune_request* req, q8k4v_config* out_table, char* report_json,
                               size_t report_cap) {
    const auto t0 = Clock::now();
    if (!req || !out_table) return fail(Q8K4V_EINVAL, "tune_select: NULL argument");
    if (req->num_kv_heads < 1 || req->num_q_heads < 1 || req->num_q_heads % req->num_kv_heads)
        return fail(Q8K4V_EINVAL, "tune_select: num_q_heads must be a positive multiple of num_kv_heads");
    const int g = req->num_q_heads / req->num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8) return fail(Q8K4V_EUNSUPPORTED, "tune_select: group must be 1, 2, 4 or 8");
    if (req->head_dim != 64 && req->head_dim != 128) return fail(Q8K4V_EINVAL, "tune_select: head_dim must be 64 or 128");
    if (req->n_draft < 1 || req->n_draft > Q8K4V_MAX_DRAFT) return fail(Q8K4V_EINVAL, "tune_select: n_draft must be in 1..16");
    if (req->ctx_small < 1 || req->ctx_large < req->ctx_small)
        return fail(Q8K4V_EINVAL, "tune_select: need 1 <= ctx_small <= ctx_large");
    if (req->n_sessions != 0 && (req->n_sessions < 2 || req->n_sessions > kMaxSessions ||
                                 (int64_t)req->n_sessions * g > kMaxPrefixRows))
        return fail(Q8K4V_EINVAL, "tune_select: n_sessions must be 0 or 2.." + std::to_string(kMaxSessions) +
                                      " with n_sessions * group <= " + std::to_string(kMaxPrefixRows));
    for (int k = 0; k < 6; ++k) {
        const q8k4v_tune_ref& r = req->ref[k];
        if (!r.cache) continue;
        const std::string term = "tune_select: inconsistent reference inputs for term " + std::to_string(k);
        if (!r.q || !r.page_table || !r.out || r.max_pages < 1 || (int64_t)r.max_pages * Q8K4V_PAGE_SIZE < r.len)
            return fail(Q8K4V_EINVAL, term);
        if (k < 4) {
            if (r.len < (k >= 2 ? req->n_draft : 1)) return fail(Q8K4V_EINVAL, term);
            continue;
        }
        if (req->n_sessions == 0)
            return fail(Q8K4V_EINVAL, "tune_select: a multi-session reference (term " + std::to_string(k) +
                                          ") needs n_sessions >= 2");
        if (!r.seq_lens || r.n_seqs < 1 || (int64_t)r.n_seqs * g > kMaxPrefixRows || r.n_prefix_pages < 1 ||
            r.n_prefix_pages > r.max_pages || (int64_t)r.n_prefix_pages * Q8K4V_PAGE_SIZE > r.len)
            return fail(Q8K4V_EINVAL, term);
    }
    const int64_t budget = std::max<int64_t>(0, std::min<int64_t>(req->budget_ms, kMaxBudgetMs));
    Tuner t(*req, t0 + std::chrono::milliseconds(budget));
    std::string report;
    const int32_t rc = t.run(out_table, &report);
    if (report_json && report_cap) {
        const std::string& r = report.size() < report_cap ? report : t.summary();
        std::snprintf(report_json, report_cap, "%s", r.c_str());
    }
    if (rc == Q8K4V_ENOMEM) return fail(Q8K4V_ENOMEM, "tune_select: " + t.error());
    return rc;
}
