// Host-side internal interface between the C ABI, the kernel launchers and
// the tuner.  Not installed; the public interface is include/q8k4v.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "q8k4v.h"

namespace q8k4v {

// Records a message for q8k4v_last_error() and returns `code`.
int32_t fail(int32_t code, const std::string& msg);
int32_t hip_fail(hipError_t e, const char* what);

struct AppendArgs {
    const q8k4v_cache* cache;
    const void* k_new;
    const void* v_new;
    int32_t dtype;
    const int32_t* cu_new;
    const int32_t* start_pos;
    const int32_t* page_table;
    int32_t max_pages, n_seqs, total_new;
    // if set (cu_new and start_pos unused): one token per sequence, token b
    // at position last_of[b] - 1
    const int32_t* last_of;
};
int32_t launch_append(const AppendArgs& a, hipStream_t stream);

// One attention launch: decode (n_draft == 1 semantics with causal offset 0)
// or verify (n_draft drafts, causal among them).
struct AttnArgs {
    const q8k4v_cache* cache;
    const void* q;
    int32_t q_dtype;
    float* out;
    int32_t n_seqs, num_q_heads, n_draft;   // n_draft == 1 for decode
    const int32_t* seq_lens;
    int32_t max_seq_len;
    const int32_t* page_table;
    int32_t max_pages;
    float softmax_scale;
};

// The two attention kernels of attn_paged.hip, numbered as the `variant`
// field of q8k4v_config selects them.
enum Kernel { kDec2 = 4, kRows = 5 };

// Fully resolved launch plan.
struct Plan {
    int32_t rows;          // query rows per kv head = n_draft * group
    int32_t kernel;        // Kernel
    int32_t tile_pages;
    int32_t waves;
    int32_t stages;        // tile buffers per wave in the LDS ring
    int32_t rows_per_wg;   // rows handled by one workgroup (row chunk)
    int32_t row_chunks;    // workgroups per (sequence, kv head, split) along rows
    int32_t split_pages;   // pages per workgroup
    int32_t n_splits;      // workgroups per (sequence, kv head)
    int32_t fused_combine;
    size_t partial_bytes;  // split partials
    size_t counter_bytes;  // fused-combine counters
};

// Default configuration for a query block of `rows` rows per kv head (the
// automatic kernel with its launch-shape defaults); used when cfg is NULL and
// no tuned entry matches.
q8k4v_config default_config(int32_t rows);

// Resolve config + shape into a plan; returns Q8K4V_OK or an error.
int32_t make_plan(const AttnArgs& a, const q8k4v_config* cfg, Plan* plan);
size_t plan_workspace(const Plan& p);

// Arrival counters of the in-launch merge: one uint32 per (sequence, kv
// head, row chunk) at the front of the workspace header.
constexpr int64_t kMaxCounters = Q8K4V_WS_HEADER_BYTES / sizeof(uint32_t);

int32_t launch_attention(const AttnArgs& a, const Plan& plan, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

// Shared-prefix cascade: the prefix pass (row-block kernel over the shared
// pages, every session's rows), the suffix pass (the decode plan past the
// prefix) and their partial areas, prefix first.
struct CascadePlan {
    Plan pre, suf;
};
constexpr int32_t kMaxPrefixRows = 4096;
constexpr int32_t kCascadeSuffixWgsPerCu = 3;   // suffix pass, when the caller gives no config
// Default suffix-pass configuration of the cascade for `group` query heads
// per kv head (the decode defaults with kCascadeSuffixWgsPerCu).
q8k4v_config cascade_default_config(int32_t group);
// Key of the multi-session unit in the tuned table (decode is n_draft 1).
constexpr int32_t kTunedCascadeKey = 0;
int32_t make_cascade_plan(const AttnArgs& a, int32_t n_prefix_pages, const q8k4v_config* cfg, CascadePlan* cp);
size_t cascade_workspace(const CascadePlan& cp);
int32_t launch_cascade(const AttnArgs& a, int32_t n_prefix_pages, const CascadePlan& cp, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

// Tuned table (installed by tune_select), per current device and shape;
// n_draft 1 is the decode unit.  lookup returns true and fills cfg on a match.
bool tuned_lookup(int32_t n_draft, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  q8k4v_config* cfg);
void tuned_install(int32_t n_draft, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   const q8k4v_config& cfg);

int32_t device_cu_count();

}  // namespace q8k4v
