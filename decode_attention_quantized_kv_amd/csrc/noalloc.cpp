// attn_decode_q8k4v_noalloc: the decode entry point for callers that cannot
// allocate device memory.  Its workspace (the header with the in-launch
// merge's arrival counters, then the split records) is this file-scope
// device array: one copy per GPU, held until the process ends.  Host code
// never uses the array's name as an address -- in host code it is a
// host-side stand-in -- but the device address hipGetSymbolAddress returns,
// looked up once per device with that device current.  Contract:
// include/q8k4v.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

static __device__ __align__(256) uint8_t scratch[Q8K4V_NOALLOC_SCRATCH_BYTES];

__global__ void zero_words_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// Device address of the current device's array.  The first call on a device
// clears the header with a fill kernel on `stream`, ahead of the call's own
// launches (a kernel rather than a memset, so the call may be captured in a
// graph).  Every completed launch leaves the counters at zero again.
int32_t scratch_address(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "attn_decode_q8k4v_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(Q8K4V_EUNSUPPORTED, "attn_decode_q8k4v_noalloc: device index above 63");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "attn_decode_q8k4v_noalloc: hipGetSymbolAddress");
        if (!ptr) return fail(Q8K4V_EHIP, "attn_decode_q8k4v_noalloc: hipGetSymbolAddress returned NULL");
        hipLaunchKernelGGL(zero_words_kernel, dim3(16), dim3(256), 0, stream, (uint32_t*)ptr,
                           (int)(Q8K4V_WS_HEADER_BYTES / sizeof(uint32_t)));
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "attn_decode_q8k4v_noalloc: header clear");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return Q8K4V_OK;
}

}  // namespace
}  // namespace q8k4v

using namespace q8k4v;

extern "C" int32_t attn_decode_q8k4v_noalloc(const q8k4v_cache* cache, const void* q, int32_t q_dtype, float* out,
                                             int32_t n_seqs, int32_t num_q_heads, const int32_t* seq_lens,
                                             int32_t max_seq_len, const int32_t* page_table, int32_t max_pages,
                                             float softmax_scale, const q8k4v_config* cfg, hipStream_t stream) {
    const std::string name = "attn_decode_q8k4v_noalloc";
    AttnArgs a{cache, q, q_dtype, out, n_seqs, num_q_heads, 1, seq_lens, max_seq_len, page_table, max_pages,
               softmax_scale};
    Plan plan;
    int32_t rc = make_plan(a, cfg, &plan);
    if (rc != Q8K4V_OK) return fail(rc, name + ": " + q8k4v_last_error());
    const size_t need = plan_workspace(plan);
    if (need > Q8K4V_NOALLOC_SCRATCH_BYTES)
        return fail(Q8K4V_EWORKSPACE, name + ": the launch needs " + std::to_string(need) +
                                          " bytes of scratch, more than the static " +
                                          std::to_string((size_t)Q8K4V_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    rc = scratch_address(stream, &ws);
    if (rc != Q8K4V_OK) return rc;
    return launch_attention(a, plan, ws, Q8K4V_NOALLOC_SCRATCH_BYTES, stream);
}
