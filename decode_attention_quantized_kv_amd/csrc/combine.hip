// Launchers of the separate split-merge kernels of attn_common.h: the
// log-sum-exp combine of one launch's split records (when the in-launch
// merge is off) and the two-source combine of the shared-prefix cascade.
#include "attn_common.h"
#include "q8k4v_internal.h"

namespace q8k4v {
namespace {

template <int D>
hipError_t launch_combine_t(const AttnParams& kp, hipStream_t stream) {
    const int blocks = kp.n_seqs * kp.H * kp.R;        // one workgroup per output row
    hipLaunchKernelGGL((combine_kernel<D>), dim3(blocks), dim3(256), 0, stream, kp);
    return hipGetLastError();
}

template <int D>
hipError_t launch_combine_cascade_t(const AttnParams& kp, hipStream_t stream) {
    const int blocks = kp.n_seqs * kp.H * kp.R;        // one workgroup per (session, q head)
    hipLaunchKernelGGL((combine_cascade_kernel<D>), dim3(blocks), dim3(256), 0, stream, kp);
    return hipGetLastError();
}

}  // namespace

int32_t launch_combine(const AttnParams& kp, int head_dim, int rows_per_wg, hipStream_t stream) {
    (void)rows_per_wg;
    const hipError_t e = head_dim == 128 ? launch_combine_t<128>(kp, stream) : launch_combine_t<64>(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
    return Q8K4V_OK;
}

int32_t launch_combine_cascade(const AttnParams& kp, int head_dim, hipStream_t stream) {
    const hipError_t e = head_dim == 128 ? launch_combine_cascade_t<128>(kp, stream) : launch_combine_cascade_t<64>(kp, stream);
    if (e != hipSuccess) return hip_fail(e, "cascade combine kernel launch");
    return Q8K4V_OK;
}

}  // namespace q8k4v
