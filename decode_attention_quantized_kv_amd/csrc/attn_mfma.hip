// MFMA verify kernel (placeholder until the dense path lands).
#include "attn_common.h"
#include "q8k4v_internal.h"

namespace q8k4v {
int32_t launch_mfma(const AttnParams&, const Plan&, int, bool, hipStream_t) {
    return fail(Q8K4V_EUNSUPPORTED, "attention: query blocks above 8 rows are not built yet");
}
}  // namespace q8k4v
