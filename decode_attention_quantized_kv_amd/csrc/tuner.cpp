// On-device tuner (placeholder: returns the defaults, unqualified).
#include <cstring>
#include <cstdio>
#include "q8k4v_internal.h"

using namespace q8k4v;

extern "C" int32_t tune_select(const q8k4v_tune_request* req, q8k4v_config* out_table, char* report_json,
                               size_t report_cap) {
    if (!req || !out_table) return fail(Q8K4V_EINVAL, "tune_select: NULL argument");
    out_table[0] = default_config(false);
    out_table[1] = default_config(true);
    if (report_json && report_cap) std::snprintf(report_json, report_cap, "{\"searched\":0}");
    return Q8K4V_OK;
}
