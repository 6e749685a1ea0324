// Host-only parts of the C ABI: capacity, status text, workspace sizing.
#include <math.h>

#include "moe_common.h"

size_t moe_dispatch_ws_bytes(int64_t T, int E, int k);

// C = ceil(T * k * cf / E) in double, in that order.  [P2] MoE basics page
// (dpshk.com/news/6005940) section 2.4 gives ceil(tokens / experts * cf);
// the tokens here are the T * k router assignments (equal for k = 1).
extern "C" int64_t moe_capacity(int64_t T, int k, int E, double cf) {
    if (T < 0 || k < 1 || E < 1 || !(cf > 0.0) || !isfinite(cf)) return -1;
    const double c = ceil((double)T * (double)k * cf / (double)E);
    if (!(c < 9.0e18)) return -1;
    return (int64_t)c;
}

extern "C" const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size is negative, zero or inconsistent";
        case MOE_ERR_DTYPE: return "unknown dtype, routing mode or activation";
        case MOE_ERR_UNSUPPORTED: return "arguments beyond this library's limits";
        case MOE_ERR_ALIGN: return "size or pointer alignment requirement not met";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

extern "C" size_t moe_workspace_bytes(int64_t T, int E, int k) {
    if (T < 0 || E < 1 || k < 1 || E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return 0;
    return moe_dispatch_ws_bytes(T, E, k);
}
