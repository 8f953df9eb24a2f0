// Status strings of the C ABI; in the traced build (MOE_TRACE=1), the trace
// buffer's attach / detach calls.
#include "common.h"

#if MOE_TRACE
#include <vector>

namespace moe {
static std::vector<TraceSetter>& trace_setters() {
    static std::vector<TraceSetter> v;
    return v;
}
int trace_register(TraceSetter f) {
    trace_setters().push_back(f);
    return 0;
}
}  // namespace moe

extern "C" moe_status moe_trace_attach(void* device_buf, uint64_t bytes) {
    if (!device_buf || bytes < sizeof(moe::TraceHdr) + moe::kTraceKernels * sizeof(moe::TraceRec))
        return MOE_ERR_INVALID_ARG;
    const uint64_t region = (bytes - sizeof(moe::TraceHdr)) / sizeof(moe::TraceRec) / moe::kTraceKernels;
    const moe::TraceHdr h{(uint32_t)(region < 0xFFFFFFFFull ? region : 0xFFFFFFFFull), 0u, 0u, 0u};
    if (hipMemset(device_buf, 0, bytes) != hipSuccess) return MOE_ERR_HIP;
    if (hipMemcpy(device_buf, &h, sizeof(h), hipMemcpyHostToDevice) != hipSuccess) return MOE_ERR_HIP;
    for (moe::TraceSetter f : moe::trace_setters())
        if (f(device_buf) != 0) return MOE_ERR_HIP;
    return MOE_OK;
}

extern "C" moe_status moe_trace_detach(void) {
    for (moe::TraceSetter f : moe::trace_setters())
        if (f(nullptr) != 0) return MOE_ERR_HIP;
    return MOE_OK;
}
#endif

extern "C" const char* moe_status_string(moe_status status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_UNSUPPORTED: return "unsupported size";
        case MOE_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}
