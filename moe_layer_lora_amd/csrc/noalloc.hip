// noalloc.hip - moe_route_noalloc: the routing call for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation). Its kernels need a workspace (the
// per-block expert histogram and the per-(block, expert) bases); here it is a
// file-scope device array instead of a caller buffer.
#include <mutex>

#include "moe.h"
#include "api_internal.hpp"

#include <hip/hip_runtime.h>

namespace {

// The routing workspace never exceeds 2 x 65536 int32: the top-k kernel's
// token blocks are sized so that the [blocks x E] histogram has at most
// 65536 entries, for every problem the library accepts (E <= 1024).
constexpr size_t kScratchBytes = 2 * 65536 * sizeof(int32_t);  // 512 KiB per GPU
static __device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

// Each GPU holds its own copy of `scratch` at its own address. Host code never
// uses the array's name as an address (in host code it is a host-side
// stand-in): it looks the device address up once per device, with that device
// current, and keeps it here.
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

hipError_t device_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" moe_status_t moe_route_noalloc(const moe_problem_t *pb, const float *logits, const moe_routing_t *rt,
                                          int32_t *host_counts, void *stream, const moe_trace_t *trace) {
    size_t need = 0;
    const moe_status_t st = moe::api::route_check(pb, logits, rt, &need);
    if (st != MOE_OK) return st;
    if (need > kScratchBytes) return MOE_E_UNSUPPORTED;
    // a copy to pageable memory would stage through runtime-allocated memory
    if (host_counts && !moe::api::pinned_host(host_counts)) return MOE_E_ARG;
    void *ws = nullptr;
    if (device_scratch(&ws) != hipSuccess) return MOE_E_HIP;
    // nothing in the scratch has to start at zero: the top-k kernel writes
    // every histogram entry and the scan every base before they are read
    return moe::api::route_impl(pb, logits, rt, host_counts, ws, stream, trace);
}
