// api_internal.hpp - pieces of the C ABI implementation shared between its
// source files (internal to the library).
#pragma once

#include <stddef.h>

#include <hip/hip_runtime.h>

#include "moe.h"

namespace moe {
namespace api {

// MOE_OK if the library supports the problem, else the status every call
// returns for it
moe_status_t problem_status(const moe_problem_t *pb);

// Argument checks of a routing call, without its workspace: MOE_OK and the
// workspace bytes it needs in *ws_bytes, or the error.
moe_status_t route_check(const moe_problem_t *pb, const float *logits, const moe_routing_t *rt, size_t *ws_bytes);

// The routing launches and the optional count copy on `stream`, for a problem
// route_check accepted, with its workspace at `ws`.
moe_status_t route_impl(const moe_problem_t *pb, const float *logits, const moe_routing_t *rt,
                        int32_t *host_counts, void *ws, void *stream, const moe_trace_t *trace);

// true if p is page-locked host memory; pageable memory returns false and
// leaves no HIP error behind
bool pinned_host(const void *p);

// Offload of a `saved` buffer of a checked problem to pinned host memory (the
// moe_saved_host_bytes bytes before H), and its reload: those bytes back,
// then H rebuilt from G and U; both enqueued on `stream`.
moe_status_t saved_offload(const moe_problem_t *pb, int keep, const void *saved, void *host, hipStream_t stream);
moe_status_t saved_reload(const moe_problem_t *pb, int keep, void *saved, const void *host, hipStream_t stream);

}  // namespace api
}  // namespace moe
