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

// What an offload of a `saved` buffer (checked problem) moves to pinned host
// memory, as byte ranges at the same offsets on both sides: [0, gu_end) is
// G and U (final once the gate/up GEMM has run, last read by the
// down-backward GEMM), [gu_end, host_end) the rest before H (H is rebuilt
// from G and U after a reload).
struct SavedParts { size_t gu_end, host_end; };
SavedParts saved_parts(const moe_problem_t *pb, int keep);
// bytes [lo, hi) of `saved` to (to_device) or from `host`, enqueued on stream
moe_status_t saved_copy_range(void *saved, void *host, bool to_device, size_t lo, size_t hi, hipStream_t stream);
// H = silu(G) U from G and U as stored, enqueued on stream
moe_status_t saved_rebuild_h(const moe_problem_t *pb, int keep, void *saved, hipStream_t stream);

}  // namespace api
}  // namespace moe
