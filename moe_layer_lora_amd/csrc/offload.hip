// offload.hip - a stack of MoE layers with their saved activations offloaded
// to pinned host memory in the forward and reloaded, double-buffered, in the
// backward: the checkpoint reload of the Unsloth x NVIDIA blog (section "core
// idea / structure / how it works", checkpoint paragraph), where two device
// buffers take turns so that the backward of one layer reads buffer A while
// a copy stream brings the next layer's activations back into buffer B.
//
// Host code only: it orders moe_route / moe_fwd / moe_bwd on the compute
// stream and the copies on the copy stream with the caller's four events.
// A copy moves `saved` without H, which the reload rebuilds from G and U on
// the copy stream. G and U (95% of the bytes at typical shapes) have their
// own timing: they are final as soon as the gate/up GEMM has run, and the
// down-backward GEMM is their last reader, so their copies start at those
// points instead of at the end of the call. Buffer of layer i: saved[i % 2].
//  forward,  layer i: wait until the offload of layer i - 2 has finished
//            reading saved[i % 2]; route; forward into saved[i % 2]; for
//            layers 0 .. n-3 the copy stream copies G, U to host i after
//            the gate/up GEMM and the rest after the forward.
//  backward, layer i (n-1 down to 0): layers n-1 and n-2 are still on the
//            device; a lower layer waits for its reload. The copy stream
//            reloads G, U of layer i - 2 into saved[i % 2] once layer i's
//            down-backward GEMM has run, and the rest (then rebuilds H) once
//            its whole backward has, under the backward of layer i - 1.
// The mid-call points come from the library's per-kernel event hook
// (moe_trace_t): one of the caller's events in both the start and the stop
// slot of a kernel ends up recorded right after that kernel.
#include <hip/hip_runtime.h>

#include "moe.h"
#include "api_internal.hpp"

namespace {

constexpr size_t kAlign = 256;

bool a16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }

moe_status_t hip_ok(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

// checks shared by both directions
moe_status_t check_stack(const moe_problem_t *pb, int n, const moe_stack_layer_t *layers, int keep,
                         const moe_offload_t *off, size_t ws_bytes, void *stream, bool bwd) {
    const moe_status_t pst = moe::api::problem_status(pb);
    if (pst != MOE_OK) return pst;
    const size_t ws_need = moe_stack_workspace(pb, keep);
    if (n < 1 || !layers || !off) return MOE_E_ARG;
    if (ws_bytes < ws_need) return MOE_E_WORKSPACE;
    if (!a16(off->saved[0]) || (n > 1 && !a16(off->saved[1]))) return MOE_E_ARG;
    if (n > 1 && off->saved[0] == off->saved[1]) return MOE_E_ARG;
    if (n >= 3) {
        if (off->copy_stream == stream) return MOE_E_ARG;  // the copies must run beside the compute
        for (int i = 0; i < 4; ++i)
            if (!off->events[i]) return MOE_E_ARG;
    }
    for (int i = 0; i < n; ++i) {
        const moe_stack_layer_t &L = layers[i];
        if (!L.rt || !L.w) return MOE_E_ARG;
        if (pb->T > 0 && (!a16(L.x) || (!bwd && (!a16(L.logits) || !a16(L.out)))))
            return MOE_E_ARG;
        if (bwd && (!L.grads || (pb->T > 0 && (!a16(L.dout) || !a16(L.dx))))) return MOE_E_ARG;
        if (bwd && (L.d_topk_w || L.d_logits) && !keep) return MOE_E_ARG;
        if (i <= n - 3 && (!L.host_saved || !moe::api::pinned_host(L.host_saved))) return MOE_E_ARG;
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_stack_workspace(const moe_problem_t *pb, int keep_expert_out) {
    const size_t r = moe_route_workspace(pb), f = moe_fwd_workspace(pb, 1, keep_expert_out),
                 b = moe_bwd_workspace(pb);
    if (moe::api::problem_status(pb) != MOE_OK) return 0;
    size_t m = r > f ? r : f;
    m = m > b ? m : b;
    return (m + kAlign - 1) / kAlign * kAlign;
}

moe_status_t moe_stack_fwd(const moe_problem_t *pb, int n, const moe_stack_layer_t *layers, int keep_expert_out,
                           const moe_offload_t *off, void *ws, size_t ws_bytes, void *stream) {
    moe_status_t st = check_stack(pb, n, layers, keep_expert_out, off, ws_bytes, stream, false);
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream), cs = static_cast<hipStream_t>(off->copy_stream);
    hipEvent_t fwd_done[2] = {static_cast<hipEvent_t>(off->events[0]), static_cast<hipEvent_t>(off->events[1])};
    hipEvent_t copy_done[2] = {static_cast<hipEvent_t>(off->events[2]), static_cast<hipEvent_t>(off->events[3])};
    const moe::api::SavedParts parts = moe::api::saved_parts(pb, keep_expert_out);
    for (int i = 0; i < n; ++i) {
        const moe_stack_layer_t &L = layers[i];
        void *buf = off->saved[i % 2];
        const bool offload = i <= n - 3;  // layers n-2 and n-1 stay on the device for the backward
        // the offload of layer i - 2 reads this buffer: it must finish first
        if (i >= 2 && (st = hip_ok(hipStreamWaitEvent(s, copy_done[i % 2], 0))) != MOE_OK) return st;
        if ((st = moe_route(pb, L.logits, L.rt, nullptr, ws, ws_bytes, stream, nullptr)) != MOE_OK) return st;
        moe_trace_t gu_done{};  // fwd_done[i % 2] recorded right after the gate/up GEMM
        gu_done.start[MOE_K_GATEUP] = gu_done.stop[MOE_K_GATEUP] = fwd_done[i % 2];
        if ((st = moe_fwd(pb, L.x, L.rt, L.w, L.out, buf, keep_expert_out, ws, ws_bytes, stream,
                          offload ? &gu_done : nullptr)) != MOE_OK)
            return st;
        if (offload) {
            if ((st = hip_ok(hipStreamWaitEvent(cs, fwd_done[i % 2], 0))) != MOE_OK) return st;
            if ((st = moe::api::saved_copy_range(buf, L.host_saved, false, 0, parts.gu_end, cs)) != MOE_OK) return st;
            if ((st = hip_ok(hipEventRecord(fwd_done[i % 2], s))) != MOE_OK) return st;  // the whole forward
            if ((st = hip_ok(hipStreamWaitEvent(cs, fwd_done[i % 2], 0))) != MOE_OK) return st;
            if ((st = moe::api::saved_copy_range(buf, L.host_saved, false, parts.gu_end, parts.host_end, cs)) !=
                MOE_OK)
                return st;
            if ((st = hip_ok(hipEventRecord(copy_done[i % 2], cs))) != MOE_OK) return st;
        }
    }
    return MOE_OK;
}

moe_status_t moe_stack_bwd(const moe_problem_t *pb, int n, const moe_stack_layer_t *layers, int keep_expert_out,
                           const moe_offload_t *off, void *ws, size_t ws_bytes, void *stream) {
    moe_status_t st = check_stack(pb, n, layers, keep_expert_out, off, ws_bytes, stream, true);
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream), cs = static_cast<hipStream_t>(off->copy_stream);
    hipEvent_t bwd_done[2] = {static_cast<hipEvent_t>(off->events[0]), static_cast<hipEvent_t>(off->events[1])};
    hipEvent_t copy_done[2] = {static_cast<hipEvent_t>(off->events[2]), static_cast<hipEvent_t>(off->events[3])};
    const moe::api::SavedParts parts = moe::api::saved_parts(pb, keep_expert_out);
    for (int i = n - 1; i >= 0; --i) {
        const moe_stack_layer_t &L = layers[i];
        void *buf = off->saved[i % 2];
        const bool reload = i - 2 >= 0;  // layer i - 2 comes back into this buffer
        // layers below n-2 were reloaded into their buffer: wait for the copy
        if (i <= n - 3 && (st = hip_ok(hipStreamWaitEvent(s, copy_done[i % 2], 0))) != MOE_OK) return st;
        moe_trace_t gu_free{};  // bwd_done[i % 2] recorded right after the down-backward GEMM
        gu_free.start[MOE_K_DOWN_BWD] = gu_free.stop[MOE_K_DOWN_BWD] = bwd_done[i % 2];
        if ((st = moe_bwd(pb, L.x, L.dout, L.rt, L.w, buf, keep_expert_out, L.dx, L.grads, L.d_topk_w, L.d_logits,
                          ws, ws_bytes, stream, reload ? &gu_free : nullptr)) != MOE_OK)
            return st;
        if (reload) {  // under the rest of layer i's backward and under layer i - 1's
            void *host = layers[i - 2].host_saved;
            if ((st = hip_ok(hipStreamWaitEvent(cs, bwd_done[i % 2], 0))) != MOE_OK) return st;
            if ((st = moe::api::saved_copy_range(buf, host, true, 0, parts.gu_end, cs)) != MOE_OK) return st;
            if ((st = hip_ok(hipEventRecord(bwd_done[i % 2], s))) != MOE_OK) return st;  // the whole backward
            if ((st = hip_ok(hipStreamWaitEvent(cs, bwd_done[i % 2], 0))) != MOE_OK) return st;
            if ((st = moe::api::saved_copy_range(buf, host, true, parts.gu_end, parts.host_end, cs)) != MOE_OK)
                return st;
            if ((st = moe::api::saved_rebuild_h(pb, keep_expert_out, buf, cs)) != MOE_OK) return st;
            if ((st = hip_ok(hipEventRecord(copy_done[i % 2], cs))) != MOE_OK) return st;
        }
    }
    return MOE_OK;
}

}  // extern "C"
