// api.hip - the C ABI declared in include/moe.h: argument checks, workspace
// and saved-buffer layouts, and the launch sequence on the caller's stream.
#include "moe.h"
#include "kernels.hpp"
#include "api_internal.hpp"

#include <cmath>
#include <cstdint>

namespace {

using moe::Dims;

constexpr size_t kAlign = 256;
size_t al(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

size_t esize(moe_dtype_t dt) { return dt == MOE_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Checks the problem description; MOE_OK if the library supports it.
moe_status_t check_problem(const moe_problem_t *pb) {
    if (!pb) return MOE_E_ARG;
    if (pb->T < 0 || pb->E < 1 || pb->k < 1 || pb->k > pb->E || pb->d < 1 || pb->F < 1 || pb->r < 1)
        return MOE_E_ARG;
    if (pb->dtype != MOE_F32 && pb->dtype != MOE_BF16) return MOE_E_ARG;
    if (!std::isfinite(pb->lora_scale)) return MOE_E_ARG;
    if (pb->d % 8 || pb->F % 8 || pb->r % 8) return MOE_E_UNSUPPORTED;
    if (pb->E > 1024 || pb->r > 256) return MOE_E_UNSUPPORTED;
    // The kernels address every tensor through 32-bit byte offsets (buffer
    // descriptors, with 2^31 as the out-of-range sentinel), so no tensor may
    // exceed 2 GiB: the [S, max(d, 2F)] activations, the fp32 [S, 2r]
    // projections, one expert's [F, d] weight and the fp32 [T, E] logits.
    const long long S = (long long)pb->T * pb->k, es = (long long)esize(pb->dtype), lim = 1LL << 31;
    const long long wide = pb->d > 2LL * pb->F ? pb->d : 2LL * pb->F;
    if (S * wide * es > lim || S * 2LL * pb->r * 4 > lim) return MOE_E_UNSUPPORTED;
    if ((long long)pb->F * pb->d * es > lim || (long long)pb->T * pb->E * 4 > lim) return MOE_E_UNSUPPORTED;
    return MOE_OK;
}

Dims dims_of(const moe_problem_t *pb) {
    return Dims{pb->T, pb->d, pb->E, pb->k, pb->F, pb->r, pb->lora_scale};
}

// ---- layouts -----------------------------------------------------------------
struct RouteWs { size_t hist, base, total; };
RouteWs route_ws(const moe_problem_t *pb) {
    const size_t n = (size_t)pb->E * moe::route_nblk(pb->T, pb->E) * sizeof(int32_t);
    RouteWs w;
    w.hist = 0;
    w.base = al(n);
    w.total = w.base + al(n);
    return w;
}

// H last: everything before it is what an offload moves (H is rebuilt from
// G and U on the reload)
struct SavedLayout { size_t G, U, Zgu, Zd, ZguT, wZdT, Y, H, total; };
SavedLayout saved_layout(const moe_problem_t *pb, int keep) {
    const size_t S = (size_t)pb->T * pb->k, es = esize(pb->dtype);
    const bool bf = pb->dtype == MOE_BF16;
    SavedLayout l;
    size_t o = 0;
    l.G = o; o += al(S * pb->F * es);
    l.U = o; o += al(S * pb->F * es);
    l.Zgu = o; o += al(S * 2 * pb->r * sizeof(float));
    l.Zd = o; o += al(S * pb->r * sizeof(float));
    const size_t ldT = (S + 7) & ~(size_t)7;
    l.ZguT = o; if (bf) o += al(ldT * 2 * pb->r * 2);
    l.wZdT = o; if (bf) o += al(ldT * pb->r * 2);
    l.Y = o; if (keep) o += al(S * pb->d * es);
    l.H = o; o += al(S * pb->F * es);
    l.total = o;
    return l;
}

// forward workspace: what the forward needs that is not kept in `saved`
struct FwdWs { size_t H, Zgu, Zd, Y, tiles, total; };

// bf16: the grouped GEMMs' row-tile table
size_t tile_table_bytes(const moe_problem_t *pb) {
    if (pb->dtype != MOE_BF16) return 0;
    return al((1 + (size_t)moe::max_row_tiles(pb->T * pb->k, pb->E, moe::kRowTile)) * 16);
}

FwdWs fwd_ws(const moe_problem_t *pb, int training, int keep) {
    const size_t S = (size_t)pb->T * pb->k, es = esize(pb->dtype);
    FwdWs w{0, 0, 0, 0, 0, 0};
    size_t o = 0;
    if (!training) {
        w.H = o; o += al(S * pb->F * es);
        w.Zgu = o; o += al(S * 2 * pb->r * sizeof(float));
        w.Zd = o; o += al(S * pb->r * sizeof(float));
    }
    if (!training || !keep) { w.Y = o; o += al(S * pb->d * es); }
    w.tiles = o; o += tile_table_bytes(pb);
    w.total = o;
    return w;
}

struct BwdWs { size_t Pd, Pgu, wPdT, PguT, w_row, dGU, dXp, partial, tiles, ppart, total; };
BwdWs bwd_ws(const moe_problem_t *pb) {
    const size_t S = (size_t)pb->T * pb->k, es = esize(pb->dtype);
    const bool bf = pb->dtype == MOE_BF16;
    BwdWs w;
    size_t o = 0;
    w.Pd = o; o += al(S * pb->r * sizeof(float));
    w.Pgu = o; o += al(S * 2 * pb->r * sizeof(float));
    const size_t ldT = (S + 7) & ~(size_t)7;
    w.wPdT = o; if (bf) o += al(ldT * pb->r * 2);
    w.PguT = o; if (bf) o += al(ldT * 2 * pb->r * 2);
    w.w_row = o; o += al(S * sizeof(float));
    w.dGU = o; o += al(S * 2 * pb->F * es);
    w.dXp = o; o += al(S * pb->d * es);
    w.partial = o; o += al(moe::lora_grad_partial_bytes(dims_of(pb)));
    w.tiles = o; o += tile_table_bytes(pb);
    w.ppart = o; if (bf && moe::pgu_in_down_bwd(pb->r)) o += al(moe::pgu_part_bytes(dims_of(pb)));
    w.total = o;
    return w;
}

char *at(void *base, size_t off) { return static_cast<char *>(base) + off; }
const char *at(const void *base, size_t off) { return static_cast<const char *>(base) + off; }

// counts and offsets always; the per-slot arrays only when T > 0 (NULL is
// accepted for an empty batch, where they have no elements)
bool routing_ok(const moe_routing_t *rt, int T) {
    if (!rt || !rt->counts || !rt->offsets || !aligned16(rt->counts) || !aligned16(rt->offsets)) return false;
    const void *p[4] = {rt->topk_idx, rt->topk_w, rt->sorted_slot, rt->slot_row};
    for (const void *q : p)
        if ((T > 0 && !q) || !aligned16(q)) return false;
    return true;
}

bool weights_ok(const moe_weights_t *w) {
    if (!w) return false;
    const void *p[9] = {w->w_gate, w->w_up, w->w_down, w->a_gate, w->b_gate, w->a_up, w->b_up, w->a_down, w->b_down};
    for (const void *q : p)
        if (!q || !aligned16(q)) return false;
    return true;
}

// the LoRA factors (the base-weight pointers are not read when the base is NF4)
bool lora_ok(const moe_weights_t *w) {
    if (!w) return false;
    const void *p[6] = {w->a_gate, w->b_gate, w->a_up, w->b_up, w->a_down, w->b_down};
    for (const void *q : p)
        if (!q || !aligned16(q)) return false;
    return true;
}

// NF4 base weights: supported shapes and pointers (MOE_OK or the error)
moe_status_t nf4_ok(const moe_problem_t *pb, const moe_nf4_base_t *q) {
    if (pb->dtype != MOE_BF16 || pb->d % 64 || pb->F % 64) return MOE_E_UNSUPPORTED;
    if (!q) return MOE_E_ARG;
    const void *c[3] = {q->codes_gate, q->codes_up, q->codes_down};
    for (const void *p : c)
        if (!p || !aligned16(p)) return MOE_E_ARG;
    const void *sc[3] = {q->scales_gate, q->scales_up, q->scales_down};
    for (const void *p : sc)
        if (!p || ((uintptr_t)p & 3u)) return MOE_E_ARG;
    // per-expert code and scale slices are addressed with 32-bit byte offsets
    const long long codes = (long long)pb->F * pb->d / 2;
    if (codes > (1LL << 31)) return MOE_E_UNSUPPORTED;
    return MOE_OK;
}

bool grads_ok(const moe_lora_grads_t *g) {
    if (!g) return false;
    const void *p[6] = {g->da_gate, g->db_gate, g->da_up, g->db_up, g->da_down, g->db_down};
    for (const void *q : p)
        if (!q || !aligned16(q)) return false;
    return true;
}

bool buf_ok(const void *p) { return p && aligned16(p); }

moe::Trace to_trace(const moe_trace_t *t) {
    moe::Trace tr{};
    if (t)
        for (int i = 0; i < MOE_K_COUNT; ++i) {
            tr.start[i] = static_cast<hipEvent_t>(t->start[i]);
            tr.stop[i] = static_cast<hipEvent_t>(t->stop[i]);
        }
    return tr;
}

struct Rec {  // event pair around one launch, if the caller asked for it
    const moe::Trace *tr; int id; hipStream_t st;
    Rec(const moe::Trace *t, int i, hipStream_t s) : tr(t), id(i), st(s) {
        if (tr && tr->start[id] && tr->stop[id]) (void)hipEventRecord(tr->start[id], st);
    }
    ~Rec() { if (tr && tr->start[id] && tr->stop[id]) (void)hipEventRecord(tr->stop[id], st); }
};

}  // namespace

extern "C" {

const char *moe_status_str(moe_status_t st) {
    switch (st) {
    case MOE_OK: return "ok";
    case MOE_E_ARG: return "invalid argument";
    case MOE_E_UNSUPPORTED: return "unsupported problem";
    case MOE_E_WORKSPACE: return "workspace too small";
    case MOE_E_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t moe_route_workspace(const moe_problem_t *pb) {
    return check_problem(pb) == MOE_OK ? route_ws(pb).total : 0;
}

size_t moe_fwd_workspace(const moe_problem_t *pb, int training, int keep_expert_out) {
    return check_problem(pb) == MOE_OK ? fwd_ws(pb, training != 0, keep_expert_out != 0).total : 0;
}

size_t moe_bwd_workspace(const moe_problem_t *pb) {
    return check_problem(pb) == MOE_OK ? bwd_ws(pb).total : 0;
}

size_t moe_workspace_part(const moe_problem_t *pb, int part, int training, int keep_expert_out) {
    if (check_problem(pb) != MOE_OK) return SIZE_MAX;
    switch (part) {
    case MOE_PART_Y:
        if (training && keep_expert_out) return SIZE_MAX;
        return fwd_ws(pb, training != 0, keep_expert_out != 0).Y;
    case MOE_PART_DGU: return bwd_ws(pb).dGU;
    case MOE_PART_DXP: return bwd_ws(pb).dXp;
    }
    return SIZE_MAX;
}

size_t moe_saved_bytes(const moe_problem_t *pb, int keep_expert_out) {
    return check_problem(pb) == MOE_OK ? saved_layout(pb, keep_expert_out != 0).total : 0;
}

}  // extern "C"

namespace moe {
namespace api {

moe_status_t problem_status(const moe_problem_t *pb) { return check_problem(pb); }

// Argument checks of a routing call, without its workspace: MOE_OK and the
// workspace bytes it needs in *ws_bytes, or the error.
moe_status_t route_check(const moe_problem_t *pb, const float *logits, const moe_routing_t *rt, size_t *ws_bytes) {
    moe_status_t st = check_problem(pb);
    if (st != MOE_OK) return st;
    if (!routing_ok(rt, pb->T)) return MOE_E_ARG;
    if (pb->T > 0 && !buf_ok(logits)) return MOE_E_ARG;
    *ws_bytes = route_ws(pb).total;
    return MOE_OK;
}

// The routing launches and the optional count copy, on a checked problem,
// with the workspace at `ws` (route_check's bytes).
moe_status_t route_impl(const moe_problem_t *pb, const float *logits, const moe_routing_t *rt,
                        int32_t *host_counts, void *ws, void *stream, const moe_trace_t *trace) {
    const RouteWs w = route_ws(pb);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const moe::Trace tr = to_trace(trace);
    int32_t *hist = reinterpret_cast<int32_t *>(at(ws, w.hist));
    int32_t *base = reinterpret_cast<int32_t *>(at(ws, w.base));
    // The one device->host crossing. Page-locked memory that the device
    // reaches at its host address (the usual case for hipHostMalloc) takes
    // the counts from the scan kernel's own stores, so no copy is enqueued;
    // other host memory gets a copy after the routing kernels (asynchronous
    // for page-locked memory; the runtime completes a copy to pageable
    // memory before returning).
    int32_t *mapped_counts = nullptr;
    if (host_counts) {
        hipPointerAttribute_t pa{};
        if (hipPointerGetAttributes(&pa, host_counts) == hipSuccess) {
            if (pa.type == hipMemoryTypeHost && pa.devicePointer == host_counts) mapped_counts = host_counts;
        } else {
            (void)hipGetLastError();  // pageable memory: not an error
        }
    }
    hipError_t e;
    {
        Rec r(&tr, MOE_K_ROUTE_TOPK, s);
        e = moe::launch_route_topk(logits, pb->T, pb->E, pb->k, rt->topk_idx, rt->topk_w, hist, s);
    }
    if (e != hipSuccess) return MOE_E_HIP;
    {
        Rec r(&tr, MOE_K_ROUTE_SCAN, s);
        e = moe::launch_route_scan(hist, pb->T, pb->E, pb->k, base, rt->counts, rt->offsets, mapped_counts, s);
    }
    if (e != hipSuccess) return MOE_E_HIP;
    {
        Rec r(&tr, MOE_K_ROUTE_SCATTER, s);
        e = moe::launch_route_scatter(rt->topk_idx, base, pb->T, pb->E, pb->k, rt->sorted_slot, rt->slot_row, s);
    }
    if (e != hipSuccess) return MOE_E_HIP;
    if (host_counts && !mapped_counts &&
        hipMemcpyAsync(host_counts, rt->counts, (size_t)pb->E * sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
            hipSuccess)
        return MOE_E_HIP;
    return MOE_OK;
}

// true if p is page-locked host memory (pageable memory is not an error to
// leave for the next call)
bool pinned_host(const void *p) {
    hipPointerAttribute_t pa{};
    if (hipPointerGetAttributes(&pa, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return pa.type == hipMemoryTypeHost;
}

SavedParts saved_parts(const moe_problem_t *pb, int keep) {
    const SavedLayout l = saved_layout(pb, keep != 0);
    return SavedParts{l.Zgu, l.H};
}

// bytes [lo, hi) of `saved` to or from the same offsets of `host`, on s
moe_status_t saved_copy_range(void *saved, void *host, bool to_device, size_t lo, size_t hi, hipStream_t s) {
    if (hi <= lo) return MOE_OK;
    const hipError_t e = to_device ? hipMemcpyAsync(at(saved, lo), at(host, lo), hi - lo, hipMemcpyHostToDevice, s)
                                   : hipMemcpyAsync(at(host, lo), at(saved, lo), hi - lo, hipMemcpyDeviceToHost, s);
    return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

moe_status_t saved_rebuild_h(const moe_problem_t *pb, int keep, void *saved, hipStream_t s) {
    const SavedLayout l = saved_layout(pb, keep != 0);
    const size_t n = (size_t)pb->T * pb->k * pb->F;
    const hipError_t e =
        pb->dtype == MOE_BF16
            ? moe::run_rebuild_h<moe::bf16_t>(n, at(saved, l.G), at(saved, l.U), at(saved, l.H), s)
            : moe::run_rebuild_h<float>(n, at(saved, l.G), at(saved, l.U), at(saved, l.H), s);
    return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // namespace api
}  // namespace moe

extern "C" {

moe_status_t moe_route(const moe_problem_t *pb, const float *logits, const moe_routing_t *rt,
                       int32_t *host_counts, void *ws, size_t ws_bytes, void *stream, const moe_trace_t *trace) {
    size_t need = 0;
    const moe_status_t st = moe::api::route_check(pb, logits, rt, &need);
    if (st != MOE_OK) return st;
    if (ws_bytes < need) return MOE_E_WORKSPACE;
    if (need > 0 && !buf_ok(ws)) return MOE_E_ARG;
    return moe::api::route_impl(pb, logits, rt, host_counts, ws, stream, trace);
}

}  // extern "C"

namespace {

// moe_fwd and moe_fwd_nf4 (q4 non-null: NF4 base weights, w's base pointers unused)
moe_status_t fwd_impl(const moe_problem_t *pb, const void *x, const moe_routing_t *rt, const moe_weights_t *w,
                      const moe_nf4_base_t *q4, void *out, void *saved, int keep_expert_out, void *ws,
                      size_t ws_bytes, void *stream, const moe_trace_t *trace) {
    moe_status_t st = check_problem(pb);
    if (st != MOE_OK) return st;
    if (q4 && (st = nf4_ok(pb, q4)) != MOE_OK) return st;
    if (!routing_ok(rt, pb->T) || !(q4 ? lora_ok(w) : weights_ok(w))) return MOE_E_ARG;
    if (pb->T > 0 && (!buf_ok(x) || !buf_ok(out))) return MOE_E_ARG;
    if (saved && !aligned16(saved)) return MOE_E_ARG;
    const bool training = saved != nullptr, keep = keep_expert_out != 0;
    const FwdWs fw = fwd_ws(pb, training, keep);
    if (ws_bytes < fw.total) return MOE_E_WORKSPACE;
    if (fw.total > 0 && !buf_ok(ws)) return MOE_E_ARG;
    const SavedLayout sl = saved_layout(pb, keep);
    moe::FwdBufs b{};
    b.x = x;
    b.sorted_slot = rt->sorted_slot; b.offsets = rt->offsets; b.slot_row = rt->slot_row; b.topk_w = rt->topk_w;
    b.wg = w->w_gate; b.wu = w->w_up; b.wd = w->w_down; b.ag = w->a_gate; b.bg = w->b_gate;
    b.au = w->a_up; b.bu = w->b_up; b.ad = w->a_down; b.bd = w->b_down;
    if (training) {
        b.G = at(saved, sl.G); b.U = at(saved, sl.U); b.H = at(saved, sl.H);
        b.Zgu = reinterpret_cast<float *>(at(saved, sl.Zgu));
        b.Zd = reinterpret_cast<float *>(at(saved, sl.Zd));
        if (pb->dtype == MOE_BF16) { b.ZguT = at(saved, sl.ZguT); b.wZdT = at(saved, sl.wZdT); }
        b.Y = keep ? at(saved, sl.Y) : at(ws, fw.Y);
    } else {
        b.G = nullptr; b.U = nullptr; b.H = at(ws, fw.H);
        b.Zgu = reinterpret_cast<float *>(at(ws, fw.Zgu));
        b.Zd = reinterpret_cast<float *>(at(ws, fw.Zd));
        b.Y = at(ws, fw.Y);
    }
    b.out = out;
    b.tiles = pb->dtype == MOE_BF16 ? reinterpret_cast<int32_t *>(at(ws, fw.tiles)) : nullptr;
    moe::Nf4Base qb{};
    if (q4) {
        qb = {q4->codes_gate, q4->codes_up, q4->codes_down, q4->scales_gate, q4->scales_up, q4->scales_down};
        b.q4 = &qb;
    }
    const moe::Trace tr = to_trace(trace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Dims D = dims_of(pb);
    const hipError_t e = pb->dtype == MOE_BF16 ? moe::run_fwd<moe::bf16_t>(D, b, s, trace ? &tr : nullptr)
                                               : moe::run_fwd<float>(D, b, s, trace ? &tr : nullptr);
    return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // namespace

extern "C" {

moe_status_t moe_fwd(const moe_problem_t *pb, const void *x, const moe_routing_t *rt, const moe_weights_t *w,
                     void *out, void *saved, int keep_expert_out, void *ws, size_t ws_bytes, void *stream,
                     const moe_trace_t *trace) {
    return fwd_impl(pb, x, rt, w, nullptr, out, saved, keep_expert_out, ws, ws_bytes, stream, trace);
}

moe_status_t moe_fwd_nf4(const moe_problem_t *pb, const void *x, const moe_routing_t *rt, const moe_weights_t *w,
                         const moe_nf4_base_t *q4, void *out, void *saved, int keep_expert_out, void *ws,
                         size_t ws_bytes, void *stream, const moe_trace_t *trace) {
    if (!q4) return MOE_E_ARG;
    return fwd_impl(pb, x, rt, w, q4, out, saved, keep_expert_out, ws, ws_bytes, stream, trace);
}

}  // extern "C"

namespace {

// moe_bwd and moe_bwd_nf4 (q4 non-null: NF4 base weights)
moe_status_t bwd_impl(const moe_problem_t *pb, const void *x, const void *dout, const moe_routing_t *rt,
                      const moe_weights_t *w, const moe_nf4_base_t *q4, const void *saved, int keep_expert_out,
                      void *dx, const moe_lora_grads_t *grads, float *d_topk_w, float *d_logits, void *ws,
                      size_t ws_bytes, void *stream, const moe_trace_t *trace) {
    moe_status_t st = check_problem(pb);
    if (st != MOE_OK) return st;
    if (q4 && (st = nf4_ok(pb, q4)) != MOE_OK) return st;
    if (!routing_ok(rt, pb->T) || !(q4 ? lora_ok(w) : weights_ok(w)) || !grads_ok(grads) || !buf_ok(saved))
        return MOE_E_ARG;
    if (pb->T > 0 && (!buf_ok(x) || !buf_ok(dout) || !buf_ok(dx))) return MOE_E_ARG;
    const bool keep = keep_expert_out != 0;
    if ((d_topk_w || d_logits) && !keep) return MOE_E_ARG;
    if ((d_topk_w && !aligned16(d_topk_w)) || (d_logits && !aligned16(d_logits))) return MOE_E_ARG;
    const BwdWs bw = bwd_ws(pb);
    if (ws_bytes < bw.total) return MOE_E_WORKSPACE;
    if (!buf_ok(ws)) return MOE_E_ARG;
    const SavedLayout sl = saved_layout(pb, keep);
    moe::BwdBufs b{};
    b.x = x; b.dout = dout;
    b.sorted_slot = rt->sorted_slot; b.offsets = rt->offsets; b.slot_row = rt->slot_row; b.topk_idx = rt->topk_idx;
    b.topk_w = rt->topk_w;
    b.wg = w->w_gate; b.wu = w->w_up; b.wd = w->w_down; b.ag = w->a_gate; b.bg = w->b_gate;
    b.au = w->a_up; b.bu = w->b_up; b.ad = w->a_down; b.bd = w->b_down;
    b.G = at(saved, sl.G); b.U = at(saved, sl.U); b.H = at(saved, sl.H);
    b.Y = keep ? at(saved, sl.Y) : nullptr;
    b.Zgu = reinterpret_cast<const float *>(at(saved, sl.Zgu));
    b.Zd = reinterpret_cast<const float *>(at(saved, sl.Zd));
    b.Pd = reinterpret_cast<float *>(at(ws, bw.Pd));
    b.Pgu = reinterpret_cast<float *>(at(ws, bw.Pgu));
    if (pb->dtype == MOE_BF16) {
        b.ZguT = at(saved, sl.ZguT); b.wZdT = at(saved, sl.wZdT);
        b.wPdT = at(ws, bw.wPdT); b.PguT = at(ws, bw.PguT);
    }
    b.w_row = reinterpret_cast<float *>(at(ws, bw.w_row));
    b.dGU = at(ws, bw.dGU); b.dXp = at(ws, bw.dXp);
    b.partial = reinterpret_cast<float *>(at(ws, bw.partial));
    b.dx = dx;
    b.da_g = grads->da_gate; b.db_g = grads->db_gate; b.da_u = grads->da_up; b.db_u = grads->db_up;
    b.da_d = grads->da_down; b.db_d = grads->db_down;
    b.d_topk_w = d_topk_w; b.d_logits = d_logits;
    b.tiles = pb->dtype == MOE_BF16 ? reinterpret_cast<int32_t *>(at(ws, bw.tiles)) : nullptr;
    b.ppart = pb->dtype == MOE_BF16 && moe::pgu_in_down_bwd(pb->r) ? reinterpret_cast<float *>(at(ws, bw.ppart))
                                                                    : nullptr;
    moe::Nf4Base qb{};
    if (q4) {
        qb = {q4->codes_gate, q4->codes_up, q4->codes_down, q4->scales_gate, q4->scales_up, q4->scales_down};
        b.q4 = &qb;
    }
    const moe::Trace tr = to_trace(trace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Dims D = dims_of(pb);
    const hipError_t e = pb->dtype == MOE_BF16 ? moe::run_bwd<moe::bf16_t>(D, b, s, trace ? &tr : nullptr)
                                               : moe::run_bwd<float>(D, b, s, trace ? &tr : nullptr);
    return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // namespace

extern "C" {

moe_status_t moe_bwd(const moe_problem_t *pb, const void *x, const void *dout, const moe_routing_t *rt,
                     const moe_weights_t *w, const void *saved, int keep_expert_out, void *dx,
                     const moe_lora_grads_t *grads, float *d_topk_w, float *d_logits, void *ws, size_t ws_bytes,
                     void *stream, const moe_trace_t *trace) {
    return bwd_impl(pb, x, dout, rt, w, nullptr, saved, keep_expert_out, dx, grads, d_topk_w, d_logits, ws,
                    ws_bytes, stream, trace);
}

moe_status_t moe_bwd_nf4(const moe_problem_t *pb, const void *x, const void *dout, const moe_routing_t *rt,
                         const moe_weights_t *w, const moe_nf4_base_t *q4, const void *saved, int keep_expert_out,
                         void *dx, const moe_lora_grads_t *grads, float *d_topk_w, float *d_logits, void *ws,
                         size_t ws_bytes, void *stream, const moe_trace_t *trace) {
    if (!q4) return MOE_E_ARG;
    return bwd_impl(pb, x, dout, rt, w, q4, saved, keep_expert_out, dx, grads, d_topk_w, d_logits, ws, ws_bytes,
                    stream, trace);
}

size_t moe_router_workspace(const moe_problem_t *pb) {
    if (check_problem(pb) != MOE_OK || pb->E % 8) return 0;
    const moe::RouterWs w = moe::router_ws(dims_of(pb));
    return al(w.dlT_bytes) + al(w.partial_bytes);
}

moe_status_t moe_router_fwd(const moe_problem_t *pb, const void *x, const void *w_router, float *logits,
                            void *stream, const moe_trace_t *trace) {
    moe_status_t st = check_problem(pb);
    if (st != MOE_OK) return st;
    if (pb->E % 8) return MOE_E_UNSUPPORTED;
    if (!buf_ok(w_router)) return MOE_E_ARG;
    if (pb->T > 0 && (!buf_ok(x) || !buf_ok(logits))) return MOE_E_ARG;
    if ((long long)pb->T * pb->d >= (1LL << 31) || (long long)pb->E * pb->d * esize(pb->dtype) > (1LL << 31))
        return MOE_E_UNSUPPORTED;
    const moe::Trace tr = to_trace(trace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Dims D = dims_of(pb);
    const hipError_t e = pb->dtype == MOE_BF16
                             ? moe::run_router_fwd<moe::bf16_t>(D, x, w_router, logits, s, trace ? &tr : nullptr)
                             : moe::run_router_fwd<float>(D, x, w_router, logits, s, trace ? &tr : nullptr);
    return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

moe_status_t moe_router_bwd(const moe_problem_t *pb, const void *x, const void *w_router, const float *d_logits,
                            const void *dx_in, void *dx, float *dw_router, void *ws, size_t ws_bytes,
                            void *stream, const moe_trace_t *trace) {
    moe_status_t st = check_problem(pb);
    if (st != MOE_OK) return st;
    if (pb->E % 8) return MOE_E_UNSUPPORTED;
    if (!buf_ok(w_router)) return MOE_E_ARG;
    if ((long long)pb->T * pb->d >= (1LL << 31) ||
        (long long)pb->E * ((pb->T + 7) & ~7) * esize(pb->dtype) > (1LL << 31) ||
        (long long)pb->E * pb->d * esize(pb->dtype) > (1LL << 31))
        return MOE_E_UNSUPPORTED;
    if (pb->T > 0 && (dx || dw_router) && (!buf_ok(x) || !buf_ok(d_logits))) return MOE_E_ARG;
    if (dx && pb->T > 0 && (!buf_ok(dx) || !buf_ok(dx_in))) return MOE_E_ARG;
    if (dw_router && !buf_ok(dw_router)) return MOE_E_ARG;
    const Dims D = dims_of(pb);
    const moe::RouterWs w = moe::router_ws(D);
    void *dlT = nullptr, *partial = nullptr;
    if (dw_router) {
        const size_t need = al(w.dlT_bytes) + al(w.partial_bytes);
        if (ws_bytes < need) return MOE_E_WORKSPACE;
        if (need > 0 && !buf_ok(ws)) return MOE_E_ARG;
        dlT = ws;
        partial = w.partial_bytes ? at(ws, al(w.dlT_bytes)) : nullptr;
    }
    const moe::Trace tr = to_trace(trace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e =
        pb->dtype == MOE_BF16
            ? moe::run_router_bwd<moe::bf16_t>(D, x, w_router, d_logits, dx_in, dx, dw_router, dlT, partial, s,
                                               trace ? &tr : nullptr)
            : moe::run_router_bwd<float>(D, x, w_router, d_logits, dx_in, dx, dw_router, dlT, partial, s,
                                         trace ? &tr : nullptr);
    return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

size_t moe_saved_host_bytes(const moe_problem_t *pb, int keep_expert_out) {
    if (check_problem(pb) != MOE_OK) return 0;
    return saved_layout(pb, keep_expert_out != 0).H;
}

moe_status_t moe_saved_copy(const moe_problem_t *pb, int keep_expert_out, int to_device, void *saved, void *host,
                            void *wait_event, void *copy_stream, void *done_event) {
    moe_status_t st = check_problem(pb);
    if (st != MOE_OK) return st;
    if (!buf_ok(saved) || !host || !moe::api::pinned_host(host)) return MOE_E_ARG;
    hipStream_t cs = static_cast<hipStream_t>(copy_stream);
    if (wait_event && hipStreamWaitEvent(cs, static_cast<hipEvent_t>(wait_event), 0) != hipSuccess)
        return MOE_E_HIP;
    const moe::api::SavedParts parts = moe::api::saved_parts(pb, keep_expert_out);
    st = moe::api::saved_copy_range(saved, host, to_device != 0, 0, parts.host_end, cs);
    if (st == MOE_OK && to_device) st = moe::api::saved_rebuild_h(pb, keep_expert_out, saved, cs);
    if (st != MOE_OK) return st;
    if (done_event && hipEventRecord(static_cast<hipEvent_t>(done_event), cs) != hipSuccess) return MOE_E_HIP;
    return MOE_OK;
}

moe_status_t moe_nf4_dequant(const uint8_t *codes, const float *scales, int64_t rows, int32_t cols, void *out,
                             void *stream) {
    if (rows < 0 || cols <= 0) return MOE_E_ARG;
    if (cols % 64) return MOE_E_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!codes || ((uintptr_t)codes & 15u) || !scales || ((uintptr_t)scales & 3u) || !buf_ok(out)) return MOE_E_ARG;
    if (rows > (int64_t(1) << 40) / cols) return MOE_E_UNSUPPORTED;
    const hipError_t e = moe::run_nf4_dequant(codes, scales, rows, cols, static_cast<moe::bf16_t *>(out),
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // extern "C"
