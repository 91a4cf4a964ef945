// kernels.hpp - host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Rows per tile of the bf16 grouped GEMMs; their row-tile table lives in the
// forward and backward workspaces.
constexpr int kRowTile = 256;

// Upper bound on the number of row tiles over all experts (a launch size
// chosen before the counts are known on the host).
__host__ __device__ inline int max_row_tiles(int S, int E, int BM) { return (S + BM - 1) / BM + E; }

typedef uint16_t bf16_t;  // bf16 bit pattern in memory

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

struct Dims {
    int T, d, E, k, F, r;
    float s;  // LoRA scale
    int S() const { return T * k; }
};

// ---- routing ---------------------------------------------------------------
// tokens per routing block: keeps the [E x nblk] histogram at <= 64K entries
int route_tokens_per_block(int T, int E);
inline int route_nblk(int T, int E) {
    const int tpb = route_tokens_per_block(T, E);
    return T > 0 ? (T + tpb - 1) / tpb : 0;
}
hipError_t launch_route_topk(const float *logits, int T, int E, int k, int32_t *topk_idx, float *topk_w,
                             int32_t *hist, hipStream_t st);
// host_counts: null, or page-locked host memory the device reaches at the
// same address (the scan stores the counts there)
hipError_t launch_route_scan(const int32_t *hist, int T, int E, int k, int32_t *base, int32_t *counts,
                             int32_t *offsets, int32_t *host_counts, hipStream_t st);
hipError_t launch_route_scatter(const int32_t *topk_idx, const int32_t *base, int T, int E, int k,
                                int32_t *sorted_slot, int32_t *slot_row, hipStream_t st);

// ---- forward / backward (T = float or bf16 bits) -----------------------------
// 4-bit NormalFloat frozen weights (bf16 layers only): codes [E*rows, cols/2]
// and fp32 scales [E*rows, cols/64] of W_gate, W_up ([F, d] per expert) and
// W_down ([d, F]); the grouped GEMMs dequantise them as they stage B tiles.
struct Nf4Base {
    const uint8_t *cg, *cu, *cd;
    const float *sg, *su, *sd;
};

struct FwdBufs {
    const void *x;
    const int32_t *sorted_slot, *offsets, *slot_row;
    const float *topk_w;
    const void *wg, *wu, *wd, *ag, *bg, *au, *bu, *ad, *bd;
    void *G, *U, *H;      // G, U may be null (inference)
    float *Zgu, *Zd;      // [S,2r], [S,r]
    void *ZguT, *wZdT;    // bf16 training only: [2r,S] Zgu^T, [r,S] (w Zd)^T; else null
    void *Y;              // [S,d]
    void *out;            // [T,d]
    int32_t *tiles;       // workspace: row-tile table of the grouped GEMMs
    const Nf4Base *q4;    // non-null: base weights in NF4 (wg, wu, wd unused)
};

struct BwdBufs {
    const void *x, *dout;
    const int32_t *sorted_slot, *offsets, *slot_row, *topk_idx;
    const float *topk_w;
    const void *wg, *wu, *wd, *ag, *bg, *au, *bu, *ad, *bd;
    const void *G, *U, *H, *Y;   // saved (Y may be null)
    const float *Zgu, *Zd;       // saved
    const void *ZguT, *wZdT;     // saved (bf16 only)
    float *Pd, *Pgu;             // workspace [S,r], [S,2r]
    void *wPdT, *PguT;           // workspace (bf16 only): [r,S] (w Pd)^T, [2r,S] Pgu^T
    float *w_row;                // workspace [S]: combine weight of each row p
    void *dGU, *dXp;             // workspace [S,2F], [S,d]
    float *partial;              // workspace for LoRA-gradient partial sums
    void *dx;
    float *da_g, *db_g, *da_u, *db_u, *da_d, *db_d;
    float *d_topk_w, *d_logits;  // optional
    int32_t *tiles;              // workspace: row-tile table of the grouped GEMMs
    const Nf4Base *q4;           // non-null: base weights in NF4 (wg, wu, wd unused)
    float *ppart;                // workspace (bf16, pgu_in_down_bwd): column-strip shares of Pgu
};

// The bf16 down-backward GEMM projects its dG, dU tiles onto B_g, B_u in the
// epilogue (instead of a separate pass over dGU) for these ranks; the shares
// of its 256-column strips take pgu_part_bytes of workspace.
inline bool pgu_in_down_bwd(int r) { return r % 16 == 0 && r <= 32; }
inline size_t pgu_part_bytes(const Dims &D) { return (size_t)cdiv(D.F, 256) * D.S() * 2 * D.r * sizeof(float); }

// per-kernel timing events (hipEvent_t or null), indexed like MOE_K_*
struct Trace {
    hipEvent_t start[32], stop[32];
};

template <typename T> hipError_t run_fwd(const Dims &D, const FwdBufs &b, hipStream_t st, const Trace *tr);
template <typename T> hipError_t run_bwd(const Dims &D, const BwdBufs &b, hipStream_t st, const Trace *tr);
// H = silu(G) U over `elems` elements (a multiple of the 16-byte chunk) from
// G and U as the forward stored them, bit-identical to the forward's H
template <typename T> hipError_t run_rebuild_h(size_t elems, const void *G, const void *U, void *H, hipStream_t st);

// ---- router projection (logits = x W_r^T) and its backward ---------------------
// Workspace of the backward: d_logits transposed [E, Tp] (Tp = T rounded up
// to 8) and, when the token range is split into nch > 1 chunks, the fp32
// partial dW_r of each chunk [nch, E, d].
struct RouterWs {
    int Tp, chunk, nch;
    size_t dlT_bytes, partial_bytes;
};
RouterWs router_ws(const Dims &D);
template <typename T>
hipError_t run_router_fwd(const Dims &D, const void *x, const void *wr, float *logits, hipStream_t st,
                          const Trace *tr);
template <typename T>
hipError_t run_router_bwd(const Dims &D, const void *x, const void *wr, const float *d_logits, const void *dx_in,
                          void *dx, float *dw, void *dlT, void *partial, hipStream_t st, const Trace *tr);

// ---- 4-bit NormalFloat frozen weights -> bf16 ---------------------------------
// the 16 NF4 levels, ascending (code q -> level q)
void nf4_level_values(float out[16]);
hipError_t run_nf4_dequant(const uint8_t *codes, const float *scales, int64_t rows, int cols, bf16_t *out,
                           hipStream_t st);

// bytes of LoRA-gradient partial sums the backward may need
size_t lora_grad_partial_bytes(const Dims &D);
// leading dimension of the transposed bf16 LoRA-gradient operands [nr, ldT]
inline int lgrad_ldT(const Dims &D) { return (D.S() + 7) & ~7; }

}  // namespace moe
