/*
 * moe.h - C ABI of the MI355X (gfx950) MoE expert layer with Split-LoRA.
 *
 * Three calls make up one training step of the layer:
 *
 *   moe_route  top-k routing and expert grouping. The Unsloth x NVIDIA blog
 *              (d9249.github.io, section "core idea / structure / how it
 *              works", MoE routing paragraph) replaces a per-expert where()
 *              scan with one flatten, stable sort by expert id, bincount and
 *              offset slice; this call produces exactly those four things
 *              (topk_idx flattened, sorted_slot, counts, offsets) on the GPU,
 *              with at most one device->host copy (the counts, optional).
 *   moe_fwd    the grouped expert MLP: one grouped GEMM over all experts
 *              (Unsloth 2026 wiki chapter, "Optimisation 3: grouped_mm and
 *              Split-LoRA in MoE training", grouped_mm subsection), SwiGLU
 *              h = silu(x W_g^T) * (x W_u^T), y = h W_d^T, each projection
 *              with Split-LoRA (same chapter, Split-LoRA subsection): the
 *              frozen W is applied and s * (x A^T) B^T is added, W + s B A is
 *              never formed; then the combine out[t] = sum_j w[t,j] y[t,j].
 *   moe_bwd    the backward with base W frozen, derived by hand in closed form
 *              (GPU MODE lecture 32 notes, "Unsloth - Faster, Lower-Memory LLM
 *              Fine-Tuning", part on hand-derived backward passes): dX, dA and
 *              dB of gate, up and down, and optionally the gradient of the
 *              combine weights and its chain through the top-k softmax into
 *              the logits.
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless marked (host). All tensors are
 *    row-major and contiguous. Device pointers must be 16-byte aligned.
 *  - Weights use the nn.Linear orientation [out, in], stacked over experts:
 *      w_gate, w_up [E,F,d]   w_down [E,d,F]
 *      a_gate, a_up [E,r,d]   b_gate, b_up [E,F,r]   a_down [E,r,F]   b_down [E,d,r]
 *  - A "slot" is q = t*k + j (token t, its j-th choice); S = T*k slots. A
 *    "row" p is a slot's position in expert-grouped order; expert e owns rows
 *    offsets[e] .. offsets[e+1]-1, in increasing token order.
 *  - dtype (moe_problem_t.dtype) applies to x, the weights, out, dout, dx and
 *    the activations kept in `saved`. logits, topk_w, LoRA gradients,
 *    d_topk_w and d_logits are always float32; indices are int32.
 *  - The caller owns every buffer, including workspaces (size them with the
 *    *_workspace queries) and `saved`. The library allocates no device
 *    memory, frees nothing and keeps no pointer after a call returns.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream). No call synchronises the stream. The only device->host
 *    transfer is moe_route's optional copy of the expert counts (see there).
 *  - Errors: arguments are checked on the host before anything is enqueued;
 *    on any error nothing is launched and outputs are untouched. MOE_E_HIP
 *    means a HIP call failed after checks passed (outputs then undefined).
 *    Nothing is printed and no exception crosses the ABI.
 *  - Limits: 0 <= T; 1 <= k <= E <= 1024; d, F, r >= 8 and multiples of 8;
 *    r <= 256; no tensor above 2 GiB, i.e. with S = T*k and es the element
 *    size of dtype: S*max(d,2F)*es, S*2r*4, F*d*es and T*E*4 bytes are each
 *    at most 2^31 (else MOE_E_UNSUPPORTED; the kernels use 32-bit byte
 *    offsets). Logits must be finite (NaN/Inf: undefined order).
 *  - Gradient outputs are overwritten, never accumulated into.
 *  - Calls on different streams may run concurrently if they share no
 *    buffers (workspaces included). The library keeps no state between calls
 *    (its only static data is the table of 16 NF4 levels, computed once).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_E_ARG = 1,         /* bad dimension, NULL or misaligned pointer */
    MOE_E_UNSUPPORTED = 2, /* valid but outside the limits above */
    MOE_E_WORKSPACE = 3,   /* workspace smaller than the *_workspace query */
    MOE_E_HIP = 4          /* a HIP runtime call failed */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef struct {
    int32_t T;          /* tokens */
    int32_t d;          /* model width */
    int32_t E;          /* experts */
    int32_t k;          /* experts per token */
    int32_t F;          /* expert FFN width */
    int32_t r;          /* LoRA rank */
    float lora_scale;   /* s = alpha / r */
    moe_dtype_t dtype;  /* storage of x, W, A, B, activations */
} moe_problem_t;

typedef struct {
    int32_t *topk_idx;     /* [T,k]  expert of each slot, j-th best first        */
    float *topk_w;         /* [T,k]  softmax over the k selected logits          */
    int32_t *counts;       /* [E]    slots per expert (bincount)                 */
    int32_t *offsets;      /* [E+1]  exclusive prefix of counts; offsets[E] = S  */
    int32_t *sorted_slot;  /* [S]    row p -> slot q (stable sort by expert id)  */
    int32_t *slot_row;     /* [S]    slot q -> row p (inverse permutation)       */
} moe_routing_t;

typedef struct {
    const void *w_gate, *w_up, *w_down;              /* frozen base weights      */
    const void *a_gate, *b_gate, *a_up, *b_up;       /* LoRA factors, gate / up  */
    const void *a_down, *b_down;                     /* LoRA factors, down       */
} moe_weights_t;

typedef struct {
    float *da_gate, *db_gate;   /* [E,r,d], [E,F,r] */
    float *da_up, *db_up;       /* [E,r,d], [E,F,r] */
    float *da_down, *db_down;   /* [E,r,F], [E,d,r] */
} moe_lora_grads_t;

/* Optional per-kernel timing: if a moe_trace_t is passed and start[i] and
 * stop[i] are both non-NULL hipEvent_t handles, the call records start[i]
 * before and stop[i] after kernel i on `stream`. Indices: */
enum {
    MOE_K_ROUTE_TOPK = 0,   /* top-k + softmax + per-block expert histogram */
    MOE_K_ROUTE_SCAN,       /* exclusive scan -> counts, offsets, bases     */
    MOE_K_ROUTE_SCATTER,    /* stable scatter -> sorted_slot, slot_row      */
    MOE_K_PROJ_GU,          /* LoRA A projection of x (gate|up)             */
    MOE_K_GATEUP,           /* grouped GEMM gate/up + LoRA + SwiGLU         */
    MOE_K_PROJ_D,           /* LoRA A projection of h (down)                */
    MOE_K_DOWN,             /* grouped GEMM down + LoRA                     */
    MOE_K_COMBINE,          /* weighted combine -> out                      */
    MOE_K_ROUTER_GRAD,      /* d_topk_w, d_logits                           */
    MOE_K_PROJ_DOUT,        /* dout B_down projection                       */
    MOE_K_DOWN_BWD,         /* grouped GEMM dH + LoRA + SwiGLU backward     */
    MOE_K_PROJ_DGU,         /* dG B_gate | dU B_up projection               */
    MOE_K_GATEUP_BWD,       /* grouped GEMM dXp + LoRA                      */
    MOE_K_DX_COMBINE,       /* dX gather-sum                                */
    MOE_K_LORA_GRAD,        /* all LoRA weight-gradient kernels             */
    MOE_K_ROUTER_LOGITS,    /* router projection x W_r^T                    */
    MOE_K_ROUTER_DX,        /* router share of dX: d_logits W_r             */
    MOE_K_ROUTER_DW,        /* router weight gradient d_logits^T x          */
    MOE_K_COUNT
};
typedef struct {
    void *start[MOE_K_COUNT];  /* hipEvent_t or NULL */
    void *stop[MOE_K_COUNT];   /* hipEvent_t or NULL */
} moe_trace_t;

/* Workspace sizes in bytes (0 is a valid answer). NULL or invalid problem -> 0. */
size_t moe_route_workspace(const moe_problem_t *pb);
size_t moe_fwd_workspace(const moe_problem_t *pb, int training, int keep_expert_out);
size_t moe_bwd_workspace(const moe_problem_t *pb);

/* Where an intermediate sits inside a caller-owned workspace, for callers
 * that inspect it after the call (tests, debugging; the next call using the
 * workspace overwrites it). Returns its byte offset, or SIZE_MAX if that
 * workspace does not hold it for these arguments or the problem is invalid.
 *   MOE_PART_Y    moe_fwd workspace (sized with the same training and
 *                 keep_expert_out): Y [S,d] dtype, the expert outputs by
 *                 row p; held unless training with keep_expert_out = 1
 *                 (then Y is in `saved`).
 *   MOE_PART_DGU  moe_bwd workspace: [S,2F] dtype, row p = dG | dU (the
 *                 gradients of the gate and up projections' outputs).
 *   MOE_PART_DXP  moe_bwd workspace: dXp [S,d] dtype, row p's share of dX
 *                 before the gather-sum over the k choices of its token.
 * training and keep_expert_out are ignored for the moe_bwd parts. */
enum { MOE_PART_Y = 0, MOE_PART_DGU = 1, MOE_PART_DXP = 2 };
size_t moe_workspace_part(const moe_problem_t *pb, int part, int training, int keep_expert_out);

/* Bytes of the `saved` buffer that moe_fwd fills for moe_bwd. Layout, each
 * part starting on a 256-byte boundary: G, U [S,F] dtype; Zgu [S,2r]
 * float32 (x A_gate^T | x A_up^T); Zd [S,r] float32 (h A_down^T); for bf16
 * only, ZguT [2r,ldT] bf16 (Zgu transposed) and wZdT [r,ldT] bf16 (Zd
 * transposed, row p scaled by its combine weight), ldT = S rounded up to a
 * multiple of 8, the operands of the LoRA-gradient kernels; if
 * keep_expert_out, Y [S,d] dtype (expert outputs, needed for d_topk_w);
 * last, H [S,F] dtype, computed from G and U as stored (bf16-rounded for
 * bf16 layers), so that it can be rebuilt from them. Rows are indexed by
 * row p. */
size_t moe_saved_bytes(const moe_problem_t *pb, int keep_expert_out);

/* Bytes of `saved` that an offload moves to host memory: everything before
 * H (moe_saved_copy and the stack calls rebuild H on the reload). */
size_t moe_saved_host_bytes(const moe_problem_t *pb, int keep_expert_out);

/* Routing. logits [T,E] float32 -> rt (all six arrays written).
 * host_counts: (host) int32[E] that receives counts, or NULL: the one
 * device->host crossing of the layer, in stream order after the routing.
 * Pinned (page-locked) memory that the device reaches at its host address
 * (as hipHostMalloc memory is) is written by the routing's scan kernel
 * itself; other host memory by a copy enqueued on `stream` after the
 * routing kernels. With pinned host memory the call returns
 * at once and host_counts is valid once the stream has passed this point
 * (synchronise the stream or an event recorded after the call); with
 * pageable memory the runtime finishes the copy, and so waits for the
 * routing, before the call returns. The GPU path itself never needs the
 * counts on the host: tiles are scheduled on the device from offsets. */
moe_status_t moe_route(const moe_problem_t *pb, const float *logits, const moe_routing_t *rt,
                       int32_t *host_counts, void *ws, size_t ws_bytes, void *stream,
                       const moe_trace_t *trace);

/* moe_route for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments, outputs and errors as moe_route except that there is no
 * workspace argument: the routing workspace comes from a device array inside
 * the library (512 KiB on each GPU the library runs on, held until the
 * process ends), which covers every problem moe_route accepts
 * (MOE_E_UNSUPPORTED otherwise). The call allocates nothing; host_counts must
 * be NULL or pinned host memory (a copy to pageable memory would allocate
 * staging memory), else MOE_E_ARG. Every call on one GPU uses that GPU's one
 * array: calls that overlap on one GPU (different streams or host threads
 * without ordering between them) race and give undefined routing; order them
 * on one stream. The stream must belong to the current device; the array's
 * device address is looked up on the first call on each device. */
moe_status_t moe_route_noalloc(const moe_problem_t *pb, const float *logits, const moe_routing_t *rt,
                               int32_t *host_counts, void *stream, const moe_trace_t *trace);

/* Forward. x [T,d] -> out [T,d]. saved: NULL for inference (no backward
 * possible), else moe_saved_bytes(pb, keep_expert_out) bytes that moe_bwd
 * reads. ws: moe_fwd_workspace(pb, saved != NULL, keep_expert_out) bytes. */
moe_status_t moe_fwd(const moe_problem_t *pb, const void *x, const moe_routing_t *rt,
                     const moe_weights_t *w, void *out, void *saved, int keep_expert_out,
                     void *ws, size_t ws_bytes, void *stream, const moe_trace_t *trace);

/* Backward: the gradients of the layer derived by hand in closed form and
 * computed by dedicated kernels rather than by autograd (GPU MODE lecture 32
 * notes, "Unsloth - Faster, Lower-Memory LLM Fine-Tuning", part on deriving
 * every layer's backward by hand), with the frozen base W getting no
 * gradient and the LoRA factors A, B getting theirs (Unsloth 2026 wiki
 * chapter, "Optimisation 3", Split-LoRA subsection: only the low-rank
 * factors train). For dout = dL/dout:
 *   dy[t,j] = w[t,j] dout[t];  dh = dy W_d + s (dy B_d) A_d;
 *   dg = dh u sigma(g) (1 + g (1 - sigma(g))),  du = dh silu(g);
 *   dx[t] = sum_j (dg W_g + du W_u + s (dg B_g) A_g + s (du B_u) A_u)[t,j];
 *   dB_d = s dy^T (h A_d^T), dA_d = s (dy B_d)^T h, and the same pattern for
 *   gate and up with (dg, x) and (du, x), each summed over an expert's rows.
 * x and dout [T,d]; saved as filled by moe_fwd for the same x, routing and
 * weights. Writes dx [T,d] and all six LoRA gradients (experts with no rows
 * get exact zeros). d_topk_w [T,k] (= <dout[t], y[t,j]>) and d_logits [T,E]
 * (its chain through the softmax over the k selected logits, 0 for experts
 * not selected) are optional (NULL to skip) and need saved to hold Y
 * (keep_expert_out = 1 in moe_fwd; pass the same flag here).
 * Errors as for every call: arguments are checked before anything is
 * enqueued (MOE_E_ARG for NULL or misaligned buffers, or d_topk_w / d_logits
 * without keep_expert_out; MOE_E_WORKSPACE if ws_bytes is below
 * moe_bwd_workspace). The result does not depend on launch timing: every
 * reduction runs in a fixed order. */
moe_status_t moe_bwd(const moe_problem_t *pb, const void *x, const void *dout,
                     const moe_routing_t *rt, const moe_weights_t *w, const void *saved,
                     int keep_expert_out, void *dx, const moe_lora_grads_t *grads,
                     float *d_topk_w, float *d_logits, void *ws, size_t ws_bytes,
                     void *stream, const moe_trace_t *trace);

/* Router projection: the linear gate in front of moe_route. The pages start
 * the layer from a per-token routing decision over router logits (Unsloth x
 * NVIDIA blog, MoE routing paragraph; Unsloth 2026 wiki chapter,
 * "Optimisation 3", opening paragraph) without writing the gate out; this
 * is the plain bias-free one, logits = x W_r^T.
 *   w_router [E,d] in dtype (nn.Linear orientation); logits [T,E] float32.
 *   Requires E to be a multiple of 8 (else MOE_E_UNSUPPORTED).
 * moe_router_fwd: x [T,d] -> logits (fp32 accumulation over d). */
moe_status_t moe_router_fwd(const moe_problem_t *pb, const void *x, const void *w_router, float *logits,
                            void *stream, const moe_trace_t *trace);

/* Workspace bytes of moe_router_bwd (0 for an invalid problem). */
size_t moe_router_workspace(const moe_problem_t *pb);

/* Backward of the router projection for d_logits [T,E] float32 (the layer's
 * logit gradient, as moe_bwd writes it):
 *   dx [T,d] dtype     = dx_in + d_logits W_r   (dx_in is typically moe_bwd's
 *                        dx; dx may be the same buffer as dx_in; d_logits is
 *                        rounded to dtype as the product reads it)
 *   dw_router [E,d] fp32 = d_logits^T x        (overwritten; zeros if T = 0)
 * Either output may be NULL to skip it (dx_in is then unused); a frozen
 * router passes dw_router = NULL. ws: moe_router_workspace(pb) bytes (only
 * used for dw_router). The result does not depend on launch timing: dW_r is
 * summed over token chunks in a fixed order. */
moe_status_t moe_router_bwd(const moe_problem_t *pb, const void *x, const void *w_router, const float *d_logits,
                            const void *dx_in, void *dx, float *dw_router, void *ws, size_t ws_bytes,
                            void *stream, const moe_trace_t *trace);

/* Offload and reload of `saved` between moe_fwd and moe_bwd: the
 * double-buffered checkpoint reload of the Unsloth x NVIDIA blog (section
 * "core idea / structure / how it works", checkpoint paragraph) keeps
 * activations in pinned host memory and brings them back for the backward on
 * a copy stream, two device buffers taking turns so that the backward of one
 * layer reads buffer A while the next layer's activations arrive in B.
 * moe_saved_copy copies the first moe_saved_host_bytes(pb, keep_expert_out)
 * bytes of one `saved` buffer (all of it but H) to (to_device = 0) or from
 * (to_device = 1) `host`, on `copy_stream`, after `wait_event` (a hipEvent_t
 * the caller recorded on its compute stream, e.g. after moe_fwd, or before
 * the backward that last read the device buffer; NULL: no wait). After a
 * copy to the device it rebuilds H from G and U with a kernel on
 * copy_stream, bit-identical to the H moe_fwd stored. It records
 * `done_event` on copy_stream after that (NULL: none); the compute stream
 * waits on that event before moe_bwd reads the buffer. `host` must be
 * pinned (page-locked, e.g. hipHostMalloc), of moe_saved_host_bytes bytes
 * at least: pageable memory would make the copy synchronous, so it is
 * rejected (MOE_E_ARG). The bytes are copied unchanged. */
moe_status_t moe_saved_copy(const moe_problem_t *pb, int keep_expert_out, int to_device, void *saved,
                            void *host, void *wait_event, void *copy_stream, void *done_event);

/* A stack of layers with the double-buffered checkpoint offload and reload
 * of the Unsloth x NVIDIA blog (section "core idea / structure / how it
 * works", checkpoint paragraph): each layer's `saved` activations go to
 * pinned host memory during the forward and come back for the backward,
 * through two device buffers that take turns, so that the backward of one
 * layer reads buffer A while a copy stream brings the next layer back into
 * buffer B. Device memory for activations is two layers' `saved` instead of
 * n. Layer i uses buffer saved[i % 2].
 *   moe_stack_fwd: for i = 0 .. n-1 on `stream`: wait for the offload of
 *     layer i-2 (it reads saved[i % 2]); moe_route (logits -> rt); moe_fwd
 *     into saved[i % 2]; for i <= n-3, copy_stream copies saved[i % 2] (all
 *     but H, as moe_saved_copy) to host_saved: G and U once the gate/up GEMM
 *     has run, the rest after the forward. Layers n-2 and n-1 stay on the
 *     device.
 *   moe_stack_bwd (after moe_stack_fwd with the same arguments and nothing
 *     else written to the two buffers in between): for i = n-1 down to 0:
 *     layers i <= n-3 wait for their reload; moe_bwd from saved[i % 2]; then
 *     copy_stream reloads layer i-2 into saved[i % 2] (G and U as soon as
 *     layer i's down-backward GEMM, their last reader, has run; the rest
 *     after layer i's backward) and rebuilds its H, under the backward of
 *     layer i-1. The mid-call points are taken with the caller's events in
 *     the moe_trace_t hook, which the stack calls therefore do not offer.
 * Every layer has the problem pb. The caller wires the stack: layer i+1's x
 * is typically layer i's out, and layer i's dout layer i+1's dx. Results are
 * bit-identical to moe_route + moe_fwd + moe_bwd per layer with a saved
 * buffer each. */
typedef struct {
    const float *logits;           /* [T,E] router logits of the layer        */
    const moe_routing_t *rt;       /* routing outputs (written by the fwd)    */
    const moe_weights_t *w;        /* the layer's weights                     */
    const void *x;                 /* [T,d] layer input                       */
    void *out;                     /* [T,d] layer output (fwd)                */
    const void *dout;              /* [T,d] gradient of out (bwd)             */
    void *dx;                      /* [T,d] gradient of x (bwd)               */
    const moe_lora_grads_t *grads; /* LoRA gradients (bwd)                    */
    float *d_topk_w, *d_logits;    /* optional, as in moe_bwd (bwd)           */
    void *host_saved;              /* (host) pinned, moe_saved_host_bytes bytes; layers 0 .. n-3 */
} moe_stack_layer_t;

typedef struct {
    void *saved[2];      /* two device buffers of moe_saved_bytes(pb, keep) bytes (saved[1] unused if n = 1) */
    void *copy_stream;   /* hipStream_t of the copies; must differ from `stream` when n >= 3 */
    void *events[4];     /* four hipEvent_t the caller created (needed when n >= 3) */
} moe_offload_t;

/* Workspace bytes of moe_stack_fwd / moe_stack_bwd (the largest of the
 * route, forward and backward workspaces: they run one after another on one
 * stream); 0 for an invalid problem. */
size_t moe_stack_workspace(const moe_problem_t *pb, int keep_expert_out);

/* Errors: MOE_E_ARG for n < 1, NULL or misaligned buffers, equal device
 * buffers, host_saved of a layer <= n-3 that is not pinned, copy_stream equal
 * to stream or missing events when n >= 3; MOE_E_WORKSPACE below
 * moe_stack_workspace. All checks run before anything is enqueued. */
moe_status_t moe_stack_fwd(const moe_problem_t *pb, int n, const moe_stack_layer_t *layers, int keep_expert_out,
                           const moe_offload_t *off, void *ws, size_t ws_bytes, void *stream);
moe_status_t moe_stack_bwd(const moe_problem_t *pb, int n, const moe_stack_layer_t *layers, int keep_expert_out,
                           const moe_offload_t *off, void *ws, size_t ws_bytes, void *stream);

/* 4-bit NormalFloat (NF4) frozen base weights, the 4-bit QLoRA variant the
 * pages name for MoE fine-tuning (Unsloth 2026 wiki chapter, model-support
 * table; QLoRA's NF4 in the GPU MODE lecture 32 notes, closing open
 * questions), dequantised to bf16 so that
 * moe_fwd / moe_bwd run on them unchanged (the frozen weights stay 4-bit in
 * memory; one projection's bf16 copy lives in a scratch buffer for the pass).
 * Format (the QLoRA paper's NormalFloat code, the 16 values its appendix
 * lists): quantiles of N(0,1) with an exact zero, scaled into [-1, 1]
 * (level 0 = -1, level 7 = 0, level 15 = +1), built with top probability
 * 0.9677083; weight = level[code] * scale, one float32 scale per 64
 * consecutive weights of a row.
 *   codes  [rows, cols/2] uint8: element 2i of a row in the low nibble of
 *          byte i, element 2i+1 in the high nibble (16-byte aligned)
 *   scales [rows, cols/64] float32
 *   out    [rows, cols] bf16 (16-byte aligned)
 * Requires cols to be a positive multiple of 64 and rows >= 0 (else
 * MOE_E_ARG / MOE_E_UNSUPPORTED). For a stacked weight [E, out, in], rows =
 * E * out and cols = in. */
moe_status_t moe_nf4_dequant(const uint8_t *codes, const float *scales, int64_t rows, int32_t cols, void *out,
                             void *stream);

/* The forward and backward with the frozen base weights W_gate, W_up, W_down
 * held in 4-bit NormalFloat (the 4-bit QLoRA variant the pages name for MoE
 * fine-tuning: Unsloth 2026 wiki chapter, model-support table; QLoRA's NF4 in
 * the GPU MODE lecture 32 notes, closing open questions), dequantised inside
 * the grouped GEMMs as each weight tile is staged into LDS: no bf16 copy of
 * a weight is ever written to memory. Format as for moe_nf4_dequant; the
 * tile the GEMM multiplies is exactly the bf16 one moe_nf4_dequant would have
 * written, so moe_fwd_nf4 / moe_bwd_nf4 give bit-identical results to
 * moe_nf4_dequant followed by moe_fwd / moe_bwd on the dequantised weights.
 * Split-LoRA is unchanged (A and B stay in dtype).
 *   codes_gate, codes_up [E*F, d/2], codes_down [E*d, F/2] uint8 (16-byte aligned)
 *   scales_gate, scales_up [E*F, d/64], scales_down [E*d, F/64] float32 (4-byte aligned)
 * Arguments otherwise as moe_fwd / moe_bwd (same workspaces and `saved`);
 * w->w_gate, w_up, w_down are not read and may be NULL. Requires dtype bf16
 * and d, F multiples of 64 (else MOE_E_UNSUPPORTED). */
typedef struct {
    const uint8_t *codes_gate, *codes_up, *codes_down;
    const float *scales_gate, *scales_up, *scales_down;
} moe_nf4_base_t;

moe_status_t moe_fwd_nf4(const moe_problem_t *pb, const void *x, const moe_routing_t *rt, const moe_weights_t *w,
                         const moe_nf4_base_t *q4, void *out, void *saved, int keep_expert_out, void *ws,
                         size_t ws_bytes, void *stream, const moe_trace_t *trace);
moe_status_t moe_bwd_nf4(const moe_problem_t *pb, const void *x, const void *dout, const moe_routing_t *rt,
                         const moe_weights_t *w, const moe_nf4_base_t *q4, const void *saved, int keep_expert_out,
                         void *dx, const moe_lora_grads_t *grads, float *d_topk_w, float *d_logits, void *ws,
                         size_t ws_bytes, void *stream, const moe_trace_t *trace);

/* Static string naming a status code. */
const char *moe_status_str(moe_status_t st);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
