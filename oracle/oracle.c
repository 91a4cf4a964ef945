/*
 * oracle.c - plain, slow CPU reference of the MoE expert layer with Split-LoRA.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file's library. The HIP
 * library never does, and shares no code with it.
 *
 * Arithmetic is fp64 throughout; inputs are read in their stored format
 * (fp32 or bf16 bit patterns) and widened exactly.
 *
 * What it computes, and where each step is defined:
 *
 *  route   - top-k expert choice per token by (logit descending, expert id
 *            ascending) and softmax over the k chosen logits (the tiny fp32
 *            layer's stated router rule). Grouping is the naive per-expert
 *            scan that the Unsloth x NVIDIA blog (d9249.github.io, section
 *            "core idea / structure / how it works", MoE routing paragraph)
 *            describes as the slow form: for each expert, find its
 *            (token, choice) slots in token order. That blog states the
 *            flatten / stable-sort / bincount / offset rewrite leaves the
 *            routing result unchanged, so this scan's order IS the stable
 *            sort order the fast path must reproduce.
 *  forward - per expert, per routed row: SwiGLU expert MLP h = silu(g) * u,
 *            y = W_d h, with Split-LoRA: the frozen W is applied first and the
 *            low-rank term s * B (A x) is added afterwards, W + s B A never
 *            formed (Unsloth 2026 wiki chapter, "Optimisation 3: grouped_mm
 *            and Split-LoRA in MoE training", Split-LoRA subsection). The
 *            expert loop is the per-expert for-loop of that chapter's
 *            "bottleneck of the existing implementation" subsection, with the
 *            combine weight applied to the expert OUTPUT and summed over the
 *            k choices.
 *  router  - the linear gate before the routing: logits = x W_r^T (no bias),
 *            and its backward (the router's share of dX and dW_r) for a
 *            given gradient of the logits.
 *  backward- hand-derived closed form (GPU MODE lecture 32 notes, "Unsloth -
 *            Faster, Lower-Memory LLM Fine-Tuning", section on deriving each
 *            layer's gradient by hand): dX, dA and dB for gate/up/down with
 *            base W frozen, the gradient of the k combine weights, and its
 *            chain through the top-k softmax into the logits.
 *
 * Layouts (row-major; nn.Linear orientation [out, in]):
 *   x [T,d]; logits [T,E] fp32; W_gate, W_up [E,F,d]; W_down [E,d,F];
 *   A_gate, A_up [E,r,d]; B_gate, B_up [E,F,r]; A_down [E,r,F]; B_down [E,d,r].
 *   A slot is q = t*k + j (token t, choice j). A row p is a position in the
 *   expert-grouped order: rows offsets[e] .. offsets[e+1]-1 belong to expert e.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t T, d, E, k, F, r;
    double s;        /* LoRA scale alpha / r */
    int32_t dtype;   /* storage of x, W, A, B, dout: 0 float32, 1 bf16 bits, 2 float64 */
    const void *x, *w_gate, *w_up, *w_down;
    const void *a_gate, *b_gate, *a_up, *b_up, *a_down, *b_down;
} orc_layer_t;

/* threads the parallel loops below will use */
int orc_threads(void) { return omp_get_max_threads(); }

/* set that number (n >= 1) */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ------------------------------------------------------------------ */
/* stored value -> double (exact)                                      */

static inline double ld(const void *p, int dtype, size_t i)
{
    if (dtype == 1) {
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    if (dtype == 2)
        return ((const double *)p)[i];
    return (double)((const float *)p)[i];
}

static void ld_row(const void *p, int dtype, size_t off, int n, double *dst)
{
    for (int i = 0; i < n; ++i)
        dst[i] = ld(p, dtype, off + (size_t)i);
}

/* logistic sigmoid, evaluated without overflow */
static double sigmoid(double g)
{
    if (g >= 0.0)
        return 1.0 / (1.0 + exp(-g));
    const double e = exp(g);
    return e / (1.0 + e);
}

/* ------------------------------------------------------------------ */
/* routing                                                             */

/* key order: a before b iff logit_a > logit_b, or equal and id_a < id_b.
 * -0.0 and +0.0 compare equal, so the lower id wins. */
static int before(const float *l, int a, int b)
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

int orc_route(int32_t T, int32_t E, int32_t k, const float *logits,
              int32_t *topk_idx, double *topk_w, int32_t *counts, int32_t *offsets,
              int32_t *sorted_slot, int32_t *slot_row)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return 1;
    char *taken = (char *)malloc((size_t)E);
    if (!taken)
        return 2;
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        /* repeated selection of the best remaining expert */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || before(l, e, best)))
                    best = e;
            taken[best] = 1;
            topk_idx[(size_t)t * k + j] = best;
        }
        /* softmax over the k selected logits, shifted by the largest */
        const double l0 = l[topk_idx[(size_t)t * k]];
        double den = 0.0;
        for (int j = 0; j < k; ++j)
            den += exp((double)l[topk_idx[(size_t)t * k + j]] - l0);
        for (int j = 0; j < k; ++j)
            topk_w[(size_t)t * k + j] = exp((double)l[topk_idx[(size_t)t * k + j]] - l0) / den;
    }
    free(taken);

    /* per-expert scan in token order (the naive where() form) */
    int32_t p = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = p;
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j)
                if (topk_idx[(size_t)t * k + j] == e) {
                    sorted_slot[p] = t * k + j;
                    slot_row[t * k + j] = p;
                    ++p;
                }
        counts[e] = p - offsets[e];
    }
    offsets[E] = p;
    return 0;
}

/* ------------------------------------------------------------------ */
/* one routed row through expert e                                     */

typedef struct {
    double *xt, *zg, *zu, *g, *u, *h, *zd, *y;        /* forward  */
    double *dout, *dy, *pd, *dh, *dg, *du, *pg, *pu, *dx; /* backward */
    double *wrow;                                      /* a weight row */
} row_buf_t;

static int row_buf_alloc(row_buf_t *b, const orc_layer_t *L)
{
    const size_t d = (size_t)L->d, F = (size_t)L->F, r = (size_t)L->r;
    size_t wmax = d > F ? d : F;
    if (r > wmax)
        wmax = r;
    const size_t n = 5 * d + 6 * r + 6 * F + wmax;
    double *m = (double *)calloc(n, sizeof(double));
    if (!m)
        return 1;
    b->xt = m;  m += d;  b->zg = m;  m += r;  b->zu = m;  m += r;
    b->g = m;   m += F;  b->u = m;   m += F;  b->h = m;   m += F;
    b->zd = m;  m += r;  b->y = m;   m += d;  b->dout = m; m += d;
    b->dy = m;  m += d;  b->pd = m;  m += r;  b->dh = m;  m += F;
    b->dg = m;  m += F;  b->du = m;  m += F;  b->pg = m;  m += r;
    b->pu = m;  m += r;  b->dx = m;  m += d;  b->wrow = m;
    return 0;
}

static void row_buf_free(row_buf_t *b) { free(b->xt); }

static double dotw(const orc_layer_t *L, const void *w, size_t off, const double *v, int n,
                   double *tmp)
{
    ld_row(w, L->dtype, off, n, tmp);
    double acc = 0.0;
    for (int i = 0; i < n; ++i)
        acc += tmp[i] * v[i];
    return acc;
}

/* forward of token t through expert e; fills b->xt, zg, zu, g, u, h, zd, y */
static void row_fwd(const orc_layer_t *L, int e, int t, row_buf_t *b)
{
    const int d = L->d, F = L->F, r = L->r;
    const double s = L->s;
    const size_t E_ = (size_t)e;
    ld_row(L->x, L->dtype, (size_t)t * d, d, b->xt);
    /* low-rank projections z = A x (the LoRA path, kept apart from W) */
    for (int j = 0; j < r; ++j) {
        b->zg[j] = dotw(L, L->a_gate, (E_ * r + j) * d, b->xt, d, b->wrow);
        b->zu[j] = dotw(L, L->a_up, (E_ * r + j) * d, b->xt, d, b->wrow);
    }
    /* base W first, then the LoRA term s * B z added afterwards */
    for (int f = 0; f < F; ++f) {
        double g = dotw(L, L->w_gate, (E_ * F + f) * d, b->xt, d, b->wrow);
        double u = dotw(L, L->w_up, (E_ * F + f) * d, b->xt, d, b->wrow);
        g += s * dotw(L, L->b_gate, (E_ * F + f) * r, b->zg, r, b->wrow);
        u += s * dotw(L, L->b_up, (E_ * F + f) * r, b->zu, r, b->wrow);
        b->g[f] = g;
        b->u[f] = u;
        b->h[f] = g * sigmoid(g) * u; /* SwiGLU: silu(gate) * up */
    }
    for (int j = 0; j < r; ++j)
        b->zd[j] = dotw(L, L->a_down, (E_ * r + j) * F, b->h, F, b->wrow);
    for (int n = 0; n < d; ++n)
        b->y[n] = dotw(L, L->w_down, (E_ * d + n) * F, b->h, F, b->wrow)
                  + s * dotw(L, L->b_down, (E_ * d + n) * r, b->zd, r, b->wrow);
}

/* backward of one row, given row_fwd's results in b and the upstream
 * gradient of the layer output for token t (b->dout) and combine weight w.
 * Produces b->dy, pd, dh, dg, du, pg, pu, dx (this slot's part of dX) and
 * returns d(loss)/d(w) for this slot. */
static double row_bwd(const orc_layer_t *L, int e, double w, row_buf_t *b)
{
    const int d = L->d, F = L->F, r = L->r;
    const double s = L->s;
    const size_t E_ = (size_t)e;
    double dw = 0.0;
    for (int n = 0; n < d; ++n) {
        b->dy[n] = w * b->dout[n]; /* out = sum_j w_j y_j */
        dw += b->dout[n] * b->y[n];
    }
    /* y = W_d h + s B_d z_d,  z_d = A_d h */
    for (int j = 0; j < r; ++j)
        b->pd[j] = 0.0;
    for (int f = 0; f < F; ++f)
        b->dh[f] = 0.0;
    for (int n = 0; n < d; ++n) {
        ld_row(L->b_down, L->dtype, (E_ * d + n) * r, r, b->wrow);
        for (int j = 0; j < r; ++j)
            b->pd[j] += b->wrow[j] * b->dy[n];
        ld_row(L->w_down, L->dtype, (E_ * d + n) * F, F, b->wrow);
        for (int f = 0; f < F; ++f)
            b->dh[f] += b->wrow[f] * b->dy[n];
    }
    for (int j = 0; j < r; ++j) {
        ld_row(L->a_down, L->dtype, (E_ * r + j) * F, F, b->wrow);
        for (int f = 0; f < F; ++f)
            b->dh[f] += s * b->wrow[f] * b->pd[j];
    }
    /* h = g sigma(g) u */
    for (int f = 0; f < F; ++f) {
        const double g = b->g[f], sg = sigmoid(g);
        b->dg[f] = b->dh[f] * b->u[f] * sg * (1.0 + g * (1.0 - sg));
        b->du[f] = b->dh[f] * g * sg;
    }
    /* g = W_g x + s B_g z_g,  z_g = A_g x  (same for u) */
    for (int j = 0; j < r; ++j) {
        b->pg[j] = 0.0;
        b->pu[j] = 0.0;
    }
    for (int n = 0; n < d; ++n)
        b->dx[n] = 0.0;
    for (int f = 0; f < F; ++f) {
        ld_row(L->b_gate, L->dtype, (E_ * F + f) * r, r, b->wrow);
        for (int j = 0; j < r; ++j)
            b->pg[j] += b->wrow[j] * b->dg[f];
        ld_row(L->b_up, L->dtype, (E_ * F + f) * r, r, b->wrow);
        for (int j = 0; j < r; ++j)
            b->pu[j] += b->wrow[j] * b->du[f];
        ld_row(L->w_gate, L->dtype, (E_ * F + f) * d, d, b->wrow);
        for (int n = 0; n < d; ++n)
            b->dx[n] += b->wrow[n] * b->dg[f];
        ld_row(L->w_up, L->dtype, (E_ * F + f) * d, d, b->wrow);
        for (int n = 0; n < d; ++n)
            b->dx[n] += b->wrow[n] * b->du[f];
    }
    for (int j = 0; j < r; ++j) {
        ld_row(L->a_gate, L->dtype, (E_ * r + j) * d, d, b->wrow);
        for (int n = 0; n < d; ++n)
            b->dx[n] += s * b->wrow[n] * b->pg[j];
        ld_row(L->a_up, L->dtype, (E_ * r + j) * d, d, b->wrow);
        for (int n = 0; n < d; ++n)
            b->dx[n] += s * b->wrow[n] * b->pu[j];
    }
    return dw;
}

/* LoRA weight gradients of one row, added into expert e's slices
 * (da_g [r,d], db_g [F,r], da_u [r,d], db_u [F,r], da_d [r,F], db_d [d,r]). */
static void row_grads(const orc_layer_t *L, const row_buf_t *b, double *da_g, double *db_g,
                      double *da_u, double *db_u, double *da_d, double *db_d)
{
    const int d = L->d, F = L->F, r = L->r;
    const double s = L->s;
    for (int n = 0; n < d; ++n)
        for (int j = 0; j < r; ++j)
            db_d[(size_t)n * r + j] += s * b->dy[n] * b->zd[j];
    for (int j = 0; j < r; ++j)
        for (int f = 0; f < F; ++f)
            da_d[(size_t)j * F + f] += s * b->pd[j] * b->h[f];
    for (int f = 0; f < F; ++f)
        for (int j = 0; j < r; ++j) {
            db_g[(size_t)f * r + j] += s * b->dg[f] * b->zg[j];
            db_u[(size_t)f * r + j] += s * b->du[f] * b->zu[j];
        }
    for (int j = 0; j < r; ++j)
        for (int n = 0; n < d; ++n) {
            da_g[(size_t)j * d + n] += s * b->pg[j] * b->xt[n];
            da_u[(size_t)j * d + n] += s * b->pu[j] * b->xt[n];
        }
}

static void load_dout(const orc_layer_t *L, const void *dout, int t, double *dst)
{
    ld_row(dout, L->dtype, (size_t)t * L->d, L->d, dst);
}

/* ------------------------------------------------------------------ */
/* full layer                                                          */

/* Forward over the whole batch, one expert at a time.
 * out [T,d]; optional per-row intermediates (row p order, NULL to skip):
 * G, U, H [S,F]; Zg, Zu, Zd [S,r]; Y [S,d]. */
int orc_fwd(const orc_layer_t *L, const int32_t *topk_idx, const double *topk_w,
            const int32_t *offsets, const int32_t *sorted_slot, const int32_t *slot_row,
            double *out, double *G, double *U, double *H, double *Zg, double *Zu,
            double *Zd, double *Y)
{
    (void)topk_idx;
    const int T = L->T, d = L->d, k = L->k, F = L->F, r = L->r, E = L->E;
    const size_t S = (size_t)T * k;
    double *ys = (double *)malloc(S * (size_t)d * sizeof(double)); /* y per slot */
    if (!ys && S)
        return 2;
    int err = 0;
#pragma omp parallel
    {
        row_buf_t b;
        int my_err = row_buf_alloc(&b, L);
        if (my_err) {
#pragma omp atomic write
            err = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int e = 0; e < E; ++e) {
            if (my_err)
                continue;
            for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
                const int q = sorted_slot[p], t = q / k;
                row_fwd(L, e, t, &b);
                memcpy(ys + (size_t)q * d, b.y, (size_t)d * sizeof(double));
                if (G)  memcpy(G + (size_t)p * F, b.g, (size_t)F * sizeof(double));
                if (U)  memcpy(U + (size_t)p * F, b.u, (size_t)F * sizeof(double));
                if (H)  memcpy(H + (size_t)p * F, b.h, (size_t)F * sizeof(double));
                if (Zg) memcpy(Zg + (size_t)p * r, b.zg, (size_t)r * sizeof(double));
                if (Zu) memcpy(Zu + (size_t)p * r, b.zu, (size_t)r * sizeof(double));
                if (Zd) memcpy(Zd + (size_t)p * r, b.zd, (size_t)r * sizeof(double));
                if (Y)  memcpy(Y + (size_t)p * d, b.y, (size_t)d * sizeof(double));
            }
        }
        if (!my_err)
            row_buf_free(&b);
    }
    if (!err) {
        /* weighted combine, choices in ascending j */
        for (int t = 0; t < T; ++t)
            for (int n = 0; n < d; ++n) {
                double acc = 0.0;
                for (int j = 0; j < k; ++j) {
                    const size_t q = (size_t)t * k + j;
                    acc += topk_w[q] * ys[q * d + n];
                }
                out[(size_t)t * d + n] = acc;
            }
    }
    (void)slot_row;
    free(ys);
    return err;
}

/* d_logits of one token from its k combine weights and their gradients:
 * softmax over the selected logits, zero for experts not selected. */
static void softmax_bwd_row(int E, int k, const int32_t *idx, const double *w,
                            const double *dw, double *dl)
{
    double dot = 0.0;
    for (int j = 0; j < k; ++j)
        dot += w[j] * dw[j];
    for (int e = 0; e < E; ++e)
        dl[e] = 0.0;
    for (int j = 0; j < k; ++j)
        dl[idx[j]] = w[j] * (dw[j] - dot);
}

/* Backward over the whole batch, one expert at a time.
 * dout [T,d] in stored dtype. Outputs (all double, overwritten):
 * dx [T,d]; da_gate/da_up [E,r,d]; db_gate/db_up [E,F,r]; da_down [E,r,F];
 * db_down [E,d,r]; d_topk_w [T,k]; d_logits [T,E]. Optional per-row
 * intermediates (NULL to skip): dG, dU [S,F]; dXp [S,d]. */
int orc_bwd(const orc_layer_t *L, const int32_t *topk_idx, const double *topk_w,
            const int32_t *offsets, const int32_t *sorted_slot, const void *dout,
            double *dx, double *da_gate, double *db_gate, double *da_up, double *db_up,
            double *da_down, double *db_down, double *d_topk_w, double *d_logits,
            double *dG, double *dU, double *dXp)
{
    const int T = L->T, d = L->d, k = L->k, F = L->F, r = L->r, E = L->E;
    const size_t S = (size_t)T * k;
    double *dxs = (double *)malloc(S * (size_t)d * sizeof(double)); /* dX part per slot */
    double *dws = (double *)malloc((S ? S : 1) * sizeof(double));
    if ((!dxs && S) || !dws) {
        free(dxs);
        free(dws);
        return 2;
    }
    memset(da_gate, 0, (size_t)E * r * d * sizeof(double));
    memset(da_up, 0, (size_t)E * r * d * sizeof(double));
    memset(db_gate, 0, (size_t)E * F * r * sizeof(double));
    memset(db_up, 0, (size_t)E * F * r * sizeof(double));
    memset(da_down, 0, (size_t)E * r * F * sizeof(double));
    memset(db_down, 0, (size_t)E * d * r * sizeof(double));
    int err = 0;
#pragma omp parallel
    {
        row_buf_t b;
        int my_err = row_buf_alloc(&b, L);
        if (my_err) {
#pragma omp atomic write
            err = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int e = 0; e < E; ++e) {
            if (my_err)
                continue;
            for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
                const int q = sorted_slot[p], t = q / k;
                row_fwd(L, e, t, &b);
                load_dout(L, dout, t, b.dout);
                dws[q] = row_bwd(L, e, topk_w[q], &b);
                memcpy(dxs + (size_t)q * d, b.dx, (size_t)d * sizeof(double));
                if (dG)  memcpy(dG + (size_t)p * F, b.dg, (size_t)F * sizeof(double));
                if (dU)  memcpy(dU + (size_t)p * F, b.du, (size_t)F * sizeof(double));
                if (dXp) memcpy(dXp + (size_t)p * d, b.dx, (size_t)d * sizeof(double));
                row_grads(L, &b, da_gate + (size_t)e * r * d, db_gate + (size_t)e * F * r,
                          da_up + (size_t)e * r * d, db_up + (size_t)e * F * r,
                          da_down + (size_t)e * r * F, db_down + (size_t)e * d * r);
            }
        }
        if (!my_err)
            row_buf_free(&b);
    }
    if (!err) {
        for (int t = 0; t < T; ++t) {
            for (int n = 0; n < d; ++n) {
                double acc = 0.0;
                for (int j = 0; j < k; ++j)
                    acc += dxs[((size_t)t * k + j) * d + n];
                dx[(size_t)t * d + n] = acc;
            }
            if (d_topk_w)
                for (int j = 0; j < k; ++j)
                    d_topk_w[(size_t)t * k + j] = dws[(size_t)t * k + j];
            if (d_logits)
                softmax_bwd_row(E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k,
                                dws + (size_t)t * k, d_logits + (size_t)t * E);
        }
    }
    free(dxs);
    free(dws);
    return err;
}

/* ------------------------------------------------------------------ */
/* sampled entry points (for full-size layers, one token / expert at a */
/* time; same row functions as the full layer)                         */

/* out rows for the n tokens listed: out_rows [n,d]; y_rows [n,k,d] or NULL. */
int orc_fwd_tokens(const orc_layer_t *L, const int32_t *topk_idx, const double *topk_w,
                   int32_t n, const int32_t *tokens, double *out_rows, double *y_rows)
{
    const int d = L->d, k = L->k;
    int err = 0;
#pragma omp parallel
    {
        row_buf_t b;
        int my_err = row_buf_alloc(&b, L);
        if (my_err) {
#pragma omp atomic write
            err = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; ++i) {
            if (my_err)
                continue;
            const int t = tokens[i];
            double *o = out_rows + (size_t)i * d;
            for (int c = 0; c < d; ++c)
                o[c] = 0.0;
            for (int j = 0; j < k; ++j) {
                const size_t q = (size_t)t * k + j;
                row_fwd(L, topk_idx[q], t, &b);
                for (int c = 0; c < d; ++c)
                    o[c] += topk_w[q] * b.y[c];
                if (y_rows)
                    memcpy(y_rows + ((size_t)i * k + j) * d, b.y, (size_t)d * sizeof(double));
            }
        }
        if (!my_err)
            row_buf_free(&b);
    }
    return err;
}

/* dX, d_topk_w and d_logits rows for the n tokens listed:
 * dx_rows [n,d]; dtw_rows [n,k] or NULL; dl_rows [n,E] or NULL. */
int orc_bwd_tokens(const orc_layer_t *L, const int32_t *topk_idx, const double *topk_w,
                   const void *dout, int32_t n, const int32_t *tokens, double *dx_rows,
                   double *dtw_rows, double *dl_rows)
{
    const int d = L->d, k = L->k, E = L->E;
    int err = 0;
#pragma omp parallel
    {
        row_buf_t b;
        double *dws = (double *)malloc((size_t)k * sizeof(double));
        int my_err = row_buf_alloc(&b, L) || !dws;
        if (my_err) {
#pragma omp atomic write
            err = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; ++i) {
            if (my_err)
                continue;
            const int t = tokens[i];
            double *o = dx_rows + (size_t)i * d;
            for (int c = 0; c < d; ++c)
                o[c] = 0.0;
            for (int j = 0; j < k; ++j) {
                const size_t q = (size_t)t * k + j;
                row_fwd(L, topk_idx[q], t, &b);
                load_dout(L, dout, t, b.dout);
                dws[j] = row_bwd(L, topk_idx[q], topk_w[q], &b);
                for (int c = 0; c < d; ++c)
                    o[c] += b.dx[c];
            }
            if (dtw_rows)
                memcpy(dtw_rows + (size_t)i * k, dws, (size_t)k * sizeof(double));
            if (dl_rows)
                softmax_bwd_row(E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k, dws,
                                dl_rows + (size_t)i * E);
        }
        if (!my_err)
            row_buf_free(&b);
        free(dws);
    }
    return err;
}

/* LoRA gradients of the n experts listed, each reduced over all of its rows.
 * Outputs, one slice per listed expert: da_g/da_u [n,r,d]; db_g/db_u [n,F,r];
 * da_d [n,r,F]; db_d [n,d,r]. An expert with no rows gets exact zeros. */
int orc_lora_grads(const orc_layer_t *L, const int32_t *topk_idx, const double *topk_w, const int32_t *offsets, const int32_t *sorted_slot,
                   const void *dout, int32_t n, const int32_t *experts, double *da_g,
                   double *db_g, double *da_u, double *db_u, double *da_d, double *db_d)
{
    (void)topk_idx;
    const int d = L->d, k = L->k, F = L->F, r = L->r;
    memset(da_g, 0, (size_t)n * r * d * sizeof(double));
    memset(da_u, 0, (size_t)n * r * d * sizeof(double));
    memset(db_g, 0, (size_t)n * F * r * sizeof(double));
    memset(db_u, 0, (size_t)n * F * r * sizeof(double));
    memset(da_d, 0, (size_t)n * r * F * sizeof(double));
    memset(db_d, 0, (size_t)n * d * r * sizeof(double));
    int err = 0;
    for (int i = 0; i < n && !err; ++i) {
        const int e = experts[i];
        const int p0 = offsets[e], ne = offsets[e + 1] - offsets[e];
        if (ne == 0)
            continue;
        /* phase 1: every row's forward and backward, rows in parallel */
        row_buf_t *rb = (row_buf_t *)calloc((size_t)ne, sizeof(row_buf_t));
        if (!rb)
            return 2;
        for (int m = 0; m < ne; ++m)
            if (row_buf_alloc(&rb[m], L)) {
                for (int z = 0; z < m; ++z)
                    row_buf_free(&rb[z]);
                free(rb);
                return 2;
            }
#pragma omp parallel for schedule(dynamic, 1)
        for (int m = 0; m < ne; ++m) {
            const int q = sorted_slot[p0 + m], t = q / k;
            row_fwd(L, e, t, &rb[m]);
            load_dout(L, dout, t, rb[m].dout);
            (void)row_bwd(L, e, topk_w[q], &rb[m]);
        }
        /* phase 2: accumulate in row order */
        for (int m = 0; m < ne; ++m) {
            row_grads(L, &rb[m], da_g + (size_t)i * r * d, db_g + (size_t)i * F * r,
                      da_u + (size_t)i * r * d, db_u + (size_t)i * F * r,
                      da_d + (size_t)i * r * F, db_d + (size_t)i * d * r);
            row_buf_free(&rb[m]);
        }
        free(rb);
    }
    return err;
}

/* ------------------------------------------------------------------------
 * Router projection: the gate that turns each token into its expert logits,
 * logits[t][e] = sum_i x[t][i] * W_r[e][i] (W_r [E,d], nn.Linear orientation,
 * no bias). The pages start the MoE layer from a per-token routing decision
 * over router logits (blog, MoE routing paragraph; wiki chapter,
 * "Optimisation 3", opening paragraph) without writing the gate out; this is
 * the plain linear gate. Inputs in the storage dtype, output fp64.
 * ------------------------------------------------------------------------ */
int orc_router_fwd(int32_t T, int32_t d, int32_t E, int32_t dtype, const void *x, const void *w_r,
                   double *logits)
{
    if (T < 0 || d < 1 || E < 1)
        return 1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += ld(x, dtype, (size_t)t * d + i) * ld(w_r, dtype, (size_t)e * d + i);
            logits[(size_t)t * E + e] = acc;
        }
    return 0;
}

/* Backward of the router projection for an upstream gradient d_logits [T,E]
 * (the layer's gradient with respect to its logits):
 *   dx_r[t][i] = sum_e d_logits[t][e] * W_r[e][i]   (the router's share of dX)
 *   dw_r[e][i] = sum_t d_logits[t][e] * x[t][i]
 * Either output may be NULL. Sums run in ascending e and t. */
int orc_router_bwd(int32_t T, int32_t d, int32_t E, int32_t dtype, const void *x, const void *w_r,
                   const double *d_logits, double *dx_r, double *dw_r)
{
    if (T < 0 || d < 1 || E < 1)
        return 1;
    if (dx_r) {
#pragma omp parallel for schedule(static)
        for (int t = 0; t < T; ++t)
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int e = 0; e < E; ++e)
                    acc += d_logits[(size_t)t * E + e] * ld(w_r, dtype, (size_t)e * d + i);
                dx_r[(size_t)t * d + i] = acc;
            }
    }
    if (dw_r) {
#pragma omp parallel for schedule(static)
        for (int e = 0; e < E; ++e)
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int t = 0; t < T; ++t)
                    acc += d_logits[(size_t)t * E + e] * ld(x, dtype, (size_t)t * d + i);
                dw_r[(size_t)e * d + i] = acc;
            }
    }
    return 0;
}
