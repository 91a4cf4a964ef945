"""The oracle's expert layer with each expert's rows as one matrix product.

TEST INFRASTRUCTURE ONLY (like the rest of this package): imported by the
test suite and the benchmark's CPU-baseline leg, never by the library. It
shares no code with the HIP path.

Same layer, same readings and same fp64 arithmetic as ``oracle.c``; only the
loop over an expert's rows is replaced by numpy float64 matrix products (a
library matmul as a step, nothing blocked or fused beyond what the
definition states). The per-expert loop itself is the one of the Unsloth
2026 wiki chapter ("Optimisation 3: grouped_mm and Split-LoRA in MoE
training", subsection on the bottleneck of the existing implementation): for
each expert, take the rows routed to it, run its SwiGLU MLP, weight the
outputs by their combine weights and sum them per token. Split-LoRA follows
the same chapter's Split-LoRA subsection: the frozen W is applied first and
s (X A^T) B^T is added afterwards, W + s B A is never formed. The backward is
the hand-derived closed form (GPU MODE lecture 32 notes, "Unsloth - Faster,
Lower-Memory LLM Fine-Tuning", part on deriving every layer's gradient by
hand), W frozen.

The matrix form makes whole layers of the large workloads (65536 routed rows)
affordable on the host in seconds, where the row-at-a-time C oracle takes
minutes; both are pinned by the same tests.

Routing (``rt``) comes from ``oracle.route``: rows of expert e are
rt["sorted_slot"][offsets[e]:offsets[e+1]], in increasing token order.
"""
from __future__ import annotations

import numpy as np

GRADS = ("da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down")


def _widen(a: np.ndarray) -> np.ndarray:
    """Stored values (float32, bf16 bit patterns as uint16, float64) -> float64, exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _sigmoid(g: np.ndarray) -> np.ndarray:
    """Logistic function without overflow: 1/(1+e^-g) for g >= 0, e^g/(1+e^g) below."""
    e = np.exp(-np.abs(g))
    return np.where(g >= 0.0, 1.0 / (1.0 + e), e / (1.0 + e))


def layer(L, rt: dict, dout=None, intermediates: bool = False) -> dict:
    """Forward (and, if dout is given, backward) of the whole layer.

    L is an ``oracle.Layer`` (dims, s and the stored tensors). Returns fp64:
    out [T,d]; with dout: dx [T,d], the six LoRA gradients, d_topk_w [T,k],
    d_logits [T,E]. intermediates adds the per-row tensors in row-p order:
    G, U, H [S,F], Zg, Zu, Zd [S,r], Y [S,d] and, with dout, dG, dU [S,F],
    dXp [S,d].
    """
    T, d, E, k, F, r, s = L.T, L.d, L.E, L.k, L.F, L.r, L.s
    S = T * k
    x = _widen(L.t["x"])
    topk_w = np.asarray(rt["topk_w"], np.float64).reshape(-1)   # per slot q = t k + j
    offsets, sorted_slot = rt["offsets"], rt["sorted_slot"]
    ys = np.zeros((S, d))                                       # expert output per slot
    o = {}
    if intermediates:
        for n, c in (("G", F), ("U", F), ("H", F), ("Zg", r), ("Zu", r), ("Zd", r), ("Y", d)):
            o[n] = np.zeros((S, c))
    bwd = dout is not None
    if bwd:
        do = _widen(np.asarray(dout))
        dxs = np.zeros((S, d))                                  # dX part per slot
        dws = np.zeros(S)                                       # d(loss)/d(w) per slot
        for n, shape in (("da_gate", (E, r, d)), ("db_gate", (E, F, r)), ("da_up", (E, r, d)),
                         ("db_up", (E, F, r)), ("da_down", (E, r, F)), ("db_down", (E, d, r))):
            o[n] = np.zeros(shape)
        if intermediates:
            for n, c in (("dG", F), ("dU", F), ("dXp", d)):
                o[n] = np.zeros((S, c))
    for e in range(E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue                                            # no rows: gradients stay exactly 0
        q = sorted_slot[p0:p1].astype(np.int64)                 # this expert's slots, token order
        tok = q // k
        Wg, Wu, Wd = (_widen(L.t[n][e]) for n in ("w_gate", "w_up", "w_down"))
        Ag, Bg, Au, Bu, Ad, Bd = (_widen(L.t[n][e]) for n in
                                  ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down"))
        X = x[tok]                                              # [n_e, d]
        # forward: base W first, then the low-rank term s (X A^T) B^T added
        Zg, Zu = X @ Ag.T, X @ Au.T
        G = X @ Wg.T + s * (Zg @ Bg.T)
        U = X @ Wu.T + s * (Zu @ Bu.T)
        sg = _sigmoid(G)
        H = G * sg * U                                          # SwiGLU: silu(gate) * up
        Zd = H @ Ad.T
        Y = H @ Wd.T + s * (Zd @ Bd.T)
        ys[q] = Y
        if intermediates:
            for n, v in (("G", G), ("U", U), ("H", H), ("Zg", Zg), ("Zu", Zu), ("Zd", Zd), ("Y", Y)):
                o[n][p0:p1] = v
        if not bwd:
            continue
        Do = do[tok]                                            # dL/dout of each row's token
        w = topk_w[q][:, None]
        dY = w * Do                                             # out = sum_j w_j y_j
        dws[q] = np.sum(Do * Y, axis=1)
        # y = W_d h + s B_d z_d,  z_d = A_d h
        Pd = dY @ Bd
        dH = dY @ Wd + s * (Pd @ Ad)
        o["db_down"][e] = s * (dY.T @ Zd)
        o["da_down"][e] = s * (Pd.T @ H)
        # h = g sigma(g) u
        dG = dH * U * sg * (1.0 + G * (1.0 - sg))
        dU = dH * G * sg
        # g = W_g x + s B_g z_g,  z_g = A_g x  (the same for u)
        Pg, Pu = dG @ Bg, dU @ Bu
        dXp = dG @ Wg + dU @ Wu + s * (Pg @ Ag + Pu @ Au)
        dxs[q] = dXp
        o["db_gate"][e] = s * (dG.T @ Zg)
        o["da_gate"][e] = s * (Pg.T @ X)
        o["db_up"][e] = s * (dU.T @ Zu)
        o["da_up"][e] = s * (Pu.T @ X)
        if intermediates:
            o["dG"][p0:p1], o["dU"][p0:p1], o["dXp"][p0:p1] = dG, dU, dXp
    # weighted combine and dX gather-sum, choices j ascending
    wk = topk_w.reshape(T, k)
    ysk = ys.reshape(T, k, d)
    out = np.zeros((T, d))
    for j in range(k):
        out += wk[:, j:j + 1] * ysk[:, j]
    o["out"] = out
    if bwd:
        dxk = dxs.reshape(T, k, d)
        dx = np.zeros((T, d))
        for j in range(k):
            dx += dxk[:, j]
        o["dx"] = dx
        dw = dws.reshape(T, k)
        o["d_topk_w"] = dw
        # softmax over the k selected logits: dl_j = w_j (dw_j - sum_i w_i dw_i), 0 elsewhere
        dot = np.sum(wk * dw, axis=1, keepdims=True)
        dl = np.zeros((T, E))
        np.put_along_axis(dl, np.asarray(rt["topk_idx"], np.int64), wk * (dw - dot), axis=1)
        o["d_logits"] = dl
    return o


def fwd(L, rt: dict, intermediates: bool = False) -> dict:
    """out (and the forward intermediates), like ``oracle.fwd``."""
    return layer(L, rt, None, intermediates)


def bwd(L, rt: dict, dout, intermediates: bool = False) -> dict:
    """The backward outputs (and dG, dU, dXp), like ``oracle.bwd``."""
    o = layer(L, rt, L.store(dout), intermediates)
    keep = ("dx", "d_topk_w", "d_logits") + GRADS + (("dG", "dU", "dXp") if intermediates else ())
    return {n: o[n] for n in keep}
