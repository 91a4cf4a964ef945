"""GPU parity of the router projection (logits = x W_r^T) and its backward
(the router's share of dX, and dW_r) through the C ABI, against the CPU
oracle. Bounds: logits 1e-5 (exact products, fp32 accumulation); dx and dW_r
the storage type's bound (bf16 2e-2, fp32 1e-5), since a bf16 layer rounds
the logit gradient to bf16 as the products read it.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
from synth.configs import LayerConfig  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}

SMALL = {
    "tiny_fp32": synth.get_config("tiny_fp32"),
    # T ragged against 128-row tiles; d ragged against 128 columns; E = 40:
    # a ragged expert tile and a ragged K in the dX product
    "ragged_bf16": LayerConfig("router_ragged_bf16", T=300, d=264, E=40, k=4, F=64, r=8,
                               dtype="bf16", alpha=16.0),
    "ragged_f32": LayerConfig("router_ragged_f32", T=300, d=264, E=40, k=4, F=64, r=8,
                              dtype="f32", alpha=16.0),
    # several token chunks for dW_r, the last one ragged
    "chunks_bf16": LayerConfig("router_chunks_bf16", T=2085, d=136, E=16, k=2, F=64, r=8,
                               dtype="bf16", alpha=16.0),
    "one_token_bf16": LayerConfig("router_one_token_bf16", T=1, d=64, E=8, k=2, F=64, r=8,
                                  dtype="bf16", alpha=16.0),
    # E = 200: a second 128-expert row tile of dW_r (72 experts) and a ragged
    # fourth 64-expert tile of the logits; d = 392: a ragged last 128-column
    # tile (8 columns); T = 777 in four token chunks, the last one ragged
    "many_experts_bf16": LayerConfig("router_many_experts_bf16", T=777, d=392, E=200, k=4, F=64, r=8,
                                     dtype="bf16", alpha=16.0),
}


def _lr():
    import layer_runner
    return layer_runner


def _run(cfg, x, w_r, d_logits, dx_in):
    import moe_layer_lora_amd as moe
    lr = _lr()
    pb = moe.Problem.from_config(cfg)
    dev = torch.device("cuda")
    xt, wt, dlt = lr.to_dev(x), lr.to_dev(w_r), lr.to_dev(d_logits)
    dx = lr.to_dev(dx_in)  # updated in place: dx = dx + d_logits W_r
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    dw = torch.full((cfg.E, cfg.d), float("nan"), dtype=torch.float32, device=dev)
    ws = moe.alloc_bytes(moe.router_workspace(pb), dev)
    moe.moe_router_fwd(pb, xt, wt, logits)
    moe.moe_router_bwd(pb, xt, wt, dlt, dx_in=dx, dx=dx, dw_router=dw, ws=ws)
    torch.cuda.synchronize()
    return {"logits": logits.cpu().numpy().astype(np.float64), "dx": lr.to_f64(dx),
            "dw": dw.cpu().numpy().astype(np.float64)}


def _inputs(cfg):
    inp = synth.make_inputs(cfg, seed=0)
    ri = synth.make_router(cfg, seed=0)
    return inp["x"], ri["w_router"], ri["d_logits"], inp["dout"]


@pytest.mark.parametrize("name", list(SMALL))
def test_router_small_parity(name):
    cfg = SMALL[name]
    lr = _lr()
    x, w_r, dl, dx_in = _inputs(cfg)
    print(f"[router] {name}: T={cfg.T} d={cfg.d} E={cfg.E} {cfg.dtype}", flush=True)
    g = _run(cfg, x, w_r, dl, dx_in)
    lo = oracle.router_fwd(x, w_r)
    ro = oracle.router_bwd(x, w_r, dl.astype(np.float64))
    tol = TOL[cfg.dtype]
    assert lr.rel_l2(g["logits"], lo) <= 1e-5
    assert lr.rel_l2(g["dx"], synth.to_f64(dx_in, cfg.dtype) + ro["dx"]) <= tol
    assert lr.rel_l2(g["dw"], ro["dw_r"]) <= tol


def test_router_chain_into_layer_tiny():
    """The layer with its router on the GPU (router -> route -> fwd -> bwd ->
    router bwd) against the same chain in the oracle."""
    import moe_layer_lora_amd as moe
    lr = _lr()
    cfg = synth.get_config("tiny_fp32").with_(router_grad=True)
    inp = synth.make_inputs(cfg, seed=0)
    w_r = synth.make_router(cfg, seed=0)["w_router"]
    pb = moe.Problem.from_config(cfg)
    dev = torch.device("cuda")
    # GPU: logits from the router feed the layer
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    moe.moe_router_fwd(pb, lr.to_dev(inp["x"]), lr.to_dev(w_r), logits)
    torch.cuda.synchronize()
    L = lr.Layer(cfg, inp, keep_expert_out=True)
    L.logits.copy_(logits)
    L.step(backward=True, router_grad=True)
    r = L.results(backward=True, router_grad=True)
    dw = torch.empty((cfg.E, cfg.d), dtype=torch.float32, device=dev)
    ws = moe.alloc_bytes(moe.router_workspace(pb), dev)
    moe.moe_router_bwd(pb, L.x, lr.to_dev(w_r), L.d_logits, dx_in=L.dx, dx=L.dx, dw_router=dw,
                       ws=ws)
    torch.cuda.synchronize()
    dx = L.dx
    # oracle: its own logits (rounded to fp32, as the routing reads them)
    lo = oracle.router_fwd(inp["x"], w_r).astype(np.float32)
    rt = oracle.route(lo, cfg.k)
    for n in ("topk_idx", "counts", "offsets", "sorted_slot", "slot_row"):
        assert np.array_equal(r[n], rt[n]), n
    OL = oracle.Layer.from_config(cfg, inp)
    b = oracle.bwd(OL, rt, inp["dout"])
    ro = oracle.router_bwd(inp["x"], w_r, b["d_logits"])
    assert lr.rel_l2(lr.to_f64(dx), b["dx"] + ro["dx"]) <= 1e-5
    assert lr.rel_l2(dw.cpu().numpy().astype(np.float64), ro["dw_r"]) <= 1e-5


@pytest.mark.slow
@pytest.mark.parametrize("name", ["qwen3_30b_a3b", "gptoss120b"])
def test_router_full_size_sampled(name):
    lr = _lr()
    cfg = synth.get_config(name)
    x, w_r, dl, dx_in = _inputs(cfg)
    print(f"[router full] {name}: GPU", flush=True)
    g = _run(cfg, x, w_r, dl, dx_in)
    rng = np.random.default_rng(0)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 30, replace=False)]))
    ex = np.array([0, 57, cfg.E - 1])
    print(f"[router full] {name}: oracle on {len(toks)} tokens, experts {ex.tolist()}", flush=True)
    tol = TOL[cfg.dtype]
    assert lr.rel_l2(g["logits"][toks], oracle.router_fwd(np.ascontiguousarray(x[toks]), w_r)) <= 1e-5
    ro = oracle.router_bwd(np.ascontiguousarray(x[toks]), w_r, dl[toks].astype(np.float64))
    assert lr.rel_l2(g["dx"][toks], synth.to_f64(dx_in[toks], cfg.dtype) + ro["dx"]) <= tol
    re = oracle.router_bwd(x, np.ascontiguousarray(w_r[ex]),
                           np.ascontiguousarray(dl[:, ex]).astype(np.float64))
    assert lr.rel_l2(g["dw"][ex], re["dw_r"]) <= tol
    assert np.all(np.isfinite(g["dw"]))


def test_router_empty_batch_writes_zero_weight_gradient():
    import moe_layer_lora_amd as moe
    cfg = LayerConfig("router_empty", T=0, d=64, E=16, k=2, F=64, r=8, dtype="bf16", alpha=16.0)
    pb = moe.Problem.from_config(cfg)
    dev = torch.device("cuda")
    w_r = torch.zeros((cfg.E, cfg.d), dtype=torch.bfloat16, device=dev)
    dw = torch.full((cfg.E, cfg.d), float("nan"), dtype=torch.float32, device=dev)
    ws = moe.alloc_bytes(moe.router_workspace(pb), dev)
    moe.moe_router_fwd(pb, None, w_r, None)
    moe.moe_router_bwd(pb, None, w_r, None, dw_router=dw, ws=ws)
    torch.cuda.synchronize()
    assert torch.all(dw == 0.0)


def test_router_backward_outputs_are_independent():
    """dx alone (frozen router: dw_router NULL) and dW_r alone (dx NULL) give
    the same values as the call that writes both."""
    import layer_runner as lr
    import moe_layer_lora_amd as moe
    cfg = SMALL["ragged_bf16"]
    x, w_r, dl, dx_in = _inputs(cfg)
    pb = moe.Problem.from_config(cfg)
    dev = torch.device("cuda")
    xt, wt, dlt = lr.to_dev(x), lr.to_dev(w_r), lr.to_dev(dl)
    ws = moe.alloc_bytes(moe.router_workspace(pb), dev)
    dx_both, dx_only = lr.to_dev(dx_in), lr.to_dev(dx_in)
    dw_both = torch.empty((cfg.E, cfg.d), dtype=torch.float32, device=dev)
    dw_only = torch.empty_like(dw_both)
    moe.moe_router_bwd(pb, xt, wt, dlt, dx_in=dx_both, dx=dx_both, dw_router=dw_both, ws=ws)
    moe.moe_router_bwd(pb, xt, wt, dlt, dx_in=dx_only, dx=dx_only)
    moe.moe_router_bwd(pb, xt, wt, dlt, dw_router=dw_only, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(dx_both, dx_only) and torch.equal(dw_both, dw_only)
