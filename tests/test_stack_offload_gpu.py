"""The double-buffered offload / reload schedule (moe_stack_fwd /
moe_stack_bwd) against the same stack run layer by layer with a device
`saved` buffer per layer: every output bit-identical (the copies move bytes
unchanged, so nothing may differ), for stacks of 1 to 5 layers, with the
layers chained (layer i+1's input is layer i's output, layer i's upstream
gradient is layer i+1's dx)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_layer_lora_amd as moe  # noqa: E402
import synth  # noqa: E402
from synth.configs import LayerConfig  # noqa: E402

pytestmark = pytest.mark.gpu

WEIGHTS = ("w_gate", "w_up", "w_down", "a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


def _dev(a, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _make_stack(cfg, n, dev):
    """n layers with their own weights and logits (seeds 10 + i); layer 0's
    input and the top gradient from seed 9."""
    pb = moe.Problem.from_config(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    top = synth.make_inputs(cfg, seed=9)
    layers = []
    for i in range(n):
        inp = synth.make_inputs(cfg, seed=10 + i, with_dout=False)
        L = {"logits": _dev(inp["logits"], dev), "w": {k: _dev(inp[k], dev) for k in WEIGHTS},
             "rt": moe.alloc_routing(pb, dev), "grads": moe.alloc_grads(pb, dev),
             "out": torch.empty((cfg.T, cfg.d), dtype=dt, device=dev),
             "dx": torch.empty((cfg.T, cfg.d), dtype=dt, device=dev)}
        if cfg.router_grad:
            L["d_topk_w"] = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
            L["d_logits"] = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
        layers.append(L)
    for i, L in enumerate(layers):
        L["x"] = _dev(top["x"], dev) if i == 0 else layers[i - 1]["out"]
        L["dout"] = _dev(top["dout"], dev) if i == n - 1 else layers[i + 1]["dx"]
    return pb, layers


def _snapshot(layers):
    torch.cuda.synchronize()
    snap = []
    for L in layers:
        d = {k: L[k].clone() for k in ("out", "dx")}
        d.update({k: v.clone() for k, v in L["rt"].items()})
        d.update({k: v.clone() for k, v in L["grads"].items()})
        for k in ("d_topk_w", "d_logits"):
            if k in L:
                d[k] = L[k].clone()
        snap.append(d)
    return snap


def _run_per_layer(cfg, pb, layers, keep, dev):
    saved = [moe.alloc_bytes(moe.saved_bytes(pb, keep), dev) for _ in layers]
    ws_r = moe.alloc_bytes(moe.route_workspace(pb), dev)
    ws_f = moe.alloc_bytes(moe.fwd_workspace(pb, True, keep), dev)
    ws_b = moe.alloc_bytes(moe.bwd_workspace(pb), dev)
    for L, sv in zip(layers, saved):
        moe.moe_route(pb, L["logits"], L["rt"], ws=ws_r)
        moe.moe_fwd(pb, L["x"], L["rt"], L["w"], L["out"], saved=sv, keep_expert_out=keep, ws=ws_f)
    for L, sv in reversed(list(zip(layers, saved))):
        moe.moe_bwd(pb, L["x"], L["dout"], L["rt"], L["w"], sv, keep, L["dx"], L["grads"],
                    d_topk_w=L.get("d_topk_w"), d_logits=L.get("d_logits"), ws=ws_b)
    return _snapshot(layers)


def _run_stack(cfg, pb, layers, keep, dev):
    nbytes, nhost = moe.saved_bytes(pb, keep), moe.saved_host_bytes(pb, keep)
    for i, L in enumerate(layers):
        L["host_saved"] = (torch.empty(nhost, dtype=torch.uint8, pin_memory=True)
                           if i <= len(layers) - 3 else None)
    dsaved = [moe.alloc_bytes(nbytes, dev) for _ in range(2)]
    # stale bytes in the buffers: whatever the forward does not write must not matter
    for b in dsaved:
        b.fill_(0x5A)
    ws = moe.alloc_bytes(moe.stack_workspace(pb, keep), dev)
    cs = torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(4)]
    for e in events:  # torch creates the HIP event at its first record
        e.record()
    for L in layers:  # outputs the stack must overwrite
        for k in ("out", "dx", "d_topk_w", "d_logits"):
            if k in L:
                L[k].fill_(7.0)
        for g in L["grads"].values():
            g.fill_(7.0)
    torch.cuda.synchronize()
    moe.moe_stack_fwd(pb, layers, keep, dsaved, cs, events, ws)
    moe.moe_stack_bwd(pb, layers, keep, dsaved, cs, events, ws)
    torch.cuda.synchronize()
    return _snapshot(layers)


CASES = {
    "ragged_bf16_x4": (LayerConfig("ragged", T=300, d=136, E=6, k=3, F=200, r=16, dtype="bf16",
                                   alpha=32.0, router_grad=True), 4),
    "ragged_bf16_x3": (LayerConfig("ragged", T=300, d=136, E=6, k=3, F=200, r=16, dtype="bf16",
                                   alpha=32.0), 3),
    "tiny_fp32_x5": (synth.get_config("tiny_fp32"), 5),
    "ragged_bf16_x2": (LayerConfig("ragged", T=300, d=136, E=6, k=3, F=200, r=16, dtype="bf16",
                                   alpha=32.0), 2),
    "ragged_bf16_x1": (LayerConfig("ragged", T=300, d=136, E=6, k=3, F=200, r=16, dtype="bf16",
                                   alpha=32.0), 1),
    # Qwen3-30B-A3B shapes on 2048 tokens: 80 MB of activations per layer, so
    # the copies take milliseconds and really run beside the compute
    "qwen3_2048_x4": (synth.get_config("qwen3_30b_a3b").with_(T=2048), 4),
}


@pytest.mark.parametrize("name", list(CASES))
def test_stack_offload_is_bit_identical_to_per_layer_buffers(name):
    cfg, n = CASES[name]
    print(f"[stack] {name}", flush=True)
    dev = torch.device("cuda:0")
    keep = cfg.router_grad
    pb, layers = _make_stack(cfg, n, dev)
    ref = _run_per_layer(cfg, pb, layers, keep, dev)
    got = _run_stack(cfg, pb, layers, keep, dev)
    for i, (a, b) in enumerate(zip(got, ref)):
        for k in b:
            assert torch.equal(a[k], b[k]), f"{name}: layer {i} {k} differs"
