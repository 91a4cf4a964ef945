"""moe_route_noalloc (the routing call that allocates nothing, for callers
under graph capture or in loops that cannot allocate) against moe_route with
a caller workspace: bit-identical routing, on two calls in a row on the same
GPU (the second with a smaller batch, so it runs on what the first left in
the shared scratch array), with and without the pinned count readback."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_layer_lora_amd as moe  # noqa: E402
import synth  # noqa: E402
from synth.configs import LayerConfig  # noqa: E402

pytestmark = pytest.mark.gpu

ROUTING = ("topk_idx", "topk_w", "counts", "offsets", "sorted_slot", "slot_row")


def _route_both(cfg, seed, host_counts):
    dev = torch.device("cuda:0")
    pb = moe.Problem.from_config(cfg)
    logits = torch.from_numpy(synth.make_inputs(cfg, seed=seed, with_dout=False)["logits"]).to(dev)
    ref = moe.alloc_routing(pb, dev)
    ws = moe.alloc_bytes(moe.route_workspace(pb), dev)
    moe.moe_route(pb, logits, ref, ws=ws)
    got = {n: torch.full_like(v, -7) for n, v in ref.items()}  # stale values must all be overwritten
    moe.moe_route_noalloc(pb, logits, got, host_counts=host_counts)
    torch.cuda.synchronize()
    for n in ROUTING:
        assert torch.equal(got[n], ref[n]), f"{cfg.name}: {n} differs from moe_route"
    if host_counts is not None:
        assert np.array_equal(host_counts.numpy(), ref["counts"].cpu().numpy())


def test_noalloc_route_matches_route_twice_second_smaller():
    big = synth.get_config("qwen3_30b_a3b")                      # 256 token blocks x 128 experts
    small = LayerConfig("small", T=300, d=64, E=6, k=3, F=64, r=8, dtype="bf16", alpha=16.0)
    print("[noalloc] qwen3_30b_a3b then T=300 E=6", flush=True)
    _route_both(big, seed=0, host_counts=None)
    hc = torch.zeros(small.E, dtype=torch.int32, pin_memory=True)
    _route_both(small, seed=1, host_counts=hc)


def test_noalloc_route_largest_histogram_then_empty_batch():
    """E = 1024 experts at 65536 tokens fills the histogram bound; then T = 0."""
    big = LayerConfig("e1024", T=65536, d=64, E=1024, k=4, F=64, r=8, dtype="bf16", alpha=16.0)
    print("[noalloc] E=1024 T=65536 then T=0", flush=True)
    _route_both(big, seed=2, host_counts=torch.zeros(1024, dtype=torch.int32, pin_memory=True))
    empty = LayerConfig("empty", T=0, d=64, E=4, k=2, F=64, r=8, dtype="bf16", alpha=16.0)
    pb = moe.Problem.from_config(empty)
    rt = moe.alloc_routing(pb, torch.device("cuda:0"))
    moe.moe_route_noalloc(pb, None, rt)
    torch.cuda.synchronize()
    assert rt["offsets"].cpu().numpy().tolist() == [0] * 5 and torch.all(rt["counts"] == 0)


def test_noalloc_route_refuses_pageable_counts():
    cfg = LayerConfig("small", T=64, d=64, E=8, k=2, F=64, r=8, dtype="bf16", alpha=16.0)
    pb = moe.Problem.from_config(cfg)
    dev = torch.device("cuda:0")
    logits = torch.zeros((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    rt = moe.alloc_routing(pb, dev)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route_noalloc(pb, logits, rt, host_counts=np.zeros(cfg.E, np.int32))
    assert ei.value.status == moe.MOE_E_ARG
