"""Offload of the saved activations to pinned host memory and their reload
(moe_saved_copy) on a copy stream: the host copy holds everything but H, the
reload rebuilds H from G and U, and the reloaded buffer must equal the one
moe_fwd wrote byte for byte, so the backward gives bit-identical results."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from synth.configs import LayerConfig  # noqa: E402

pytestmark = pytest.mark.gpu


ROUND_TRIP = {
    "ragged_bf16": LayerConfig("offload_bf16", T=300, d=136, E=6, k=3, F=200, r=16, dtype="bf16",
                               alpha=32.0, router_grad=True),
    "ragged_f32": LayerConfig("offload_f32", T=300, d=136, E=6, k=3, F=200, r=16, dtype="f32",
                              alpha=32.0, router_grad=True),
}


@pytest.mark.parametrize("name", list(ROUND_TRIP))
def test_offload_reload_round_trip_is_bit_exact(name):
    import layer_runner as lr
    import moe_layer_lora_amd as moe
    cfg = ROUND_TRIP[name]
    inp = synth.make_inputs(cfg, seed=0)
    L = lr.Layer(cfg, inp, keep_expert_out=True)
    L.step(backward=True, router_grad=True)
    ref = L.results(backward=True, router_grad=True)
    pb = L.pb
    n, nh = moe.saved_bytes(pb, True), moe.saved_host_bytes(pb, True)
    assert L.saved.numel() >= n and 0 < nh < n
    host = torch.empty(nh, dtype=torch.uint8, pin_memory=True)
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    ev_fwd, ev_off, ev_zero, ev_back = (torch.cuda.Event() for _ in range(4))
    for e in (ev_off, ev_back):  # make the events exist before the library records them
        e.record(compute)
    print(f"[offload] {name}: {nh} of {n} bytes of saved activations", flush=True)
    L.fwd()
    ev_fwd.record(compute)
    moe.moe_saved_copy(pb, True, False, L.saved, host, wait_event=ev_fwd, copy_stream=copy,
                       done_event=ev_off)
    compute.wait_event(ev_off)
    before = L.saved[:n].clone()
    L.saved.zero_()  # the device copy is gone; only the host copy remains
    ev_zero.record(compute)
    moe.moe_saved_copy(pb, True, True, L.saved, host, wait_event=ev_zero, copy_stream=copy,
                       done_event=ev_back)
    compute.wait_event(ev_back)
    L.bwd(router_grad=True)
    got = L.results(backward=True, router_grad=True)
    for k in ("dx", "da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down", "d_topk_w", "d_logits"):
        assert np.array_equal(got[k], ref[k]), f"{name}: {k}"
    assert torch.equal(host.to(before.device), before[:nh])
    # H (last; its alignment padding holds nothing) rebuilt bit for bit
    h_end = nh + pb.S * pb.F * (2 if cfg.dtype == "bf16" else 4)
    assert h_end <= n
    assert torch.equal(L.saved[:h_end], before[:h_end])


def test_pageable_host_memory_is_rejected():
    import moe_layer_lora_amd as moe
    cfg = LayerConfig("offload_small", T=64, d=64, E=4, k=2, F=64, r=8, dtype="bf16", alpha=16.0)
    pb = moe.Problem.from_config(cfg)
    dev = torch.device("cuda")
    saved = moe.alloc_bytes(moe.saved_bytes(pb, False), dev)
    host = np.zeros(moe.saved_host_bytes(pb, False), np.uint8)  # pageable
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_saved_copy(pb, False, False, saved, host.ctypes.data, copy_stream=torch.cuda.Stream())
    assert ei.value.status == moe.MOE_E_ARG
