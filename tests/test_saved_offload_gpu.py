"""Offload of the saved activations to pinned host memory and their reload
(moe_saved_copy) on a copy stream: a backward that reads the reloaded buffer
must give bit-identical results to one that reads the buffer moe_fwd wrote."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from synth.configs import LayerConfig  # noqa: E402

pytestmark = pytest.mark.gpu


def test_offload_reload_round_trip_is_bit_exact():
    import layer_runner as lr
    import moe_layer_lora_amd as moe
    cfg = LayerConfig("offload_bf16", T=300, d=136, E=6, k=3, F=200, r=16, dtype="bf16", alpha=32.0,
                      router_grad=True)
    inp = synth.make_inputs(cfg, seed=0)
    L = lr.Layer(cfg, inp, keep_expert_out=True)
    L.step(backward=True, router_grad=True)
    ref = L.results(backward=True, router_grad=True)
    pb = L.pb
    n = moe.saved_bytes(pb, True)
    assert L.saved.numel() >= n
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    ev_fwd, ev_off, ev_zero, ev_back = (torch.cuda.Event() for _ in range(4))
    for e in (ev_off, ev_back):  # make the events exist before the library records them
        e.record(compute)
    print(f"[offload] {n} bytes of saved activations", flush=True)
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
    assert torch.equal(host.to(before.device), before)
    assert torch.equal(L.saved[:n], before)
    for name in ("dx", "da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down", "d_topk_w",
                 "d_logits"):
        assert np.array_equal(got[name], ref[name]), name


def test_pageable_host_memory_is_rejected():
    import moe_layer_lora_amd as moe
    cfg = LayerConfig("offload_small", T=64, d=64, E=4, k=2, F=64, r=8, dtype="bf16", alpha=16.0)
    pb = moe.Problem.from_config(cfg)
    dev = torch.device("cuda")
    saved = moe.alloc_bytes(moe.saved_bytes(pb, False), dev)
    host = np.zeros(moe.saved_bytes(pb, False), np.uint8)  # pageable
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_saved_copy(pb, False, False, saved, host.ctypes.data, copy_stream=torch.cuda.Stream())
    assert ei.value.status == moe.MOE_E_ARG
