"""Run the HIP layer (through the C ABI binding) on stored synth inputs.

Test helper: moves inputs to the GPU, calls moe_route / moe_fwd / moe_bwd and
returns every output as numpy (floats widened to float64, routing as int32).
"""
from __future__ import annotations

import numpy as np
import torch

import moe_layer_lora_amd as moe
import synth

WEIGHTS = ("w_gate", "w_up", "w_down", "a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


def to_dev(a: np.ndarray, device="cuda"):
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return synth.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


class Layer:
    """Device copies of one layer's inputs and every buffer the three calls need."""

    def __init__(self, cfg, inputs: dict, T=None, device="cuda", keep_expert_out=False,
                 training=True, q4=None):
        self.cfg = cfg
        self.pb = moe.Problem.from_config(cfg, T=T)
        self.device = device
        self.keep = keep_expert_out
        self.training = training
        pb = self.pb
        self.dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.x = to_dev(inputs["x"], device)
        self.logits = to_dev(inputs["logits"], device)
        # q4: NF4 base weights (codes_* / scales_* numpy arrays): the forward and
        # backward then take them through moe_fwd_nf4 / moe_bwd_nf4
        self.q4 = None if q4 is None else {n: to_dev(v, device) for n, v in q4.items()}
        self.w = {n: to_dev(inputs[n], device) for n in WEIGHTS
                  if q4 is None or n not in ("w_gate", "w_up", "w_down")}
        self.dout = to_dev(inputs["dout"], device) if "dout" in inputs else None
        self.rt = moe.alloc_routing(pb, device)
        self.ws_route = moe.alloc_bytes(moe.route_workspace(pb), device)
        self.ws_fwd = moe.alloc_bytes(moe.fwd_workspace(pb, training, keep_expert_out), device)
        self.saved = moe.alloc_bytes(moe.saved_bytes(pb, keep_expert_out), device) if training else None
        self.out = torch.empty((pb.T, pb.d), dtype=self.dt, device=device)
        if training:
            self.ws_bwd = moe.alloc_bytes(moe.bwd_workspace(pb), device)
            self.dx = torch.empty((pb.T, pb.d), dtype=self.dt, device=device)
            self.grads = moe.alloc_grads(pb, device)
            self.d_topk_w = torch.empty((pb.T, pb.k), dtype=torch.float32, device=device)
            self.d_logits = torch.empty((pb.T, pb.E), dtype=torch.float32, device=device)

    def route(self, host_counts=None):
        moe.moe_route(self.pb, self.logits, self.rt, host_counts=host_counts, ws=self.ws_route)

    def fwd(self):
        if self.q4 is not None:
            moe.moe_fwd_nf4(self.pb, self.x, self.rt, self.w, self.q4, self.out, saved=self.saved,
                            keep_expert_out=self.keep, ws=self.ws_fwd)
            return
        moe.moe_fwd(self.pb, self.x, self.rt, self.w, self.out, saved=self.saved,
                    keep_expert_out=self.keep, ws=self.ws_fwd)

    def bwd(self, router_grad=False):
        if self.q4 is not None:
            moe.moe_bwd_nf4(self.pb, self.x, self.dout, self.rt, self.w, self.q4, self.saved, self.keep,
                            self.dx, self.grads, d_topk_w=self.d_topk_w if router_grad else None,
                            d_logits=self.d_logits if router_grad else None, ws=self.ws_bwd)
            return
        moe.moe_bwd(self.pb, self.x, self.dout, self.rt, self.w, self.saved, self.keep, self.dx,
                    self.grads, d_topk_w=self.d_topk_w if router_grad else None,
                    d_logits=self.d_logits if router_grad else None, ws=self.ws_bwd)

    def step(self, backward=True, router_grad=False):
        self.route()
        self.fwd()
        if backward:
            self.bwd(router_grad)

    def results(self, backward=True, router_grad=False, intermediates=False) -> dict:
        torch.cuda.synchronize()
        r = {n: self.rt[n].cpu().numpy() for n in ("topk_idx", "counts", "offsets", "sorted_slot",
                                                   "slot_row")}
        r["topk_w"] = self.rt["topk_w"].cpu().numpy().astype(np.float64)
        r["out"] = to_f64(self.out)
        if intermediates and self.training:
            for n, v in moe.saved_views(self.pb, self.saved, self.keep).items():
                r[n] = to_f64(v)
        if intermediates:
            ws = moe.workspace_views(self.pb, ws_fwd=self.ws_fwd,
                                     ws_bwd=self.ws_bwd if (backward and self.training) else None,
                                     training=self.training, keep_expert_out=self.keep)
            for n, v in ws.items():
                r[n] = to_f64(v)
        if backward:
            r["dx"] = to_f64(self.dx)
            for n, v in self.grads.items():
                r[n] = to_f64(v)
            if router_grad:
                r["d_topk_w"] = to_f64(self.d_topk_w)
                r["d_logits"] = to_f64(self.d_logits)
        return r


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)
