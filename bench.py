"""Benchmark of the MoE expert layer (routing + grouped GEMMs with Split-LoRA,
forward + backward) on one MI355X.

A step is one pass of the whole hot path over one batch of the workload:
moe_route (with the one count readback to the host) + moe_fwd + moe_bwd.
Inputs are seeded synthetic tensors with the workload's shapes and
distributions, resident in HBM before timing starts. Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload qwen3_30b_a3b]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 MFMA/vector
PEAK_HBM_GBS = 8000.0

METRIC = "MoE layer fwd+bwd tokens/s; grouped-GEMM TFLOP/s as % of bf16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_30b_a3b")
    ap.add_argument("--no-readback", action="store_true",
                    help="route without copying the expert counts to the host")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of the workload the CPU oracle baseline runs on (all cores)")
    ap.add_argument("--cpu-tokens-1t", type=int, default=128,
                    help="tokens of the workload for the single-thread oracle run")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--no-other-workloads", dest="other_workloads", action="store_false",
                    help="skip the timing of the other configurations")
    ap.add_argument("--other-steps", type=int, default=10)
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the HIP-graph replay of the step")
    ap.add_argument("--no-nf4", dest="nf4", action="store_false",
                    help="skip the step on 4-bit NormalFloat base weights")
    ap.add_argument("--offload-reps", type=int, default=3,
                    help="repetitions of the stacked-layer offload measurement (0 = skip)")
    ap.add_argument("--offload-layers", type=int, default=4,
                    help="layers in the stacked-layer offload measurement")
    ap.add_argument("--whereloop-steps", type=int, default=3,
                    help="steps of the per-expert where() loop baseline (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before warm-up, run a plain device copy (y = -x, fp32) of MIB MiB "
                         "three times: the known-size kernel that scales rocprofv3's "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes")
    return ap.parse_args()


def gemm_flops_per_slot(c):
    d, F, r = c.d, c.F, c.r
    return {
        "proj_gu": 4 * d * r, "gateup": 4 * d * F + 4 * r * F, "proj_d": 2 * F * r,
        "down": 2 * d * F + 2 * d * r, "proj_dout": 2 * d * r, "down_bwd": 2 * d * F + 2 * r * F,
        "proj_dgu": 4 * F * r, "gateup_bwd": 4 * d * F + 4 * r * d, "lora_grad": 6 * r * (d + F),
    }


class Hip:
    """hipEvent_* from the HIP runtime torch has loaded (same soname)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev.value

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def kernel_source_hash():
    """Hash of the HIP sources and build flags: a counter summary taken on other
    sources no longer describes the kernels being timed."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_layer_lora_amd", "csrc")
    for n in sorted(os.listdir(csrc)):
        if n.endswith((".hip", ".hpp")):
            h.update(n.encode())
            with open(os.path.join(csrc, n), "rb") as f:
                h.update(f.read())
    with open(os.path.join(ROOT, "moe_layer_lora_amd", "_build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


# the other configurations the bench line also times (parity cases of the
# tests; the headline metric is the workload above)
OTHER_WORKLOADS = ("gptoss20b", "qwen3_30b_a3b_skewed", "gptoss120b")


def profile_values(name):
    """The `- key: value` lines of a committed rocprofv3 summary under
    profiles/, or None if it is absent or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                kv[k.strip()] = v.strip().strip("`")
    if kv.get("source_hash") != kernel_source_hash():
        return None
    return kv


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated on a copy kernel), or None if
    there is none for these sources."""
    kv = profile_values(f"hbm_traffic_{kernel}_{workload}.md")
    try:
        return int(kv["fetch_bytes_per_launch"]) + int(kv["write_bytes_per_launch"])
    except (TypeError, KeyError, ValueError):
        return None


def measured_clock(kernel, workload):
    """Shader clock (GHz) while `kernel` runs, from the committed counter
    summary: GRBM_GUI_ACTIVE cycles per XCD over the kernel-trace duration.
    The counter window also spans the dispatch, so this bounds the clock from
    above; None if there is no summary for these sources."""
    kv = profile_values(f"counters_{workload}.md")
    try:
        return float(kv[f"clock_ghz_{kernel}"])
    except (TypeError, KeyError, ValueError):
        return None


def copy_calibration(torch, mib, dev):
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


def cpu_baseline(cfg, tokens, tokens_1t):
    """The fp64 row-loop oracle as it stands, on the first `tokens` tokens of
    the same layer with all of its OpenMP threads, and on the first
    `tokens_1t` with one thread: seconds per phase and GFLOP/s of the
    algorithmic GEMM work."""
    import oracle
    import synth

    def run(ntok, threads):
        inputs = synth.make_inputs(cfg, seed=0, tokens=ntok, with_dout=cfg.backward)
        L = oracle.Layer.from_config(cfg, inputs, tokens=ntok)
        oracle.set_threads(threads)
        t0 = time.perf_counter()
        rt = oracle.route(inputs["logits"], cfg.k)
        t1 = time.perf_counter()
        oracle.fwd(L, rt)
        t2 = time.perf_counter()
        if cfg.backward:
            oracle.bwd(L, rt, inputs["dout"])
        t3 = time.perf_counter()
        flops = cfg.with_(T=ntok).gemm_flops()["total"]
        return {"tokens": ntok, "threads": threads, "route_s": round(t1 - t0, 4),
                "fwd_s": round(t2 - t1, 3), "bwd_s": round(t3 - t2, 3), "seconds": round(t3 - t0, 3),
                "tokens_per_s": round(ntok / (t3 - t0), 2), "gflops": round(flops / (t3 - t0) / 1e9, 3)}

    nthreads = oracle.threads()
    all_cores = run(tokens, nthreads)
    single = run(tokens_1t, 1)
    oracle.set_threads(nthreads)
    return {"value": all_cores["tokens_per_s"], "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "cpu_model": cpu_model(), "all_cores": all_cores, "single_thread": single,
            "sample": f"first {tokens} (all {nthreads} threads) and first {tokens_1t} (one thread) of "
                      f"the {cfg.T} tokens of the same layer (same weights and generator), route+fwd" +
                      ("+bwd" if cfg.backward else "") + "; fp64 row loops, OpenMP over experts; bwd "
                      "recomputes each row's forward; gflops = algorithmic GEMM flops / seconds"}


def whereloop_baseline(torch, cfg, x, logits, w, dout, steps, warmup=1):
    """The per-expert loop that sorted routing and the grouped GEMM replace, in
    plain PyTorch on the same GPU and inputs: top-k + softmax over the selected
    logits, then for every expert a where() over the routing table (one host
    sync each, to size the gather), a gathered copy of its tokens, its SwiGLU
    MLP with the LoRA terms added after the base product, and a weighted
    index_add into the output; the backward is autograd over x and the LoRA
    factors (base weights frozen). Library GEMMs (hipBLASLt) do the products.
    Returns ms per step (forward, backward) and the output it computed."""
    E, k, s = cfg.E, cfg.k, cfg.s
    # frozen base weights transposed once, outside the timed region
    wt = {n: w[n].transpose(1, 2).contiguous() for n in ("w_gate", "w_up", "w_down")}
    lora = {n: w[n].detach().clone().requires_grad_(True)
            for n in ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")}
    xr = x.detach().clone().requires_grad_(cfg.backward)

    def lin(h, e, base, a, b):  # h W^T + s (h A^T) B^T, never forming W + s B A
        return h @ wt[base][e] + s * ((h @ lora[a][e].t()) @ lora[b][e].t())

    def forward():
        top = torch.topk(logits, k, dim=1)
        wts = torch.softmax(top.values, dim=1)
        out = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device=x.device)
        for e in range(E):
            tok, j = torch.where(top.indices == e)
            if tok.numel() == 0:
                continue
            h = xr[tok]
            g = lin(h, e, "w_gate", "a_gate", "b_gate")
            u = lin(h, e, "w_up", "a_up", "b_up")
            y = lin(torch.nn.functional.silu(g) * u, e, "w_down", "a_down", "b_down")
            out = out.index_add(0, tok, wts[tok, j, None] * y.float())
        return out

    fwd_ms, bwd_ms, out = [], [], None
    for it in range(warmup + steps):
        for t in list(lora.values()) + [xr]:
            t.grad = None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.set_grad_enabled(cfg.backward):
            out = forward()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if cfg.backward:
            out.backward(dout.float())
            torch.cuda.synchronize()
        t2 = time.perf_counter()
        if it >= warmup:
            fwd_ms.append((t1 - t0) * 1e3)
            bwd_ms.append((t2 - t1) * 1e3)
    return sum(fwd_ms) / steps, sum(bwd_ms) / steps, out.detach()


def router_bench(torch, moe, synth, cfg, pb, x, hip, dev, iters=20):
    """The router projection in front of the layer (logits = x W_r^T) and its
    backward (dx += d_logits W_r; dW_r = d_logits^T x), timed with events on
    its own: ms per call and TF/s (2 T d E flops per product)."""
    import numpy as np
    ri = synth.make_router(cfg, seed=0)
    w_r = torch.from_numpy(ri["w_router"].view(np.int16)).to(dev).view(torch.bfloat16)
    dl = torch.from_numpy(ri["d_logits"]).to(dev)
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    dxr = torch.zeros((cfg.T, cfg.d), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((cfg.E, cfg.d), dtype=torch.float32, device=dev)
    ws = moe.alloc_bytes(moe.router_workspace(pb), dev)
    names = ("router_logits", "router_dx", "router_dw")
    traces = []
    for _ in range(iters):
        tr = moe.Trace()
        for n in names:
            k = moe.KERNELS.index(n)
            tr.start[k], tr.stop[k] = hip.event(), hip.event()
        traces.append(tr)
    stream = torch.cuda.current_stream()
    for it in range(3 + iters):
        tr = traces[it - 3] if it >= 3 else None
        moe.moe_router_fwd(pb, x, w_r, logits, stream=stream, trace=tr)
        moe.moe_router_bwd(pb, x, w_r, dl, dx_in=dxr, dx=dxr, dw_router=dw, ws=ws, stream=stream,
                           trace=tr)
    torch.cuda.synchronize()
    ms = {}
    for n in names:
        k = moe.KERNELS.index(n)
        ms[n] = sum(hip.elapsed_ms(tr.start[k], tr.stop[k]) for tr in traces) / iters
    for tr in traces:
        for n in names:
            k = moe.KERNELS.index(n)
            hip.destroy(tr.start[k])
            hip.destroy(tr.stop[k])
    f_ms, b_ms = ms["router_logits"], ms["router_dx"] + ms["router_dw"]
    fl = 2.0 * cfg.T * cfg.d * cfg.E
    return {"fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
            "kernels_ms": {n: round(v, 4) for n, v in ms.items()},
            "fwd_tflops": round(fl / (f_ms * 1e-3) / 1e12, 1),
            "bwd_tflops": round(2 * fl / (b_ms * 1e-3) / 1e12, 1),
            "note": "not part of the step: the workloads take logits as an input"}


def stack_offload_bench(torch, moe, cfg, pb, x, logits, w, dout, keep, n=4, reps=3):
    """n stacked layers of the workload's shape (the step's weights in every
    layer, each layer's logits rolled by its index so each routes differently;
    layer i+1's input is layer i's output) forward + backward, timed (a) with
    a device `saved` buffer per layer and (b) with moe_stack_fwd / bwd, which
    offload layers 0 .. n-3 to pinned host memory and reload them
    double-buffered. Also the time of one layer's copy each way alone, so the
    share of the copies the schedule hides is measured, not assumed. A copy
    moves `saved` without H (rebuilt from G and U on the reload)."""
    dev = x.device
    dt = x.dtype
    nbytes, nhost = moe.saved_bytes(pb, keep), moe.saved_host_bytes(pb, keep)
    layers = []
    for i in range(n):
        L = {"logits": torch.roll(logits, shifts=i, dims=1).contiguous(), "w": w,
             "rt": moe.alloc_routing(pb, dev), "grads": moe.alloc_grads(pb, dev),
             "out": torch.empty_like(x), "dx": torch.empty_like(x),
             "host_saved": torch.empty(nhost, dtype=torch.uint8, pin_memory=True) if i <= n - 3 else None}
        layers.append(L)
    for i, L in enumerate(layers):
        L["x"] = x if i == 0 else layers[i - 1]["out"]
        L["dout"] = dout if i == n - 1 else layers[i + 1]["dx"]
    per_layer = [moe.alloc_bytes(nbytes, dev) for _ in range(n)]
    ws_r = moe.alloc_bytes(moe.route_workspace(pb), dev)
    ws_f = moe.alloc_bytes(moe.fwd_workspace(pb, True, keep), dev)
    ws_b = moe.alloc_bytes(moe.bwd_workspace(pb), dev)
    dsaved = [moe.alloc_bytes(nbytes, dev) for _ in range(2)]
    ws = moe.alloc_bytes(moe.stack_workspace(pb, keep), dev)
    cs = torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(4)]
    for e in events:  # torch creates the HIP event at its first record
        e.record()

    def resident():
        for L, sv in zip(layers, per_layer):
            moe.moe_route(pb, L["logits"], L["rt"], ws=ws_r)
            moe.moe_fwd(pb, L["x"], L["rt"], L["w"], L["out"], saved=sv, keep_expert_out=keep, ws=ws_f)
        for L, sv in reversed(list(zip(layers, per_layer))):
            moe.moe_bwd(pb, L["x"], L["dout"], L["rt"], L["w"], sv, keep, L["dx"], L["grads"], ws=ws_b)

    def offloaded():
        moe.moe_stack_fwd(pb, layers, keep, dsaved, cs, events, ws)
        moe.moe_stack_bwd(pb, layers, keep, dsaved, cs, events, ws)

    def timed(fn):
        ts = []
        for _ in range(reps + 1):  # the first run warms up
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        return sorted(ts[1:])[len(ts[1:]) // 2] * 1e3

    t_res = timed(resident)
    ref_dx = layers[0]["dx"].clone()
    t_off = timed(offloaded)
    same = bool(torch.equal(layers[0]["dx"], ref_dx))
    host = layers[0]["host_saved"]
    d2h = timed(lambda: moe.moe_saved_copy(pb, keep, False, dsaved[0], host, copy_stream=cs))
    h2d = timed(lambda: moe.moe_saved_copy(pb, keep, True, dsaved[0], host, copy_stream=cs))
    copies = (n - 2) * (d2h + h2d)
    hidden = 1.0 - (t_off - t_res) / copies if copies > 0 else None
    return {"layers": n, "saved_bytes_per_layer": nbytes, "copied_bytes_per_layer": nhost,
            "device_activation_bytes": {"per_layer_buffers": n * nbytes, "double_buffered": 2 * nbytes},
            "fwd_bwd_ms_per_layer_buffers": round(t_res, 3), "fwd_bwd_ms_offloaded": round(t_off, 3),
            "copy_ms_per_layer": {"d2h": round(d2h, 3), "h2d": round(h2d, 3)},
            "copy_GBs": {"d2h": round(nhost / d2h / 1e6, 1), "h2d": round(nhost / h2d / 1e6, 1)},
            "copies_ms_total": round(copies, 3),
            "hidden_fraction": None if hidden is None else round(max(0.0, min(1.0, hidden)), 3),
            "dx_equal_to_per_layer_buffers": same,
            "note": "median of %d runs each; hidden_fraction = 1 - (offloaded - resident) / (time of the "
                    "2(n-2) copies alone); layers n-2 and n-1 stay on the device; h2d includes the "
                    "rebuild of H from G and U" % reps}


def nf4_step_bench(torch, moe, synth, cfg, pb, ctx, hip, bf16_step_ms, steps, warmup):
    """The same step with the frozen base weights W_g, W_u, W_d in 4-bit
    NormalFloat (codes + one fp32 scale per 64 weights; random codes, scales
    for a weight standard deviation of about 0.02): moe_fwd_nf4 / moe_bwd_nf4
    dequantise every weight tile as the grouped GEMMs stage it into LDS, so no
    bf16 copy of a weight exists. Step time against the bf16 step, the four
    grouped GEMMs' times, and the weight bytes each form keeps resident."""
    dev = ctx["x"].device
    keys = (("gate", cfg.E * cfg.F, cfg.d, 20), ("up", cfg.E * cfg.F, cfg.d, 21),
            ("down", cfg.E * cfg.d, cfg.F, 22))
    if cfg.d % 64 or cfg.F % 64:
        return None
    q4 = {}
    for name, rows, cols, tau in keys:
        q = synth.make_nf4(rows, cols, seed=0, tensor=tau)
        q4["codes_" + name] = torch.from_numpy(q["codes"]).to(dev)
        q4["scales_" + name] = torch.from_numpy(q["scales"]).to(dev)
    lora = {k: v for k, v in ctx["w"].items() if not k.startswith("w_")}
    keep = ctx["keep"]
    st = torch.cuda.current_stream()

    def step(trace=None):
        moe.moe_route(pb, ctx["logits"], ctx["rt"], ws=ctx["ws_r"], stream=st, trace=trace)
        moe.moe_fwd_nf4(pb, ctx["x"], ctx["rt"], lora, q4, ctx["out"], saved=ctx["saved"], keep_expert_out=keep,
                        ws=ctx["ws_f"], stream=st, trace=trace)
        if cfg.backward:
            moe.moe_bwd_nf4(pb, ctx["x"], ctx["dout"], ctx["rt"], lora, q4, ctx["saved"], keep, ctx["dx"],
                            ctx["grads"], d_topk_w=ctx["dtw"], d_logits=ctx["dlg"], ws=ctx["ws_b"], stream=st,
                            trace=trace)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(hip.event(), hip.event()) for _ in range(steps)]
    for a, b in ev:
        hip.record(a, st.cuda_stream)
        step()
        hip.record(b, st.cuda_stream)
    torch.cuda.synchronize()
    ms = sorted(hip.elapsed_ms(a, b) for a, b in ev)
    # per-GEMM times from traced steps after the timed ones
    names = [n for n in ("gateup", "down", "down_bwd", "gateup_bwd") if cfg.backward or n in ("gateup", "down")]
    traces = []
    for _ in range(min(steps, 10)):
        tr = moe.Trace()
        for n in names:
            i = moe.KERNELS.index(n)
            tr.start[i], tr.stop[i] = hip.event(), hip.event()
        traces.append(tr)
        step(tr)
    torch.cuda.synchronize()
    kms = {}
    for n in names:
        i = moe.KERNELS.index(n)
        v = [hip.elapsed_ms(tr.start[i], tr.stop[i]) for tr in traces]
        kms[n] = round(sum(v) / len(v), 4)
    for tr in traces:
        for n in names:
            i = moe.KERNELS.index(n)
            hip.destroy(tr.start[i])
            hip.destroy(tr.stop[i])
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    med = ms[len(ms) // 2]
    nf4_bytes = sum(v.numel() * v.element_size() for v in q4.values())
    bf16_bytes = sum(rows * cols * 2 for _, rows, cols, _ in keys)
    return {"ms_per_step_median": round(med, 4), "ms_per_step_min": round(ms[0], 4),
            "ratio_to_bf16_step": round(med / bf16_step_ms, 3), "gemm_kernels_ms": kms,
            "base_weight_bytes": {"nf4": int(nf4_bytes), "bf16": int(bf16_bytes)},
            "note": "route + moe_fwd_nf4 + moe_bwd_nf4: NF4 codes dequantised inside the grouped GEMMs' "
                    "B-tile staging; no dequantisation pass, no bf16 weight copy"}


def graph_replay(torch, step, out, dx, steps):
    """The same step captured once in a HIP graph and replayed: ms per step
    (no per-kernel launch work on the host), and whether a replay's outputs
    equal the eager step's bit for bit."""
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, dx) if t is not None]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(st=s)
    torch.cuda.current_stream().wait_stream(s)
    for t in (out, dx):
        if t is not None:
            t.zero_()
    g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(ref, [t for t in (out, dx) if t is not None]))
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    del g
    return {"ms_per_step": round(ms, 4), "replay_equals_eager": bool(same),
            "note": "same step captured once and replayed; value above is the eager step"}


class Setup:
    pass


def setup(torch, np, moe, synth, cfg, dev, no_readback=False):
    """Seeded synthetic inputs of the workload in HBM, the library's buffers
    and workspaces, and the step (route + fwd + bwd) as a closure."""
    W = Setup()
    W.cfg = cfg
    W.pb = pb = moe.Problem.from_config(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    t_gen = time.perf_counter()
    inputs = synth.make_inputs(cfg, seed=0, with_dout=cfg.backward)
    W.x, W.logits = up(inputs["x"]), up(inputs["logits"])
    names = ("w_gate", "w_up", "w_down", "a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")
    W.w = {n: up(inputs[n]) for n in names}
    W.dout = up(inputs["dout"]) if cfg.backward else None
    del inputs
    W.t_gen = time.perf_counter() - t_gen

    W.keep = keep = cfg.router_grad
    W.rt = moe.alloc_routing(pb, dev)
    W.ws_r = moe.alloc_bytes(moe.route_workspace(pb), dev)
    W.ws_f = moe.alloc_bytes(moe.fwd_workspace(pb, cfg.backward, keep), dev)
    W.saved = moe.alloc_bytes(moe.saved_bytes(pb, keep), dev) if cfg.backward else None
    W.out = torch.empty((cfg.T, cfg.d), dtype=dt, device=dev)
    W.ws_b = W.dx = W.grads = W.dtw = W.dlg = None
    if cfg.backward:
        W.ws_b = moe.alloc_bytes(moe.bwd_workspace(pb), dev)
        W.dx = torch.empty((cfg.T, cfg.d), dtype=dt, device=dev)
        W.grads = moe.alloc_grads(pb, dev)
        W.dtw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev) if keep else None
        W.dlg = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev) if keep else None
    # pinned: the count readback is a stream-ordered copy that needs no host wait
    host_counts = torch.zeros(cfg.E, dtype=torch.int32, pin_memory=True)
    W.stream = stream = torch.cuda.current_stream()

    def step(trace=None, st=None):
        st = stream if st is None else st
        moe.moe_route(pb, W.logits, W.rt, host_counts=None if no_readback else host_counts,
                      ws=W.ws_r, stream=st, trace=trace)
        moe.moe_fwd(pb, W.x, W.rt, W.w, W.out, saved=W.saved, keep_expert_out=keep, ws=W.ws_f,
                    stream=st, trace=trace)
        if cfg.backward:
            moe.moe_bwd(pb, W.x, W.dout, W.rt, W.w, W.saved, keep, W.dx, W.grads, d_topk_w=W.dtw,
                        d_logits=W.dlg, ws=W.ws_b, stream=st, trace=trace)
    W.step = step
    return W


def other_workload(torch, np, moe, synth, hip, name, steps, warmup):
    """One of the other configurations: route + fwd (+ bwd) timed like the
    headline step (per-step HIP events, median), with the grouped GEMMs'
    rate from one traced step after the timed ones."""
    cfg = synth.get_config(name)
    dev = torch.device("cuda:0")
    W = setup(torch, np, moe, synth, cfg, dev)
    for _ in range(warmup):
        W.step()
    torch.cuda.synchronize()
    sh = W.stream.cuda_stream
    ev = [(hip.event(), hip.event()) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        hip.record(a, sh)
        W.step()
        hip.record(b, sh)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = sorted(hip.elapsed_ms(a, b) for a, b in ev)
    fps = gemm_flops_per_slot(cfg)
    names = [n for n in fps if cfg.backward or n in ("proj_gu", "gateup", "proj_d", "down")]
    tr = moe.Trace()
    tev = []
    for n in names:
        i = moe.KERNELS.index(n)
        tr.start[i], tr.stop[i] = hip.event(), hip.event()
        tev += [tr.start[i], tr.stop[i]]
    W.step(tr)
    torch.cuda.synchronize()
    gemm_ms = sum(hip.elapsed_ms(tr.start[moe.KERNELS.index(n)], tr.stop[moe.KERNELS.index(n)]) for n in names)
    gemm_flops = sum(fps[n] * cfg.S for n in names)
    for e in tev + [e for pair in ev for e in pair]:
        hip.destroy(e)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    rec = {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "F": cfg.F, "r": cfg.r,
           "step": "route(+count readback)+fwd" + ("+bwd" if cfg.backward else "") +
                   ("+router-weight grad" if cfg.router_grad else ""),
           "steps": steps, "warmup": warmup,
           "ms_per_step": round(elapsed / steps * 1e3, 4),
           "step_ms": {"median": round(ms[len(ms) // 2], 4), "min": round(ms[0], 4)},
           "tokens_per_s": round(cfg.T * steps / elapsed, 1),
           "grouped_gemm": {"tflops": round(tflops, 2), "frac_of_peak": round(tflops / peak, 4),
                            "ms": round(gemm_ms, 4), "kernels": names}}
    del W
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for "
              f"{max(args.gpus, world)} GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_layer_lora_amd as moe
    import synth

    cfg = synth.get_config(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W = setup(torch, np, moe, synth, cfg, dev, args.no_readback)
    pb, x, logits, w, dout, rt, out = W.pb, W.x, W.logits, W.w, W.dout, W.rt, W.out
    ws_r, ws_f, saved, keep, step, t_gen = W.ws_r, W.ws_f, W.saved, W.keep, W.step, W.t_gen
    if cfg.backward:
        ws_b, dx, grads, dtw, dlg = W.ws_b, W.dx, W.grads, W.dtw, W.dlg
    stream = W.stream
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration, dev)

    hip = Hip()
    gemm_kernels = [n for n in ("gateup", "down", "down_bwd", "gateup_bwd") if cfg.backward or
                    n in ("gateup", "down")]
    events = []

    def make_trace(names):
        tr = moe.Trace()
        for name in names:
            i = moe.KERNELS.index(name)
            a, b = hip.event(), hip.event()
            tr.start[i], tr.stop[i] = a, b
            events.extend([a, b])
        return tr

    def kernel_ms(traces, names):
        out = {}
        for name in names:
            i = moe.KERNELS.index(name)
            v = [hip.elapsed_ms(tr.start[i], tr.stop[i]) for tr in traces]
            out[name] = sum(v) / len(v)
        return out

    # The timed region records HIP events around the four grouped GEMMs only
    # (an event pair costs a few microseconds of GPU time; one per kernel
    # would add ~5% to the step). The full per-kernel breakdown comes from a
    # separate traced pass after the timed region.
    timed_traces = [make_trace(gemm_kernels) for _ in range(args.steps)]
    all_names = [n for n in moe.KERNELS
                 if (cfg.backward or moe.KERNELS.index(n) < moe.KERNELS.index("router_grad"))
                 and (n != "router_grad" or keep)
                 and n not in ("router_logits", "router_dx", "router_dw")]  # not in the step
    n_breakdown = min(args.steps, 10)
    full_traces = [make_trace(all_names) for _ in range(n_breakdown)]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps (an event pair per step on the launch stream
    # gives each step's own duration: median and min next to the mean)
    step_ev = [(hip.event(), hip.event()) for _ in range(args.steps)]
    events.extend(e for pair in step_ev for e in pair)
    sh = stream.cuda_stream
    t0 = time.perf_counter()
    for s in range(args.steps):
        hip.record(step_ev[s][0], sh)
        step(timed_traces[s])
        hip.record(step_ev[s][1], sh)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(hip.elapsed_ms(a, b) for a, b in step_ev)

    gemm_ms_timed = kernel_ms(timed_traces, gemm_kernels)
    for s in range(n_breakdown):  # untimed: every kernel bracketed by events
        step(full_traces[s])
    torch.cuda.synchronize()
    kern_ms = kernel_ms(full_traces, all_names)
    for ev in events:
        hip.destroy(ev)

    graph = graph_replay(torch, step, out, dx if cfg.backward else None, args.steps) \
        if args.graph else None
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = cfg.T * args.steps / elapsed
    fps = gemm_flops_per_slot(cfg)
    S = cfg.S
    gemm_names = [n for n in fps if n in kern_ms]
    gemm_flops = sum(fps[n] * S for n in gemm_names)
    gemm_ms = sum(kern_ms[n] for n in gemm_names)
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    dom = max(gemm_kernels, key=lambda n: gemm_ms_timed[n])
    ach = fps[dom] * S / (gemm_ms_timed[dom] * 1e-3) / 1e12

    # HBM-bound kernels: algorithmic bytes / time
    T, d, k, E = cfg.T, cfg.d, cfg.k, cfg.E
    es = 2 if cfg.dtype == "bf16" else 4
    hbm_bytes = {
        "route_topk": T * E * 4 + T * k * 8,
        "route_scatter": S * 4 + 2 * S * 4,
        "combine": T * ((k + 1) * d * es + k * 8),
        "dx_combine": T * ((k + 1) * d * es + k * 4),
        "router_grad": T * ((k + 1) * d * es + k * 8 + E * 4),
    }
    hbm = {n: {"bytes": b, "GBs": round(b / (kern_ms[n] * 1e-3) / 1e9, 1)}
           for n, b in hbm_bytes.items() if n in kern_ms}
    traffic = measured_traffic(dom, cfg.name)

    rec = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 4), "min": round(step_ms[0], 4),
                    "mean_of_events": round(sum(step_ms) / len(step_ms), 4),
                    "note": "per-step HIP events on the launch stream inside the timed region"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name} MoE layer", "T": cfg.T, "d": cfg.d, "E": cfg.E,
                   "k": cfg.k, "F": cfg.F, "r": cfg.r, "lora_scale": cfg.s,
                   "step": "route" + ("" if args.no_readback else "(+count readback)") + "+fwd" +
                           ("+bwd" if cfg.backward else "") +
                           ("+router-weight grad" if keep else ""),
                   "parallelism": "single GPU"},
        "grouped_gemm": {"tflops": round(gemm_tflops, 2),
                         "frac_of_peak": round(gemm_tflops / peak, 4),
                         "flops_per_step": gemm_flops, "ms_per_step": round(gemm_ms, 4),
                         "kernels": gemm_names},
        "kernels_ms": {n: round(v, 4) for n, v in kern_ms.items()},
        "kernels_ms_note": f"per-kernel means from {n_breakdown} extra traced steps after the timed region",
        "gemm_ms_timed": {n: round(v, 4) for n, v in gemm_ms_timed.items()},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                     "launch_ms": round(gemm_ms_timed[dom], 4),
                     "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
                     "flops_per_launch": fps[dom] * S},
        "hbm_kernels": hbm,
        "graph_replay": graph,
        "kernel_source_hash": kernel_source_hash(),
        "input_setup_s": round(t_gen, 2),
    }
    if cfg.dtype == "bf16":
        rec["router_projection"] = router_bench(torch, moe, synth, cfg, pb, x, hip, dev)
    if cfg.dtype == "bf16" and args.nf4:
        ctx = {"x": x, "logits": logits, "dout": dout, "w": w, "rt": rt, "ws_r": ws_r, "ws_f": ws_f,
               "ws_b": ws_b if cfg.backward else None, "saved": saved, "keep": keep, "out": out,
               "dx": dx if cfg.backward else None, "grads": grads if cfg.backward else None,
               "dtw": dtw if cfg.backward else None, "dlg": dlg if cfg.backward else None}
        rec["nf4_step"] = nf4_step_bench(torch, moe, synth, cfg, pb, ctx, hip, step_ms[len(step_ms) // 2],
                                         args.steps, args.warmup)
    if cfg.backward and args.offload_reps > 0:
        rec["stack_offload"] = stack_offload_bench(torch, moe, cfg, pb, x, logits, w, dout, keep,
                                                   n=args.offload_layers, reps=args.offload_reps)
    if args.whereloop_steps > 0 and cfg.dtype == "bf16":
        # the library's forward and backward alone (routing excluded), to set
        # against the loop's
        fb = make_trace(["proj_gu", "combine"] + (["proj_dout", "lora_grad"] if cfg.backward else []))
        step(fb)
        torch.cuda.synchronize()
        i = moe.KERNELS.index
        lib_fwd = hip.elapsed_ms(fb.start[i("proj_gu")], fb.stop[i("combine")])
        lib_bwd = (hip.elapsed_ms(fb.start[i("proj_dout")], fb.stop[i("lora_grad")])
                   if cfg.backward else 0.0)
        for n in range(moe.MOE_K_COUNT):
            if fb.start[n]:
                hip.destroy(fb.start[n])
                hip.destroy(fb.stop[n])
        wl_fwd, wl_bwd, wl_out = whereloop_baseline(torch, cfg, x, logits, w, dout,
                                                    args.whereloop_steps)
        diff = (wl_out - out.float()).norm() / wl_out.norm()
        rec["whereloop_baseline"] = {
            "what": "per-expert where() loop in PyTorch on the same GPU and inputs "
                    "(one host sync per expert, gathered copies, hipBLASLt products, "
                    "index_add combine; autograd backward)",
            "steps": args.whereloop_steps, "fwd_ms": round(wl_fwd, 3), "bwd_ms": round(wl_bwd, 3),
            "library_fwd_ms": round(lib_fwd, 4), "library_bwd_ms": round(lib_bwd, 4),
            "fwd_speedup": round(wl_fwd / lib_fwd, 2),
            "bwd_speedup": round(wl_bwd / lib_bwd, 2) if cfg.backward else None,
            "out_rel_l2_vs_library": float(diff)}
    ghz = measured_clock(dom, cfg.name)
    if ghz:
        # the dense bf16 rate at the clock the kernel ran at (the published
        # peak is at 2.4 GHz); the clock is an upper bound, so this fraction
        # is a lower bound
        pk = peak * min(ghz, 2.4) / 2.4
        rec["roofline"]["clock_ghz"] = ghz
        rec["roofline"]["peak_at_clock"] = round(pk, 1)
        rec["roofline"]["frac_at_clock"] = round(ach / pk, 4)
        rec["roofline"]["clock_source"] = (f"profiles/counters_{cfg.name}.md: GRBM_GUI_ACTIVE / 8 "
                                           "XCDs / kernel-trace duration (upper bound)")
    if args.other_workloads:
        rec["other_workloads"] = [other_workload(torch, np, moe, synth, hip, n, args.other_steps, 3)
                                  for n in OTHER_WORKLOADS if n != cfg.name]
    if not args.skip_cpu:
        rec["cpu_baseline"] = cpu_baseline(cfg, min(args.cpu_tokens, cfg.T),
                                           min(args.cpu_tokens_1t, cfg.T))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
