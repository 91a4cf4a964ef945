"""GPU parity: the HIP layer (through the C ABI) against the CPU oracle.

Routing outputs must match bit for bit; floating-point outputs within the
rel-L2 bound of their storage type (1e-5 fp32, 2e-2 bf16), measured over the
whole tensor, for the small layers (row-loop oracle) and for the four
full-size workloads (the oracle's matrix form, which computes a whole
65536-row layer in seconds).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
from synth.configs import LayerConfig  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
GRADS = ("da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down")


def _runner():
    import layer_runner
    return layer_runner


def check_routing(r, o, tag=""):
    for n in ("topk_idx", "counts", "offsets", "sorted_slot", "slot_row"):
        assert np.array_equal(r[n], o[n]), f"{tag} routing {n} differs"
    # the weights are fp32 softmax values: fp32 rounding only
    lr = _runner()
    assert lr.rel_l2(r["topk_w"], o["topk_w"]) <= 1e-6, tag


def check(name, got, want, tol, tag=""):
    lr = _runner()
    e = lr.rel_l2(got, want)
    assert e <= tol, f"{tag} {name}: rel-L2 {e:.3e} > {tol:.1e}"
    return e


SMALL = {
    "tiny_fp32": synth.get_config("tiny_fp32"),
    "ragged_bf16": LayerConfig("ragged_bf16", T=300, d=136, E=6, k=3, F=200, r=16, dtype="bf16",
                               alpha=32.0, router_grad=True),
    "ragged_f32": LayerConfig("ragged_f32", T=300, d=136, E=6, k=3, F=200, r=16, dtype="f32",
                              alpha=32.0, router_grad=True),
    "rank32_bf16": LayerConfig("rank32_bf16", T=200, d=96, E=5, k=2, F=160, r=32, dtype="bf16",
                               alpha=64.0, router_grad=True),
    "wide_bf16": LayerConfig("wide_bf16", T=520, d=264, E=4, k=2, F=328, r=8, dtype="bf16",
                             alpha=16.0, router_grad=True),
    # 2r = 128: the LoRA gradients of gate/up take two 64-column slices
    "rank64_bf16": LayerConfig("rank64_bf16", T=160, d=128, E=5, k=2, F=96, r=64, dtype="bf16",
                               alpha=128.0, router_grad=True),
    # E = 300: 5 logits per lane in the top-k kernel
    "many_experts_bf16": LayerConfig("many_experts_bf16", T=256, d=64, E=300, k=6, F=64, r=16,
                                     dtype="bf16", alpha=32.0, router_grad=True),
    # F = 1288: six 256-column strips of Pgu shares (four summed as a group,
    # two after), an 11th gate/up column tile with 8 valid f and a ragged
    # 64-deep K tail in the down GEMM
    "wide_ffn_bf16": LayerConfig("wide_ffn_bf16", T=256, d=128, E=4, k=2, F=1288, r=16, dtype="bf16",
                                 alpha=32.0, router_grad=True),
}


def run_small(cfg, inputs, keep=True, router_grad=True):
    lr = _runner()
    L = lr.Layer(cfg, inputs, keep_expert_out=keep)
    L.step(backward=True, router_grad=router_grad)
    return L, L.results(backward=True, router_grad=router_grad, intermediates=True)


def oracle_full(cfg, inputs, rt=None):
    if rt is None:
        rt = oracle.route(inputs["logits"], cfg.k)
    L = oracle.Layer.from_config(cfg, inputs)
    f = oracle.fwd(L, rt, intermediates=True)
    b = oracle.bwd(L, rt, inputs["dout"], intermediates=True)
    return rt, f, b


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_full_parity(name):
    cfg = SMALL[name]
    print(f"[parity] {name}", flush=True)
    inputs = synth.make_inputs(cfg, seed=0)
    _, r = run_small(cfg, inputs)
    rt, f, b = oracle_full(cfg, inputs)
    check_routing(r, rt, name)
    tol = TOL[cfg.dtype]
    check("G", r["G"], f["G"], tol, name)
    check("U", r["U"], f["U"], tol, name)
    check("H", r["H"], f["H"], tol, name)
    check("Zgu", r["Zgu"], np.concatenate([f["Zg"], f["Zu"]], 1), tol, name)
    check("Zd", r["Zd"], f["Zd"], tol, name)
    if cfg.dtype == "bf16":
        # transposed bf16 copies kept for the LoRA-gradient kernels; the down
        # one carries each row's combine weight
        w_row = rt["topk_w"].reshape(-1)[rt["sorted_slot"]][:, None]
        check("ZguT", r["ZguT"], np.concatenate([f["Zg"], f["Zu"]], 1).T, tol, name)
        check("wZdT", r["wZdT"], (w_row * f["Zd"]).T, tol, name)
    check("Y", r["Y"], f["Y"], tol, name)
    check("out", r["out"], f["out"], tol, name)
    check("dx", r["dx"], b["dx"], tol, name)
    for g in GRADS:
        check(g, r[g], b[g], tol, name)
    check("d_topk_w", r["d_topk_w"], b["d_topk_w"], tol, name)
    check("d_logits", r["d_logits"], b["d_logits"], tol, name)
    unselected = b["d_logits"] == 0.0
    assert np.all(r["d_logits"][unselected] == 0.0)


# ------------------------------------------------------------------ edge cases

def edge_case(name):
    base = dict(d=64, F=64, r=8, dtype="bf16", alpha=16.0, router_grad=True)
    if name == "one_token":
        return LayerConfig(name, T=1, E=4, k=2, **base), None
    if name == "k_equals_E":
        return LayerConfig(name, T=40, E=4, k=4, **base), None
    if name == "single_expert":
        return LayerConfig(name, T=70, E=1, k=1, **base), None
    if name == "all_to_one_expert":
        cfg = LayerConfig(name, T=90, E=5, k=1, **base)
        return cfg, lambda l: l.__setitem__((slice(None), 2), 100.0)
    if name == "integer_ties":
        cfg = LayerConfig(name, T=128, E=8, k=3, **base)
        return cfg, lambda l: l.__setitem__(slice(None), np.floor(l * 0.7))
    if name == "multi_chunk_expert":  # > 1024 rows on one expert: chunked LoRA gradients
        cfg = LayerConfig(name, T=2100, E=3, k=1, **base)
        return cfg, lambda l: l.__setitem__((slice(0, 2050), 0), 50.0)
    if name == "many_choices":  # k > 64: two result slots per lane in the top-k kernel
        return LayerConfig(name, T=12, E=96, k=72, **base), None
    if name == "signed_zero_ties":  # -0.0 and +0.0 compare equal: the lower id wins
        cfg = LayerConfig(name, T=64, E=8, k=3, **base)

        def mutate(l):
            rng = np.random.default_rng(5)
            l[:] = np.where(rng.random(l.shape) < 0.5, np.float32(-0.0), np.float32(0.0))
            l[rng.random(l.shape) < 0.15] = 1.0
        return cfg, mutate
    if name == "fp32_ties":
        cfg = LayerConfig(name, T=64, E=6, k=2, d=32, F=40, r=8, dtype="f32", alpha=16.0,
                          router_grad=True)
        return cfg, lambda l: l.__setitem__(slice(None), np.floor(l))
    raise KeyError(name)


EDGE = ["one_token", "k_equals_E", "single_expert", "all_to_one_expert", "integer_ties",
        "signed_zero_ties", "multi_chunk_expert", "many_choices", "fp32_ties"]


@pytest.mark.parametrize("name", EDGE)
def test_edge_cases(name):
    cfg, mutate = edge_case(name)
    print(f"[edge] {name}", flush=True)
    inputs = synth.make_inputs(cfg, seed=1)
    if mutate is not None:
        mutate(inputs["logits"])
        inputs["logits"] = np.ascontiguousarray(inputs["logits"], dtype=np.float32)
    _, r = run_small(cfg, inputs)
    rt, f, b = oracle_full(cfg, inputs)
    check_routing(r, rt, name)
    tol = TOL[cfg.dtype]
    check("out", r["out"], f["out"], tol, name)
    check("dx", r["dx"], b["dx"], tol, name)
    for g in GRADS:
        check(g, r[g], b[g], tol, name)
        empty = rt["counts"] == 0
        assert np.all(r[g][empty] == 0.0), f"{name} {g}: empty experts must get exact zeros"
    check("d_topk_w", r["d_topk_w"], b["d_topk_w"], tol, name)
    check("d_logits", r["d_logits"], b["d_logits"], tol, name)


# ------------------------------------------------------------------ shape sweep

def sweep_configs(n=24, seed=20261203):
    """Seeded random legal shapes beside the hand-picked ones: d, F and r any
    multiple of 8 up to 512 / 640 / 72 (ranks that are not a multiple of 16
    take the register-staged projection and odd LoRA K windows), 1 to 130
    experts with k up to 8, and a Zipf-like skew on some, so that empty
    experts, one-row experts and ragged tiles all occur. Every fourth case
    runs without the kept expert outputs (no router gradient)."""
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        dt = "f32" if i % 6 == 5 else "bf16"
        E = int(rs.choice([1, 2, 3, 7, 16, 33, 64, 130]))
        k = int(rs.randint(1, min(E, 8) + 1))
        r = 8 * int(rs.randint(1, 10))
        out.append(LayerConfig(f"sweep{i:02d}_{dt}", T=int(rs.randint(1, 601)), d=8 * int(rs.randint(1, 65)),
                               E=E, k=k, F=8 * int(rs.randint(1, 81)), r=r, dtype=dt, alpha=2.0 * r,
                               router_grad=i % 4 != 3, skew_bias=float(rs.choice([0.0, 0.0, 2.0, 4.0]))))
    return out


SWEEP = {c.name: c for c in sweep_configs()}


@pytest.mark.parametrize("name", list(SWEEP))
def test_shape_sweep(name):
    cfg = SWEEP[name]
    print(f"[sweep] {cfg}", flush=True)
    inputs = synth.make_inputs(cfg, seed=4)
    _, r = run_small(cfg, inputs, keep=cfg.router_grad, router_grad=cfg.router_grad)
    rt, f, b = oracle_full(cfg, inputs)
    check_routing(r, rt, name)
    tol = TOL[cfg.dtype]
    for n in ("G", "U", "H", "Zd", "out", "dx", "dXp"):
        check(n, r[n], (b if n in ("dx", "dXp") else f)[n], tol, name)
    check("Zgu", r["Zgu"], np.concatenate([f["Zg"], f["Zu"]], 1), tol, name)
    check("dGU", r["dGU"], np.concatenate([b["dG"], b["dU"]], 1), tol, name)
    if cfg.router_grad:
        check("Y", r["Y"], f["Y"], tol, name)
        check("d_topk_w", r["d_topk_w"], b["d_topk_w"], tol, name)
        check("d_logits", r["d_logits"], b["d_logits"], tol, name)
    empty = rt["counts"] == 0
    ne = np.nonzero(~empty)[0]
    for g in GRADS:
        check(g, r[g], b[g], tol, name)
        assert np.all(r[g][empty] == 0.0), f"{name} {g}: empty experts must get exact zeros"
        for e in ne:
            check(f"{g}[{e}]", r[g][e], b[g][e], tol, name)


# Row counts on both sides of every boundary of the LoRA-gradient kernel's
# work items: one chunk holds up to 1024 rows, and an expert takes 4, 3 or 2
# column tiles per item as its chunks hold up to 585, 586-819 or 820-1024
# rows (about 2048 / rows). d = 1800 and 2F = 1680 leave ragged last column
# tiles and groups of unequal size; r = 40 runs the gate/up modes as two
# slices (64 + 16 columns) of the wide-rank kernel.
ITEM_COUNTS = [0, 1, 585, 586, 587, 819, 820, 1024, 1025, 2049, 3000]


@pytest.mark.parametrize("r", [16, 40])
def test_lora_grad_item_boundaries(r):
    from oracle import grouped
    counts = np.array(ITEM_COUNTS)
    T, E = int(counts.sum()), len(counts)
    cfg = LayerConfig(f"items_r{r}", T=T, d=1800, E=E, k=1, F=840, r=r, dtype="bf16", alpha=2.0 * r,
                      router_grad=True)
    print(f"[items] {cfg}", flush=True)
    inputs = synth.make_inputs(cfg, seed=6)
    rs = np.random.RandomState(6)
    assign = rs.permutation(np.repeat(np.arange(E), counts))
    logits = 0.1 * rs.standard_normal((T, E)).astype(np.float32)
    logits[np.arange(T), assign] += 10.0  # top-1 is the assigned expert
    inputs["logits"] = np.ascontiguousarray(logits)
    _, res = run_small(cfg, inputs)
    rt = oracle.route(inputs["logits"], cfg.k)
    assert np.array_equal(rt["counts"], counts)
    check_routing(res, rt, cfg.name)
    o = grouped.layer(oracle.Layer.from_config(cfg, inputs), rt, inputs["dout"], intermediates=True)
    tol = TOL[cfg.dtype]
    for n in ("out", "dx", "d_topk_w", "d_logits"):
        check(n, res[n], o[n], tol, cfg.name)
    for g in GRADS:
        assert np.all(res[g][0] == 0.0), f"{g}: the empty expert must get exact zeros"
        for e in range(1, E):
            check(f"{g}[{e}] ({counts[e]} rows)", res[g][e], o[g][e], tol, cfg.name)


def test_max_experts_skewed():
    """The largest expert count (E = 1024) under a strong skew. 1004 experts
    are empty, eight hold more than one 1024-row chunk (up to every token),
    and the rest hold 136 to 1123 rows, so the LoRA-gradient kernel's
    scheduler tables and the finalize's scans run at their full length with
    every tiles-per-item class. Whole tensors; every non-empty expert's
    gradients are checked on their own, and the empty ones must be exact
    zeros."""
    from oracle import grouped
    cfg = LayerConfig("max_experts", T=2048, d=128, E=1024, k=8, F=64, r=16, dtype="bf16", alpha=32.0,
                      router_grad=True, skew_bias=4.0)
    print(f"[max experts] {cfg}", flush=True)
    inputs = synth.make_inputs(cfg, seed=3)
    _, r = run_small(cfg, inputs)
    rt = oracle.route(inputs["logits"], cfg.k)
    check_routing(r, rt, cfg.name)
    counts = rt["counts"]
    assert (counts == 0).sum() > 900 and (counts > 1024).sum() >= 4
    o = grouped.layer(oracle.Layer.from_config(cfg, inputs), rt, inputs["dout"], intermediates=True)
    tol = TOL[cfg.dtype]
    for n in ("out", "dx", "G", "U", "H", "Y", "dXp", "d_topk_w", "d_logits"):
        check(n, r[n], o[n], tol, cfg.name)
    empty = counts == 0
    for g in GRADS:
        assert np.all(r[g][empty] == 0.0), f"{g}: empty experts must get exact zeros"
        for e in np.nonzero(~empty)[0]:
            check(f"{g}[{e}] ({counts[e]} rows)", r[g][e], o[g][e], tol, cfg.name)


def test_empty_batch():
    lr = _runner()
    cfg = LayerConfig("empty", T=0, d=64, E=4, k=2, F=64, r=8, dtype="bf16", alpha=16.0)
    inputs = synth.make_inputs(cfg.with_(T=1), seed=0)
    for n in ("x", "logits", "dout"):
        inputs[n] = inputs[n][:0]
    L = lr.Layer(cfg, inputs, keep_expert_out=True)
    for g in L.grads.values():
        g.fill_(7.0)
    hc = np.full(cfg.E, -1, np.int32)
    L.route(host_counts=hc)
    hp = torch.full((cfg.E,), -1, dtype=torch.int32, pin_memory=True)
    L.route(host_counts=hp)
    L.fwd()
    L.bwd(router_grad=True)
    torch.cuda.synchronize()
    assert np.all(hc == 0) and torch.all(hp == 0)
    assert L.rt["offsets"].cpu().numpy().tolist() == [0] * (cfg.E + 1)
    for g in L.grads.values():
        assert torch.all(g == 0.0)


def test_host_counts_readback_and_determinism():
    lr = _runner()
    cfg = SMALL["ragged_bf16"]
    inputs = synth.make_inputs(cfg, seed=2)
    L = lr.Layer(cfg, inputs, keep_expert_out=True)
    hc = np.zeros(cfg.E, np.int32)
    L.route(host_counts=hc)
    L.fwd()
    L.bwd(router_grad=True)
    r1 = L.results(router_grad=True, intermediates=True)
    assert np.array_equal(hc, oracle.route(inputs["logits"], cfg.k)["counts"])
    # pinned host memory: written in stream order (by the scan kernel itself
    # when the device reaches it at its host address), valid after a sync
    hp = torch.zeros(cfg.E, dtype=torch.int32, pin_memory=True)
    L.route(host_counts=hp)
    torch.cuda.synchronize()
    assert np.array_equal(hp.numpy(), hc)
    # an interior pointer of a larger pinned buffer: only its E entries change
    big = torch.full((cfg.E + 8,), -1, dtype=torch.int32, pin_memory=True)
    L.route(host_counts=big[4:4 + cfg.E])
    torch.cuda.synchronize()
    assert np.array_equal(big[4:4 + cfg.E].numpy(), hc)
    assert torch.all(big[:4] == -1) and torch.all(big[4 + cfg.E:] == -1)
    L.step(backward=True, router_grad=True)
    r2 = L.results(router_grad=True, intermediates=True)
    for n in r1:
        assert np.array_equal(r1[n], r2[n]), f"{n} not bit-identical across runs"


def test_graph_capture_has_no_hidden_sync():
    """route (no readback) + fwd + bwd captured in one HIP graph, replayed."""
    lr = _runner()
    cfg = SMALL["ragged_bf16"]
    inputs = synth.make_inputs(cfg, seed=3)
    L = lr.Layer(cfg, inputs, keep_expert_out=True)
    L.step(backward=True, router_grad=True)
    ref = L.results(router_grad=True, intermediates=True)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            L.step(backward=True, router_grad=True)
    torch.cuda.current_stream().wait_stream(s)
    for it in range(3):
        L.out.zero_()
        L.dx.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = L.results(router_grad=True, intermediates=True)
        for n in ref:
            assert np.array_equal(got[n], ref[n]), f"replay {it}: {n} differs from eager"


# ------------------------------------------------------------------ largest accepted batches

MAX_SIZE = {
    # the largest GPT-OSS-120B-shaped batch the byte bound admits: dG|dU
    # [S, 2F] bf16 is 2,147,466,240 bytes, 17 KB under 2 GiB
    "gptoss120b_max": synth.get_config("gptoss120b").with_(T=46603),
    # dG|dU exactly 2^31 bytes (S = 262144 rows of 2F = 4096)
    "exact_2gib": LayerConfig("exact_2gib", T=65536, d=1024, E=128, k=4, F=2048, r=16, dtype="bf16",
                              alpha=32.0, router_grad=True),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", list(MAX_SIZE))
def test_largest_accepted_batch(name):
    """The largest batches the library accepts (every tensor at most 2 GiB,
    addressed through 32-bit byte offsets): routing bit-exact over the whole
    batch; out, dx, d_topk_w and d_logits of the tokens whose rows come last
    in the expert order (the largest offsets) and of tokens spread over the
    batch, and the six LoRA gradients of the expert owning the last rows,
    against the oracle's per-token and per-expert entry points."""
    import moe_layer_lora_amd as moe
    lr = _runner()
    cfg = MAX_SIZE[name]
    assert moe.route_workspace(moe.Problem.from_config(cfg)) > 0  # accepted
    print(f"[max] {name}: generating inputs", flush=True)
    inputs = synth.make_inputs(cfg, seed=0)
    L = lr.Layer(cfg, inputs, keep_expert_out=True)
    print(f"[max] {name}: GPU step", flush=True)
    L.step(backward=True, router_grad=True)
    r = L.results(backward=True, router_grad=True)
    del L
    torch.cuda.empty_cache()
    rt = oracle.route(inputs["logits"], cfg.k)
    check_routing(r, rt, name)
    last = rt["sorted_slot"][cfg.S - 16:] // cfg.k
    toks = np.unique(np.concatenate([last, np.linspace(0, cfg.T - 1, 16).astype(np.int64)])).astype(np.int32)
    print(f"[max] {name}: oracle, {len(toks)} tokens", flush=True)
    OL = oracle.Layer.from_config(cfg, inputs)
    f = oracle.fwd_tokens(OL, rt, toks)
    b = oracle.bwd_tokens(OL, rt, inputs["dout"], toks)
    tol = TOL[cfg.dtype]
    check("out", r["out"][toks], f["out"], tol, name)
    check("dx", r["dx"][toks], b["dx"], tol, name)
    check("d_topk_w", r["d_topk_w"][toks], b["d_topk_w"], tol, name)
    check("d_logits", r["d_logits"][toks], b["d_logits"], tol, name)
    e_last = int(np.searchsorted(rt["offsets"], cfg.S - 1, side="right") - 1)
    print(f"[max] {name}: oracle LoRA gradients of expert {e_last}", flush=True)
    g = oracle.lora_grads(OL, rt, inputs["dout"], [e_last])
    for n in GRADS:
        check(f"{n}[{e_last}]", r[n][e_last], g[n][0], tol, name)


# ------------------------------------------------------------------ full-size workloads

@pytest.mark.slow
def test_full_size_step_is_bitwise_deterministic():
    """The Qwen3-30B-A3B-shaped step (65536 routed rows, 2560 tiles per
    grouped GEMM spread over all CUs and XCDs) run twice: every output,
    gradient and stored intermediate bit-identical (no float atomics; every
    cross-block sum has a fixed order)."""
    lr = _runner()
    cfg = synth.get_config("qwen3_30b_a3b")
    print("[determinism] qwen3_30b_a3b", flush=True)
    inputs = synth.make_inputs(cfg, seed=7)
    L = lr.Layer(cfg, inputs, keep_expert_out=True)
    L.step(backward=True, router_grad=True)
    first = L.results(backward=True, router_grad=True, intermediates=True)
    for t in [L.out, L.dx, L.d_topk_w, L.d_logits, *L.grads.values()]:
        t.fill_(7.0)
    L.step(backward=True, router_grad=True)
    second = L.results(backward=True, router_grad=True, intermediates=True)
    assert set(first) == set(second)
    for n in first:
        assert np.array_equal(first[n], second[n]), f"{n} differs between two runs"


FULL = ["gptoss20b", "qwen3_30b_a3b", "qwen3_30b_a3b_skewed", "gptoss120b"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size_whole_tensor(name):
    """The four large workloads at full size, in the launch configuration the
    benchmark times (same buffers, same keep_expert_out), against the
    oracle's matrix form over WHOLE tensors: every output, every expert's
    six LoRA gradients and every intermediate the path stores (G, U, H, the
    fp32 rank-r projections and their transposed bf16 copies, Y, dG|dU,
    dXp). Routing bit-exact over the whole batch."""
    import gc
    from oracle import grouped
    lr = _runner()
    cfg = synth.get_config(name)
    print(f"[full] {name}: generating inputs", flush=True)
    inputs = synth.make_inputs(cfg, seed=0, with_dout=cfg.backward)
    L = lr.Layer(cfg, inputs, keep_expert_out=cfg.router_grad, training=cfg.backward)
    print(f"[full] {name}: GPU step", flush=True)
    L.step(backward=cfg.backward, router_grad=cfg.router_grad)
    r = L.results(backward=cfg.backward, router_grad=cfg.router_grad, intermediates=True)
    del L
    torch.cuda.empty_cache()
    print(f"[full] {name}: oracle", flush=True)
    rt = oracle.route(inputs["logits"], cfg.k)
    check_routing(r, rt, name)
    OL = oracle.Layer.from_config(cfg, inputs)
    o = grouped.layer(OL, rt, inputs["dout"] if cfg.backward else None, intermediates=True)
    del inputs, OL
    tol = TOL[cfg.dtype]
    worst = {}
    worst["out"] = check("out", r["out"], o["out"], tol, name)
    worst["Y"] = check("Y", r["Y"], o["Y"], tol, name)
    if cfg.backward:
        for n in ("G", "U", "H", "Zd"):
            worst[n] = check(n, r[n], o[n], tol, name)
        zgu = np.concatenate([o["Zg"], o["Zu"]], 1)
        worst["Zgu"] = check("Zgu", r["Zgu"], zgu, tol, name)
        worst["ZguT"] = check("ZguT", r["ZguT"], zgu.T, tol, name)
        w_row = rt["topk_w"].reshape(-1)[rt["sorted_slot"]][:, None]
        worst["wZdT"] = check("wZdT", r["wZdT"], (w_row * o["Zd"]).T, tol, name)
        del zgu
        worst["dGU"] = check("dGU", r["dGU"], np.concatenate([o["dG"], o["dU"]], 1), tol, name)
        worst["dXp"] = check("dXp", r["dXp"], o["dXp"], tol, name)
        worst["dx"] = check("dx", r["dx"], o["dx"], tol, name)
        empty = rt["counts"] == 0
        for g in GRADS:
            worst[g] = check(g, r[g], o[g], tol, name)
            assert np.all(r[g][empty] == 0.0), f"{name} {g}: empty experts must get exact zeros"
            # every expert with rows on its own, so a wrong expert cannot hide in the total
            ne = np.nonzero(~empty)[0]
            num = np.linalg.norm((r[g] - o[g])[ne].reshape(len(ne), -1), axis=1)
            den = np.linalg.norm(o[g][ne].reshape(len(ne), -1), axis=1)
            per = float(np.max(num / den))
            assert per <= tol, f"{name} {g}: worst single expert rel-L2 {per:.3e}"
        if cfg.router_grad:
            worst["d_topk_w"] = check("d_topk_w", r["d_topk_w"], o["d_topk_w"], tol, name)
            worst["d_logits"] = check("d_logits", r["d_logits"], o["d_logits"], tol, name)
            assert np.all(r["d_logits"][o["d_logits"] == 0.0] == 0.0)
    print(f"[full] {name}: rel-L2 " + ", ".join(f"{n} {v:.2e}" for n, v in worst.items()),
          flush=True)
    del r, o
    gc.collect()
