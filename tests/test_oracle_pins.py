"""Pins of the CPU oracle to what the mathematics and the stated rules fix.

None of these compares the oracle with itself or with a retyped copy of its
own formula: routing is checked against a different formulation (rank
counting, numpy's stable argsort), Split-LoRA against the materialised
W + s*B*A form evaluated densely over all experts with numpy, the backward
against central finite differences, and the rest against closed forms and
invariants. CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import grouped as oracle_grouped

# The two forms of the oracle's expert layer (row-at-a-time C loops, and one
# matrix product per expert and step): every layer pin below runs on both.
IMPLS = {"loops": oracle, "grouped": oracle_grouped}
impl_param = pytest.mark.parametrize("impl", list(IMPLS))

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def rand_tensors(T, d, E, F, r, seed, sigma=0.5):
    rng = np.random.default_rng(seed)
    sh = {"x": (T, d), "w_gate": (E, F, d), "w_up": (E, F, d), "w_down": (E, d, F),
          "a_gate": (E, r, d), "b_gate": (E, F, r), "a_up": (E, r, d), "b_up": (E, F, r),
          "a_down": (E, r, F), "b_down": (E, d, r)}
    t = {n: rng.normal(0.0, sigma, s) for n, s in sh.items()}
    t["x"] = rng.normal(0.0, 1.0, sh["x"])
    logits = rng.normal(0.0, 1.0, (T, E)).astype(np.float32)
    dout = rng.normal(0.0, 1.0, (T, d))
    return t, logits, dout


def make(T, d, E, k, F, r, s, seed, sigma=0.5):
    t, logits, dout = rand_tensors(T, d, E, F, r, seed, sigma)
    L = oracle.Layer(T, d, E, k, F, r, s, "f64", t)
    return L, t, logits, dout


def silu(z):
    return z / (1.0 + np.exp(-z))


def dense_materialised_out(t, logits_rt, s):
    """out[t] = sum_e gate[t,e] * expert_e(x_t) with W_eff = W + s B A formed
    explicitly, every expert evaluated on every token (gate 0 if unselected)."""
    X = t["x"]
    T = X.shape[0]
    E = t["w_gate"].shape[0]
    gate = np.zeros((T, E))
    k = logits_rt["topk_idx"].shape[1]
    for tt in range(T):
        for j in range(k):
            gate[tt, logits_rt["topk_idx"][tt, j]] = logits_rt["topk_w"][tt, j]
    out = np.zeros((T, t["w_down"].shape[1]))
    for e in range(E):
        wg = t["w_gate"][e] + s * t["b_gate"][e] @ t["a_gate"][e]
        wu = t["w_up"][e] + s * t["b_up"][e] @ t["a_up"][e]
        wd = t["w_down"][e] + s * t["b_down"][e] @ t["a_down"][e]
        h = silu(X @ wg.T) * (X @ wu.T)
        out += gate[:, e:e + 1] * (h @ wd.T)
    return out


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- routing

def brute_topk(l, k):
    """rank_e = #{e': l_e' > l_e or (l_e' == l_e and e' < e)}; chosen iff rank < k."""
    E = len(l)
    idx = [None] * k
    for e in range(E):
        rank = sum(1 for e2 in range(E) if l[e2] > l[e] or (l[e2] == l[e] and e2 < e))
        if rank < k:
            idx[rank] = e
    return idx


def test_route_matches_rank_counting_exhaustive_ties():
    # every logit row over {0,1,2}^4: all tie patterns, every k
    rows = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=4)), dtype=np.float32)
    for k in range(1, 5):
        rt = oracle.route(rows, k)
        for t in range(rows.shape[0]):
            assert list(rt["topk_idx"][t]) == brute_topk(list(rows[t]), k)


def test_route_matches_rank_counting_random():
    rng = np.random.default_rng(1)
    for E, k in [(8, 2), (16, 5), (33, 33), (64, 8)]:
        # coarse values force many ties
        l = rng.integers(-3, 4, size=(50, E)).astype(np.float32) * 0.5
        rt = oracle.route(l, k)
        for t in range(l.shape[0]):
            assert list(rt["topk_idx"][t]) == brute_topk(list(l[t]), k)


def test_route_signed_zero_ties_go_to_lower_id():
    l = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    rt = oracle.route(l, 1)
    assert rt["topk_idx"][:, 0].tolist() == [0, 0]
    assert rt["topk_w"][:, 0].tolist() == [1.0, 1.0]


def test_route_golden_cases():
    """Hand-worked cases of the stated rule (tests/golden/routing_cases.json)."""
    with open(os.path.join(GOLDEN, "routing_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        l = np.array([c["logits"]], dtype=np.float32)
        rt = oracle.route(l, c["k"])
        assert rt["topk_idx"][0].tolist() == c["topk_idx"], c["name"]
        w = rt["topk_w"][0]
        want = [eval(expr, {"exp": math.exp}) for expr in c["topk_w"]]  # closed forms
        assert np.allclose(w, want, rtol=1e-14, atol=0), c["name"]


def test_softmax_weights_closed_forms():
    rng = np.random.default_rng(2)
    l = rng.normal(size=(200, 16)).astype(np.float32)
    # k = 1: exactly one
    assert np.all(oracle.route(l, 1)["topk_w"] == 1.0)
    # k = 2: w0 = 1 / (1 + exp(l1 - l0))
    rt = oracle.route(l, 2)
    for t in range(l.shape[0]):
        l0 = float(l[t, rt["topk_idx"][t, 0]])
        l1 = float(l[t, rt["topk_idx"][t, 1]])
        assert rt["topk_w"][t, 0] == pytest.approx(1.0 / (1.0 + math.exp(l1 - l0)), rel=1e-14)
    # any k: sums to one, non-increasing in j
    for k in (3, 8, 16):
        w = oracle.route(l, k)["topk_w"]
        assert np.allclose(w.sum(1), 1.0, atol=1e-14)
        assert np.all(np.diff(w, axis=1) <= 0)


def test_grouping_equals_stable_sort_bincount_offsets():
    for name in ("tiny_fp32", "qwen3_30b_a3b_skewed"):
        cfg = synth.get_config(name)
        T = min(cfg.T, 2048)
        logits = synth.make_inputs(cfg.with_(d=8, F=8, r=8), tokens=T, with_dout=False)["logits"]
        rt = oracle.route(logits, cfg.k)
        flat = rt["topk_idx"].reshape(-1)
        order = np.argsort(flat, kind="stable")
        assert np.array_equal(rt["sorted_slot"], order.astype(np.int32))
        counts = np.bincount(flat, minlength=cfg.E)
        assert np.array_equal(rt["counts"], counts)
        assert np.array_equal(rt["offsets"], np.concatenate([[0], np.cumsum(counts)]))


def test_grouping_invariants():
    cfg = synth.get_config("qwen3_30b_a3b_skewed")
    logits = synth.make_inputs(cfg.with_(d=8, F=8, r=8), with_dout=False)["logits"]
    rt = oracle.route(logits, cfg.k)
    S = cfg.T * cfg.k
    assert rt["counts"].sum() == S and rt["offsets"][-1] == S
    assert np.all(np.diff(rt["offsets"]) >= 0)
    ss, sr = rt["sorted_slot"], rt["slot_row"]
    assert np.array_equal(np.sort(ss), np.arange(S))            # bijection
    assert np.array_equal(sr[ss], np.arange(S))                  # inverse
    tok = ss // cfg.k
    assert np.array_equal(np.bincount(tok, minlength=cfg.T), np.full(cfg.T, cfg.k))
    for e in range(cfg.E):
        g = tok[rt["offsets"][e]:rt["offsets"][e + 1]]
        assert np.all(np.diff(g) > 0)                            # strictly ascending tokens
        assert np.all(rt["topk_idx"].reshape(-1)[ss[rt["offsets"][e]:rt["offsets"][e + 1]]] == e)
    # the skewed workload does leave experts empty and one expert hot
    assert (rt["counts"] == 0).sum() > 0
    assert rt["counts"].max() > 0.10 * S


# ---------------------------------------------------------------- forward

@impl_param
@pytest.mark.parametrize("shape", [(7, 8, 4, 2, 12, 3), (5, 16, 1, 1, 8, 4), (9, 8, 6, 6, 8, 2)])
def test_split_lora_equals_materialised_dense(shape, impl):
    T, d, E, k, F, r = shape
    L, t, logits, _ = make(T, d, E, k, F, r, s=1.7, seed=3)
    rt = oracle.route(logits, k)
    out = IMPLS[impl].fwd(L, rt)["out"]
    ref = dense_materialised_out(t, rt, 1.7)
    assert rel_l2(out, ref) < 1e-13


@impl_param
def test_swiglu_closed_form_tiny(impl):
    """T=d... one token, one expert: g = x0 + s*bg*(ag . x), u = 2 x1, h = silu(g) u,
    z_d = a_d h, y = (h, 3h + s*z_d)."""
    s = 2.0
    t = {"x": np.array([[1.0, 0.5]]),
         "w_gate": np.array([[[1.0, 0.0]]]), "w_up": np.array([[[0.0, 2.0]]]),
         "w_down": np.array([[[1.0], [3.0]]]),
         "a_gate": np.array([[[1.0, -1.0]]]), "b_gate": np.array([[[0.5]]]),
         "a_up": np.zeros((1, 1, 2)), "b_up": np.zeros((1, 1, 1)),
         "a_down": np.array([[[2.0]]]), "b_down": np.array([[[0.0], [1.0]]])}
    L = oracle.Layer(1, 2, 1, 1, 1, 1, s, "f64", t)
    rt = oracle.route(np.zeros((1, 1), np.float32), 1)
    f = IMPLS[impl].fwd(L, rt, intermediates=True)
    g = 1.0 + s * 0.5 * 0.5                 # 1.5
    u = 1.0
    h = g / (1.0 + math.exp(-g)) * u
    assert f["G"][0, 0] == pytest.approx(g, rel=1e-15)
    assert f["U"][0, 0] == pytest.approx(u, rel=1e-15)
    assert f["H"][0, 0] == pytest.approx(h, rel=1e-15)
    assert f["Zd"][0, 0] == pytest.approx(2 * h, rel=1e-15)
    assert f["out"][0].tolist() == pytest.approx([h, 3 * h + s * 2 * h], rel=1e-15)
    # gate and up are not interchangeable: silu applies to the gate only
    assert f["H"][0, 0] != pytest.approx(u / (1 + math.exp(-u)) * g)


@impl_param
def test_identical_experts_make_routing_irrelevant(impl):
    T, d, E, k, F, r = 11, 8, 5, 3, 12, 2
    t, logits, _ = rand_tensors(T, d, E, F, r, seed=4)
    for n in t:
        if n != "x":
            t[n] = np.repeat(t[n][:1], E, axis=0)
    L = oracle.Layer(T, d, E, k, F, r, 0.9, "f64", t)
    out = IMPLS[impl].fwd(L, oracle.route(logits, k))["out"]
    wg = t["w_gate"][0] + 0.9 * t["b_gate"][0] @ t["a_gate"][0]
    wu = t["w_up"][0] + 0.9 * t["b_up"][0] @ t["a_up"][0]
    wd = t["w_down"][0] + 0.9 * t["b_down"][0] @ t["a_down"][0]
    single = (silu(t["x"] @ wg.T) * (t["x"] @ wu.T)) @ wd.T
    assert rel_l2(out, single) < 1e-13


@impl_param
def test_token_permutation_equivariance_bit_exact(impl):
    """Bit-exact for the row loops; the matrix form's library products may
    round a row differently at another position inside an expert's block,
    so there the bound is a few ulps."""
    T, d, E, k, F, r = 13, 8, 6, 2, 8, 2
    L, t, logits, _ = make(T, d, E, k, F, r, s=2.0, seed=5)
    out = IMPLS[impl].fwd(L, oracle.route(logits, k))["out"]
    perm = np.random.default_rng(0).permutation(T)
    t2 = dict(t)
    t2["x"] = t["x"][perm]
    L2 = oracle.Layer(T, d, E, k, F, r, 2.0, "f64", t2)
    out2 = IMPLS[impl].fwd(L2, oracle.route(logits[perm], k))["out"]
    if impl == "loops":
        assert np.array_equal(out2, out[perm])
    else:
        assert rel_l2(out2, out[perm]) < 1e-14


@impl_param
def test_lora_b_zero_gives_base_only_bit_exact(impl):
    T, d, E, k, F, r = 9, 8, 4, 2, 8, 3
    L, t, logits, dout = make(T, d, E, k, F, r, s=2.0, seed=6)
    rt = oracle.route(logits, k)
    t0 = dict(t)
    for n in ("b_gate", "b_up", "b_down"):
        t0[n] = np.zeros_like(t[n])
    Lb0 = oracle.Layer(T, d, E, k, F, r, 2.0, "f64", t0)
    Ls0 = oracle.Layer(T, d, E, k, F, r, 0.0, "f64", t)
    O = IMPLS[impl]
    assert np.array_equal(O.fwd(Lb0, rt)["out"], O.fwd(Ls0, rt)["out"])
    gb0 = O.bwd(Lb0, rt, dout)
    gs0 = O.bwd(Ls0, rt, dout)
    assert np.array_equal(gb0["dx"], gs0["dx"])
    for n in ("da_gate", "da_up", "da_down"):
        assert np.all(gb0[n] == 0.0)
    for n in ("da_gate", "da_up", "da_down", "db_gate", "db_up", "db_down"):
        assert np.all(gs0[n] == 0.0)


@impl_param
def test_storage_formats_agree(impl):
    """bf16 bits, their exact float32 widening and float64 give identical results."""
    cfg = synth.get_config("tiny_fp32").with_(dtype="bf16", T=32)
    inp = synth.make_inputs(cfg)
    rt = oracle.route(inp["logits"], cfg.k)
    names = oracle.Layer.NAMES
    Lb = oracle.Layer.from_config(cfg, inp)
    Lf = oracle.Layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.r, cfg.s, "f32",
                      {n: synth.bf16_to_f32(inp[n]) for n in names})
    Ld = oracle.Layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.r, cfg.s, "f64",
                      {n: synth.bf16_to_f32(inp[n]).astype(np.float64) for n in names})
    O = IMPLS[impl]
    ob, of_, od = (O.fwd(L, rt)["out"] for L in (Lb, Lf, Ld))
    assert np.array_equal(ob, of_) and np.array_equal(ob, od)
    gb = O.bwd(Lb, rt, inp["dout"])
    gd = O.bwd(Ld, rt, synth.bf16_to_f32(inp["dout"]).astype(np.float64))
    for n in gb:
        assert np.array_equal(gb[n], gd[n]), n


# ---------------------------------------------------------------- backward

def _loss(L, rt, dout):
    # the loss is evaluated by the row-loop forward for both forms: its
    # derivatives are then what each form's backward must reproduce
    return float(np.sum(dout * oracle.fwd(L, rt)["out"]))


FD_SHAPE = (6, 8, 4, 2, 12, 3)


@pytest.fixture(scope="module", params=list(IMPLS))
def fd_case(request):
    T, d, E, k, F, r = FD_SHAPE
    L, t, logits, dout = make(T, d, E, k, F, r, s=1.3, seed=7)
    rt = oracle.route(logits, k)
    g = IMPLS[request.param].bwd(L, rt, dout)
    return T, d, E, k, F, r, t, logits, dout, rt, g


@pytest.mark.parametrize("name,gname", [
    ("x", "dx"), ("a_gate", "da_gate"), ("b_gate", "db_gate"), ("a_up", "da_up"),
    ("b_up", "db_up"), ("a_down", "da_down"), ("b_down", "db_down")])
def test_gradients_match_central_differences(fd_case, name, gname):
    T, d, E, k, F, r, t, logits, dout, rt, g = fd_case
    h = 1e-6
    base = t[name]
    fd = np.empty(base.size)
    for i in range(base.size):
        for sign in (+1, -1):
            tt = dict(t)
            p = base.copy().reshape(-1)
            p[i] += sign * h
            tt[name] = p.reshape(base.shape)
            val = _loss(oracle.Layer(T, d, E, k, F, r, 1.3, "f64", tt), rt, dout)
            fd[i] = val if sign > 0 else (fd[i] - val) / (2 * h)
    ana = g[gname].reshape(-1)
    assert np.max(np.abs(fd - ana)) <= 1e-7 * max(1.0, np.max(np.abs(ana)))


def test_router_weight_gradient_matches_central_differences(fd_case):
    T, d, E, k, F, r, t, logits, dout, rt, g = fd_case
    L = oracle.Layer(T, d, E, k, F, r, 1.3, "f64", t)
    h = 1e-6
    for tt in range(T):
        for j in range(k):
            vals = []
            for sign in (+1, -1):
                rt2 = dict(rt)
                w = rt["topk_w"].copy()
                w[tt, j] += sign * h
                rt2["topk_w"] = w
                vals.append(_loss(L, rt2, dout))
            assert (vals[0] - vals[1]) / (2 * h) == pytest.approx(g["d_topk_w"][tt, j],
                                                                  rel=1e-6, abs=1e-9)


def test_logit_gradient_matches_central_differences(fd_case):
    T, d, E, k, F, r, t, logits, dout, rt, g = fd_case
    L = oracle.Layer(T, d, E, k, F, r, 1.3, "f64", t)
    h = 1e-3  # logits are float32: a step float32 can carry exactly
    for tt in range(T):
        for e in range(E):
            vals = []
            for sign in (+1, -1):
                l2 = logits.copy()
                l2[tt, e] = np.float32(float(logits[tt, e]) + sign * h)
                rt2 = oracle.route(l2, k)
                assert np.array_equal(rt2["topk_idx"], rt["topk_idx"])  # selection unchanged
                vals.append((_loss(L, rt2, dout), float(l2[tt, e])))
            fd = (vals[0][0] - vals[1][0]) / (vals[0][1] - vals[1][1])
            assert fd == pytest.approx(g["d_logits"][tt, e], rel=1e-4, abs=1e-8)
    # unselected experts get exactly zero; each row sums to zero
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, rt["topk_idx"], True, axis=1)
    assert np.all(g["d_logits"][~sel] == 0.0)
    assert np.allclose(g["d_logits"].sum(1), 0.0, atol=1e-14)


@impl_param
def test_empty_expert_gradients_are_exact_zeros(impl):
    T, d, E, k, F, r = 8, 8, 6, 2, 8, 2
    L, t, logits, dout = make(T, d, E, k, F, r, s=2.0, seed=8)
    logits[:, 4:] = -50.0  # experts 4 and 5 never chosen
    rt = oracle.route(logits, k)
    assert rt["counts"][4] == 0 and rt["counts"][5] == 0
    g = IMPLS[impl].bwd(L, rt, dout)
    for n in ("da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down"):
        assert np.all(g[n][4:] == 0.0)


def test_sampled_entry_points_agree_with_full_layer():
    cfg = synth.get_config("tiny_fp32")
    inp = synth.make_inputs(cfg)
    rt = oracle.route(inp["logits"], cfg.k)
    L = oracle.Layer.from_config(cfg, inp)
    f = oracle.fwd(L, rt)
    b = oracle.bwd(L, rt, inp["dout"])
    toks = [0, 17, 255]
    ft = oracle.fwd_tokens(L, rt, toks)
    bt = oracle.bwd_tokens(L, rt, inp["dout"], toks)
    assert np.array_equal(ft["out"], f["out"][toks])
    assert np.array_equal(bt["dx"], b["dx"][toks])
    assert np.array_equal(bt["d_logits"], b["d_logits"][toks])
    assert np.array_equal(bt["d_topk_w"], b["d_topk_w"][toks])
    ex = [2, 7]
    lg = oracle.lora_grads(L, rt, inp["dout"], ex)
    for n in lg:
        assert np.allclose(lg[n], b[n][ex], rtol=1e-12, atol=1e-18)


# ---------------------------------------------------------------- router projection

def _route_f64(logits64, k):
    """Routing of fp64 logits: selection, order and grouping from their fp32
    rounding (no near-ties in these cases), weights from the fp64 values."""
    rt = oracle.route(logits64.astype(np.float32), k)
    sel = np.take_along_axis(logits64, rt["topk_idx"].astype(np.int64), axis=1)
    w = np.exp(sel - sel[:, :1])
    rt["topk_w"] = w / w.sum(1, keepdims=True)
    return rt


def test_router_identity_gate_passes_x_through():
    rng = np.random.default_rng(3)
    x = rng.normal(0.0, 1.0, (5, 8))
    assert np.array_equal(oracle.router_fwd(x, np.eye(8)), x)
    # one-hot rows pick columns: logits[:, e] = x[:, perm[e]]
    perm = rng.permutation(8)
    assert np.array_equal(oracle.router_fwd(x, np.eye(8)[perm]), x[:, perm])


def test_router_storage_formats_agree():
    rng = np.random.default_rng(4)
    xb = synth.f32_to_bf16(rng.normal(0.0, 1.0, (6, 16)).astype(np.float32))
    wb = synth.f32_to_bf16(rng.normal(0.0, 1.0, (8, 16)).astype(np.float32))
    x64, w64 = synth.to_f64(xb, "bf16"), synth.to_f64(wb, "bf16")
    assert np.array_equal(oracle.router_fwd(xb, wb), oracle.router_fwd(x64, w64))
    dl = rng.normal(0.0, 1.0, (6, 8))
    a, b = oracle.router_bwd(xb, wb, dl), oracle.router_bwd(x64, w64, dl)
    assert np.array_equal(a["dx"], b["dx"]) and np.array_equal(a["dw_r"], b["dw_r"])


@pytest.fixture(scope="module")
def router_fd_case():
    T, d, E, k, F, r = FD_SHAPE
    L, t, _, dout = make(T, d, E, k, F, r, s=1.3, seed=11)
    rng = np.random.default_rng(12)
    w_r = rng.normal(0.0, 0.7, (E, d))
    rt = _route_f64(oracle.router_fwd(t["x"], w_r), k)
    g = oracle.bwd(L, rt, dout)
    rg = oracle.router_bwd(t["x"], w_r, g["d_logits"])
    return T, d, E, k, F, r, t, w_r, dout, rt, g, rg


def _chain_loss(shape, t, w_r, dout, idx):
    """Loss of the layer with its router: logits = x W_r^T feed the routing."""
    T, d, E, k, F, r = shape
    rt = _route_f64(oracle.router_fwd(t["x"], w_r), k)
    assert np.array_equal(rt["topk_idx"], idx)  # a small step keeps the selection
    return _loss(oracle.Layer(T, d, E, k, F, r, 1.3, "f64", t), rt, dout)


def test_router_chain_dx_matches_central_differences(router_fd_case):
    """dX of the whole layer = the expert path's dX + the router's share."""
    T, d, E, k, F, r, t, w_r, dout, rt, g, rg = router_fd_case
    h = 1e-6
    fd = np.empty(T * d)
    for i in range(T * d):
        vals = []
        for sign in (+1, -1):
            tt = dict(t)
            p = t["x"].copy().reshape(-1)
            p[i] += sign * h
            tt["x"] = p.reshape(T, d)
            vals.append(_chain_loss(FD_SHAPE, tt, w_r, dout, rt["topk_idx"]))
        fd[i] = (vals[0] - vals[1]) / (2 * h)
    ana = (g["dx"] + rg["dx"]).reshape(-1)
    assert np.max(np.abs(fd - ana)) <= 1e-7 * max(1.0, np.max(np.abs(ana)))
    # the router's share is not negligible here, so a dropped term would fail
    assert np.max(np.abs(rg["dx"])) > 1e-3 * np.max(np.abs(ana))


def test_router_weight_gradient_chain_matches_central_differences(router_fd_case):
    T, d, E, k, F, r, t, w_r, dout, rt, g, rg = router_fd_case
    h = 1e-6
    fd = np.empty(E * d)
    for i in range(E * d):
        vals = []
        for sign in (+1, -1):
            p = w_r.copy().reshape(-1)
            p[i] += sign * h
            vals.append(_chain_loss(FD_SHAPE, t, p.reshape(E, d), dout, rt["topk_idx"]))
        fd[i] = (vals[0] - vals[1]) / (2 * h)
    ana = rg["dw_r"].reshape(-1)
    assert np.max(np.abs(fd - ana)) <= 1e-7 * max(1.0, np.max(np.abs(ana)))
    # logit gradients sum to zero per token, so the columns of dW_r sum to zero
    assert np.allclose(rg["dw_r"].sum(0), 0.0, atol=1e-12)


# ---------------------------------------------------------------- 4-bit NormalFloat weights

def test_nf4_levels_are_normal_quantiles():
    import math
    from oracle import nf4
    lv = nf4.levels()
    assert lv.shape == (16,) and np.all(np.diff(lv) > 0)
    assert lv[0] == -1.0 and lv[7] == 0.0 and lv[15] == 1.0
    assert np.sum(lv < 0) == 7 and np.sum(lv > 0) == 8
    # inverse relation through the error function (not the quantile routine
    # that built them): Phi(level * Q(p)) hits the stated probabilities
    p = nf4.P_TOP
    qmax = float(np.sqrt(2.0)) * _erfinv_newton(2 * p - 1)  # Q(p)

    def phi(x):
        return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))

    for j in range(1, 9):
        assert phi(lv[7 + j] * qmax) == pytest.approx(0.5 + j / 8 * (p - 0.5), abs=1e-12)
    for j in range(1, 8):
        assert phi(-lv[7 - j] * qmax) == pytest.approx(0.5 + j / 7 * (p - 0.5), abs=1e-12)


def test_nf4_levels_match_the_published_table():
    """The 16 levels against the values the QLoRA paper's appendix prints
    (float32 there, so agreement is to float32 rounding)."""
    from oracle import nf4
    with open(os.path.join(GOLDEN, "nf4_levels_qlora.json")) as f:
        pub = np.array(json.load(f)["levels"], dtype=np.float64)
    lv = nf4.levels()
    assert np.max(np.abs(lv - pub)) <= 2.5e-7
    # the float32 values are the float32 roundings of the fp64 levels, up to
    # the last bit of the published rounding
    assert np.max(np.abs(lv.astype(np.float32).astype(np.float64) - pub)) <= 1.2e-7


def _erfinv_newton(y):
    import math
    x = 0.0
    for _ in range(100):
        step = (math.erf(x) - y) / (2.0 / math.sqrt(math.pi) * math.exp(-x * x))
        x -= step
        if abs(step) < 1e-16:
            break
    return x


def test_nf4_nibble_order_and_block_scales():
    from oracle import nf4
    codes = np.zeros((1, 64), np.uint8)
    codes[0, 0] = 0x21        # element 0 -> code 1, element 1 -> code 2
    codes[0, 32] = 0xF0       # element 64 -> code 0, element 65 -> code 15
    q = nf4.unpack_codes(codes, 128)
    assert q[0, 0] == 1 and q[0, 1] == 2 and q[0, 64] == 0 and q[0, 65] == 15 and q[0, 2] == 0
    w = nf4.dequant(codes, np.array([[2.0, 0.5]], np.float32), 128)
    lv = nf4.levels()
    assert w[0, 0] == 2.0 * lv[1] and w[0, 1] == 2.0 * lv[2] and w[0, 2] == 2.0 * lv[0]
    assert w[0, 64] == 0.5 * lv[0] and w[0, 65] == 0.5 * lv[15] and w[0, 127] == 0.5 * lv[0]


def test_bf16_rounding_ties_to_even():
    from oracle import nf4
    one = 1.0
    assert nf4.round_bf16(np.array([one]))[0] == 1.0
    assert nf4.round_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0            # tie -> even
    assert nf4.round_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6  # tie -> even (up)
    assert nf4.round_bf16(np.array([one + 3 * 2.0 ** -9]))[0] == one + 2.0 ** -7
    assert nf4.round_bf16(np.array([-0.0]))[0] == 0.0


@pytest.mark.parametrize("cfg_name,tokens", [("tiny_fp32", None), ("qwen3_30b_a3b", 96)])
def test_the_two_forms_agree_on_the_workloads(cfg_name, tokens):
    """Both forms on stored workload inputs (fp32; bf16 on the first tokens of
    the Qwen3-30B-A3B shapes, 128 experts, many of them with few rows), every
    output and intermediate: they differ only in the summation order of fp64
    dot products."""
    cfg = synth.get_config(cfg_name)
    inp = synth.make_inputs(cfg, seed=0, tokens=tokens)
    L = oracle.Layer.from_config(cfg, inp, tokens=tokens)
    rt = oracle.route(inp["logits"], cfg.k)
    a = {**oracle.fwd(L, rt, intermediates=True), **oracle.bwd(L, rt, inp["dout"], intermediates=True)}
    b = oracle_grouped.layer(L, rt, inp["dout"], intermediates=True)
    for n in a:
        assert rel_l2(b[n], a[n]) < 1e-12, n
