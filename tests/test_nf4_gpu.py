"""4-bit NormalFloat frozen weights on the GPU (moe_nf4_dequant) against the
oracle's fp64 dequantisation, and the whole layer run on dequantised weights
against the oracle layer on the same weights. Dequantised weights are bf16:
each element within one bf16 rounding of the oracle's value."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle import nf4  # noqa: E402
from synth.configs import LayerConfig  # noqa: E402

pytestmark = pytest.mark.gpu


def _dequant_gpu(codes, scales, rows, cols):
    import layer_runner as lr
    import moe_layer_lora_amd as moe
    out = torch.full((rows, cols), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_nf4_dequant(lr.to_dev(codes), lr.to_dev(scales), rows, cols, out)
    torch.cuda.synchronize()
    return out


def _within_one_bf16_rounding(got, want):
    # |got - want| <= half a bf16 ulp of want (plus the fp32 product's rounding)
    tol = np.abs(want) * 2.0 ** -8 * 1.0001 + 1e-30
    return np.all(np.abs(got - want) <= tol)


def test_nf4_codebook_on_gpu():
    import layer_runner as lr
    codes = np.array([[(2 * i) | ((2 * i + 1) << 4) for i in range(8)] * 4], dtype=np.uint8)  # 0..15, x4
    scales = np.ones((1, 1), np.float32)
    got = lr.to_f64(_dequant_gpu(codes, scales, 1, 64))[0]
    want = np.tile(nf4.levels(), 4)
    assert _within_one_bf16_rounding(got, want)
    assert got[7] == 0.0 and got[0] == -1.0 and got[15] == 1.0


@pytest.mark.parametrize("rows,cols", [(1, 64), (300, 192), (7, 2880)])
def test_nf4_dequant_matches_oracle(rows, cols):
    import layer_runner as lr
    q = synth.make_nf4(rows, cols, seed=1)
    got = lr.to_f64(_dequant_gpu(q["codes"], q["scales"], rows, cols))
    want = nf4.dequant(q["codes"], q["scales"], cols)
    assert _within_one_bf16_rounding(got, want)


def test_layer_on_nf4_weights_matches_oracle():
    """x, A, B in bf16, W_g / W_u / W_d in NF4: dequantise on the GPU, run the
    layer; the oracle runs on its own dequantisation rounded to bf16."""
    import layer_runner as lr
    cfg = LayerConfig("nf4_bf16", T=300, d=128, E=6, k=3, F=192, r=16, dtype="bf16", alpha=32.0,
                      router_grad=True)
    inp = synth.make_inputs(cfg, seed=0)
    q = {"w_gate": synth.make_nf4(cfg.E * cfg.F, cfg.d, seed=0, tensor=20),
         "w_up": synth.make_nf4(cfg.E * cfg.F, cfg.d, seed=0, tensor=21),
         "w_down": synth.make_nf4(cfg.E * cfg.d, cfg.F, seed=0, tensor=22)}
    shapes = {"w_gate": (cfg.E, cfg.F, cfg.d), "w_up": (cfg.E, cfg.F, cfg.d),
              "w_down": (cfg.E, cfg.d, cfg.F)}
    L = lr.Layer(cfg, inp, keep_expert_out=True)
    for n, qq in q.items():
        rows, cols = shapes[n][0] * shapes[n][1], shapes[n][2]
        L.w[n].copy_(_dequant_gpu(qq["codes"], qq["scales"], rows, cols).view(*shapes[n]))
    L.step(backward=True, router_grad=True)
    r = L.results(backward=True, router_grad=True)
    # oracle: every tensor in fp64; W from its own dequantisation rounded to bf16
    t = {n: synth.to_f64(inp[n], "bf16") for n in ("x", "a_gate", "b_gate", "a_up", "b_up", "a_down",
                                                   "b_down")}
    for n, qq in q.items():
        t[n] = nf4.round_bf16(nf4.dequant(qq["codes"], qq["scales"], shapes[n][2])).reshape(shapes[n])
    OL = oracle.Layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.r, cfg.s, "f64", t)
    rt = oracle.route(inp["logits"], cfg.k)
    f = oracle.fwd(OL, rt)
    b = oracle.bwd(OL, rt, synth.to_f64(inp["dout"], "bf16"))
    for n in ("topk_idx", "counts", "offsets", "sorted_slot", "slot_row"):
        assert np.array_equal(r[n], rt[n]), n
    assert lr.rel_l2(r["out"], f["out"]) <= 2e-2
    for n in ("dx", "da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down", "d_topk_w",
              "d_logits"):
        assert lr.rel_l2(r[n], b[n]) <= 2e-2, n


@pytest.mark.slow
def test_nf4_full_size_gate_weights_sampled_rows():
    """The Qwen3-30B-A3B-shaped gate weight [128 x 768, 2048] dequantised in
    one call; sampled rows against the oracle."""
    import layer_runner as lr
    rows, cols = 128 * 768, 2048
    q = synth.make_nf4(rows, cols, seed=0, tensor=20)
    got = _dequant_gpu(q["codes"], q["scales"], rows, cols)
    sel = np.array([0, 1, 4095, 50000, rows - 1])
    want = nf4.dequant(q["codes"][sel], q["scales"][sel], cols)
    assert _within_one_bf16_rounding(lr.to_f64(got[torch.from_numpy(sel).cuda()]), want)
    assert not torch.isnan(got.float()).any()


# ------------------------------------------------------------------ NF4 inside the GEMMs

def _nf4_base(cfg, seed=0):
    """NF4 codes and scales of W_g, W_u ([E*F, d]) and W_d ([E*d, F])."""
    q = {"gate": synth.make_nf4(cfg.E * cfg.F, cfg.d, seed=seed, tensor=20),
         "up": synth.make_nf4(cfg.E * cfg.F, cfg.d, seed=seed, tensor=21),
         "down": synth.make_nf4(cfg.E * cfg.d, cfg.F, seed=seed, tensor=22)}
    out = {}
    for n, v in q.items():
        out["codes_" + n] = v["codes"]
        out["scales_" + n] = v["scales"]
    return out


FUSED = {
    # d, F multiples of 64 but not of the 256-wide tiles: ragged column tiles
    # in every GEMM (gate/up 320 = 2.5 x 128 f, down-backward 320 = 1.25 x 256,
    # gate/up-backward and down 192 < 256), ragged row tiles, 3 of 6 experts
    # with a 128-row tail
    "ragged": LayerConfig("nf4_ragged", T=300, d=192, E=6, k=3, F=320, r=16, dtype="bf16", alpha=32.0,
                          router_grad=True),
    "qwen3_30b_a3b": synth.get_config("qwen3_30b_a3b"),
    # GPT-OSS-120B widths (2880 = 11.25 x 256) on 2048 tokens
    "gptoss120b_2048": synth.get_config("gptoss120b").with_(T=2048),
}


def _fused_equals_unfused(cfg, name, keep=True, seed=0):
    import layer_runner as lr
    inp = synth.make_inputs(cfg, seed=seed)
    q = _nf4_base(cfg, seed=seed)
    ref = lr.Layer(cfg, inp, keep_expert_out=keep)
    for n, key, rows, cols in (("w_gate", "gate", cfg.E * cfg.F, cfg.d), ("w_up", "up", cfg.E * cfg.F, cfg.d),
                               ("w_down", "down", cfg.E * cfg.d, cfg.F)):
        ref.w[n].copy_(_dequant_gpu(q["codes_" + key], q["scales_" + key], rows, cols).view(ref.w[n].shape))
    ref.step(backward=True, router_grad=keep)
    want = ref.results(backward=True, router_grad=keep, intermediates=True)
    del ref
    fused = lr.Layer(cfg, inp, keep_expert_out=keep, q4=q)
    assert "w_gate" not in fused.w  # no bf16 base weight exists on the fused path
    fused.step(backward=True, router_grad=keep)
    got = fused.results(backward=True, router_grad=keep, intermediates=True)
    assert set(got) == set(want)
    for n in want:
        assert np.array_equal(got[n], want[n]), f"{name}: {n} differs from the unfused path"


@pytest.mark.parametrize("name", list(FUSED))
def test_fused_nf4_equals_dequantise_then_bf16(name):
    """moe_fwd_nf4 / moe_bwd_nf4 (codes dequantised while each B tile is
    staged into LDS) against moe_nf4_dequant + moe_fwd / moe_bwd on the
    dequantised weights: every output and intermediate bit for bit (the GEMMs
    multiply the same bf16 tiles in the same order)."""
    print(f"[nf4 fused] {name}", flush=True)
    _fused_equals_unfused(FUSED[name], name)


def nf4_sweep_configs(n=10, seed=20261204):
    """Seeded random shapes the 4-bit path accepts: d and F any multiple of
    64 up to 576 / 704 (the per-64 scale groups), r any multiple of 8 up to
    72, 1 to 130 experts, k up to 8, skew on some, every third case without
    the kept expert outputs."""
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        E = int(rs.choice([1, 3, 8, 33, 130]))
        k = int(rs.randint(1, min(E, 8) + 1))
        r = 8 * int(rs.randint(1, 10))
        out.append(LayerConfig(f"nf4_sweep{i:02d}", T=int(rs.randint(1, 601)), d=64 * int(rs.randint(1, 10)),
                               E=E, k=k, F=64 * int(rs.randint(1, 12)), r=r, dtype="bf16", alpha=2.0 * r,
                               router_grad=i % 3 != 2, skew_bias=float(rs.choice([0.0, 0.0, 3.0]))))
    return out


NF4_SWEEP = {c.name: c for c in nf4_sweep_configs()}


@pytest.mark.parametrize("name", list(NF4_SWEEP))
def test_fused_nf4_shape_sweep(name):
    cfg = NF4_SWEEP[name]
    print(f"[nf4 sweep] {cfg}", flush=True)
    _fused_equals_unfused(cfg, name, keep=cfg.router_grad, seed=5)


def test_fused_nf4_layer_matches_oracle():
    """The fused path against the oracle layer on the oracle's own
    dequantisation rounded to bf16 (routing bit-exact, rel-L2 within the
    bf16 bound)."""
    import layer_runner as lr
    cfg = FUSED["ragged"]
    inp = synth.make_inputs(cfg, seed=3)
    q = _nf4_base(cfg, seed=3)
    L = lr.Layer(cfg, inp, keep_expert_out=True, q4=q)
    L.step(backward=True, router_grad=True)
    r = L.results(backward=True, router_grad=True)
    t = {n: synth.to_f64(inp[n], "bf16") for n in ("x", "a_gate", "b_gate", "a_up", "b_up", "a_down",
                                                   "b_down")}
    for n, key, shape in (("w_gate", "gate", (cfg.E, cfg.F, cfg.d)), ("w_up", "up", (cfg.E, cfg.F, cfg.d)),
                          ("w_down", "down", (cfg.E, cfg.d, cfg.F))):
        t[n] = nf4.round_bf16(nf4.dequant(q["codes_" + key], q["scales_" + key], shape[2])).reshape(shape)
    OL = oracle.Layer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.r, cfg.s, "f64", t)
    rt = oracle.route(inp["logits"], cfg.k)
    f = oracle.fwd(OL, rt)
    b = oracle.bwd(OL, rt, synth.to_f64(inp["dout"], "bf16"))
    for n in ("topk_idx", "counts", "offsets", "sorted_slot", "slot_row"):
        assert np.array_equal(r[n], rt[n]), n
    assert lr.rel_l2(r["out"], f["out"]) <= 2e-2
    for n in ("dx", "da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down", "d_topk_w",
              "d_logits"):
        assert lr.rel_l2(r[n], b[n]) <= 2e-2, n
