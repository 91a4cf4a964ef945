"""The C-ABI library on the host: it loads, exports every symbol include/moe.h
declares, sizes its buffers as documented and rejects bad arguments before
enqueuing anything. No kernel is launched by these tests: every call that is
not a size query fails a host-side check (and, as a second guard, passes no
workspace where one is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import moe_layer_lora_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS)
    for n in names:
        assert hasattr(moe.lib(), n), n
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)$", out, flags=re.M))
    assert set(names) <= exported  # unmangled (extern "C")


def test_trace_indices_match_header():
    src = open(HEADER).read()
    body = re.search(r"enum \{(.*?)\};", src, flags=re.S).group(1)
    ids = re.findall(r"MOE_K_(\w+)", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert ids[-1] == "COUNT"
    assert [i.lower() for i in ids[:-1]] == moe.KERNELS


def test_status_strings():
    assert moe.moe_status_str(moe.MOE_OK) == "ok"
    assert moe.moe_status_str(moe.MOE_E_WORKSPACE) == "workspace too small"
    assert moe.moe_status_str(99) == "unknown status"


def pb(**kw):
    base = dict(T=512, d=256, E=16, k=4, F=128, r=16, lora_scale=2.0, dtype=moe.MOE_BF16)
    base.update(kw)
    return moe.Problem(**base)


def al(x):
    return (x + 255) // 256 * 256


def test_saved_and_workspace_sizes():
    p = pb()
    S, es = p.T * p.k, 2
    ldT = (S + 7) // 8 * 8
    want = (3 * al(S * p.F * es) + al(S * 2 * p.r * 4) + al(S * p.r * 4)
            + al(2 * p.r * ldT * 2) + al(p.r * ldT * 2))  # bf16: transposed copies for the LoRA gradients
    assert moe.saved_bytes(p, False) == want
    assert moe.saved_bytes(p, True) == want + al(S * p.d * es)
    # an offload moves everything but H, which is last
    assert moe.saved_host_bytes(p, False) == want - al(S * p.F * es)
    assert moe.saved_host_bytes(p, True) == want + al(S * p.d * es) - al(S * p.F * es)
    assert moe.saved_host_bytes(pb(k=0), True) == 0
    tiles = al((1 + (S + 255) // 256 + p.E) * 16)  # bf16: row-tile table of the grouped GEMMs
    assert moe.fwd_workspace(p, True, True) == tiles
    assert moe.fwd_workspace(p, True, False) == al(S * p.d * es) + tiles
    assert moe.fwd_workspace(p, False, False) == (al(S * p.F * es) + al(S * 2 * p.r * 4)
                                                  + al(S * p.r * 4) + al(S * p.d * es) + tiles)
    assert moe.route_workspace(p) > 0 and moe.bwd_workspace(p) > 0
    p32 = pb(dtype=moe.MOE_F32)
    assert moe.fwd_workspace(p32, True, True) == 0
    assert moe.saved_bytes(p32, False) == 3 * al(S * p.F * 4) + al(S * 2 * p.r * 4) + al(S * p.r * 4)
    assert moe.saved_host_bytes(p32, False) == 2 * al(S * p.F * 4) + al(S * 2 * p.r * 4) + al(S * p.r * 4)


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), moe.MOE_E_ARG), (dict(k=17), moe.MOE_E_ARG), (dict(T=-1), moe.MOE_E_ARG),
    (dict(dtype=7), moe.MOE_E_ARG), (dict(lora_scale=float("nan")), moe.MOE_E_ARG),
    (dict(d=100), moe.MOE_E_UNSUPPORTED), (dict(F=36), moe.MOE_E_UNSUPPORTED),
    (dict(r=12), moe.MOE_E_UNSUPPORTED), (dict(E=1025, k=2), moe.MOE_E_UNSUPPORTED),
    (dict(T=1 << 20, d=4096, k=8), moe.MOE_E_UNSUPPORTED),
    # GPT-OSS-120B shapes at 49152 tokens: the [S, 2F] bf16 dG|dU tensor is 2.26 GB
    (dict(T=49152, d=2880, E=128, k=4, F=2880, r=32), moe.MOE_E_UNSUPPORTED),
    # fp32 [S, d] activations of 4 GB
    (dict(T=1 << 17, d=2048, E=16, k=4, F=128, dtype=moe.MOE_F32), moe.MOE_E_UNSUPPORTED),
    # one expert's [F, d] weight above 2 GiB
    (dict(T=8, d=32768, E=2, k=1, F=32768 + 8), moe.MOE_E_UNSUPPORTED),
])
def test_bad_problems_rejected(kw, code):
    p = pb(**kw)
    assert moe.route_workspace(p) == 0 and moe.saved_bytes(p, True) == 0
    fake = 1 << 20  # aligned, never dereferenced: the call fails before any launch
    st = moe.lib().moe_route(ctypes.byref(p), fake, ctypes.byref(_routing(fake)), None, None, 0,
                             None, None)
    assert st == code


def _routing(ptr):
    return moe.Routing(*([ptr] * 6))


def _weights(ptr):
    return moe.Weights(*([ptr] * 9))


def _grads(ptr):
    return moe.LoraGrads(*([ptr] * 6))


def test_argument_errors_before_launch():
    p = pb()
    L = moe.lib()
    A = 1 << 20
    ok_rt, w, g = _routing(A), _weights(A), _grads(A)
    # null / misaligned pointers
    assert L.moe_route(ctypes.byref(p), A, None, None, None, 0, None, None) == moe.MOE_E_ARG
    assert L.moe_route(ctypes.byref(p), A + 4, ctypes.byref(ok_rt), None, None, 0, None,
                       None) == moe.MOE_E_ARG
    bad_rt = _routing(A)
    bad_rt.sorted_slot = None
    assert L.moe_route(ctypes.byref(p), A, ctypes.byref(bad_rt), None, None, 0, None,
                       None) == moe.MOE_E_ARG
    # workspace too small
    assert L.moe_route(ctypes.byref(p), A, ctypes.byref(ok_rt), None, A, 16, None,
                       None) == moe.MOE_E_WORKSPACE
    # forward: missing weight, misaligned out, short workspace
    w2 = _weights(A)
    w2.b_down = None
    assert L.moe_fwd(ctypes.byref(p), A, ctypes.byref(ok_rt), ctypes.byref(w2), A, A, 0, A, 0,
                     None, None) == moe.MOE_E_ARG
    assert L.moe_fwd(ctypes.byref(p), A, ctypes.byref(ok_rt), ctypes.byref(w), A + 8, A, 0, A, 0,
                     None, None) == moe.MOE_E_ARG
    assert L.moe_fwd(ctypes.byref(p), A, ctypes.byref(ok_rt), ctypes.byref(w), A, A, 0, A, 0,
                     None, None) == moe.MOE_E_WORKSPACE
    # backward: saved is required; router gradients need the kept expert outputs
    assert L.moe_bwd(ctypes.byref(p), A, A, ctypes.byref(ok_rt), ctypes.byref(w), None, 1, A,
                     ctypes.byref(g), None, None, A, 0, None, None) == moe.MOE_E_ARG
    assert L.moe_bwd(ctypes.byref(p), A, A, ctypes.byref(ok_rt), ctypes.byref(w), A, 0, A,
                     ctypes.byref(g), A, None, A, 0, None, None) == moe.MOE_E_ARG
    g2 = _grads(A)
    g2.da_up = A + 2
    assert L.moe_bwd(ctypes.byref(p), A, A, ctypes.byref(ok_rt), ctypes.byref(w), A, 1, A,
                     ctypes.byref(g2), None, None, A, 0, None, None) == moe.MOE_E_ARG
    assert L.moe_bwd(ctypes.byref(p), A, A, ctypes.byref(ok_rt), ctypes.byref(w), A, 1, A,
                     ctypes.byref(g), None, None, A, 0, None, None) == moe.MOE_E_WORKSPACE


def test_binding_raises_on_error():
    p = pb(k=99)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(p, 1 << 20, {n: 1 << 20 for n in ("topk_idx", "topk_w", "counts", "offsets",
                                                         "sorted_slot", "slot_row")},
                      stream=0)
    assert ei.value.status == moe.MOE_E_ARG


def test_router_workspace_and_argument_errors():
    p = pb()  # T=512, d=256, E=16
    Tp = (p.T + 7) // 8 * 8
    # token chunks for dW_r: about 256 blocks of 128 x 128 tiles, at most 32,
    # at least ~256 tokens each
    tiles = -(-p.E // 128) * -(-p.d // 128)
    nch0 = min(32, -(-256 // tiles), max(1, -(-p.T // 256)))
    chunk = ((p.T + nch0 - 1) // nch0 + 31) // 32 * 32
    nch = (p.T + chunk - 1) // chunk
    want = al(p.E * Tp * 4) + (al(nch * p.E * p.d * 4) if nch > 1 else 0)
    assert nch == 2 and moe.router_workspace(p) == want
    p12 = pb(E=12, k=2)
    assert moe.router_workspace(p12) == 0
    L, A = moe.lib(), 1 << 20
    assert L.moe_router_fwd(ctypes.byref(p12), A, A, A, None, None) == moe.MOE_E_UNSUPPORTED
    assert L.moe_router_fwd(ctypes.byref(p), A, None, A, None, None) == moe.MOE_E_ARG
    assert L.moe_router_fwd(ctypes.byref(p), A + 4, A, A, None, None) == moe.MOE_E_ARG
    # dx without dx_in; misaligned dw; short workspace for dw
    assert L.moe_router_bwd(ctypes.byref(p), A, A, A, None, A, None, None, 0, None,
                            None) == moe.MOE_E_ARG
    assert L.moe_router_bwd(ctypes.byref(p), A, A, A, None, None, A + 8, A, want, None,
                            None) == moe.MOE_E_ARG
    assert L.moe_router_bwd(ctypes.byref(p), A, A, A, None, None, A, A, want - 1, None,
                            None) == moe.MOE_E_WORKSPACE
    # a router weight above 2 GiB (E d bf16 elements) is refused by both calls
    big = pb(T=8, d=(1 << 20) + 8, E=1024, k=1, F=8)
    assert moe.route_workspace(big) > 0  # the layer itself is accepted
    assert L.moe_router_fwd(ctypes.byref(big), A, A, A, None, None) == moe.MOE_E_UNSUPPORTED
    assert L.moe_router_bwd(ctypes.byref(big), A, A, A, None, None, A, A, 1 << 40, None,
                            None) == moe.MOE_E_UNSUPPORTED


def test_saved_copy_argument_errors_before_any_call():
    p, L, A = pb(), moe.lib(), 1 << 20
    assert L.moe_saved_copy(ctypes.byref(p), 0, 0, A, None, None, None, None) == moe.MOE_E_ARG
    assert L.moe_saved_copy(ctypes.byref(p), 0, 0, None, A, None, None, None) == moe.MOE_E_ARG
    assert L.moe_saved_copy(ctypes.byref(p), 0, 0, A + 8, A, None, None, None) == moe.MOE_E_ARG
    assert L.moe_saved_copy(ctypes.byref(pb(k=0)), 0, 0, A, A, None, None, None) == moe.MOE_E_ARG


def test_nf4_dequant_argument_errors_before_launch():
    L, A = moe.lib(), 1 << 20
    assert L.moe_nf4_dequant(A, A, -1, 64, A, None) == moe.MOE_E_ARG
    assert L.moe_nf4_dequant(A, A, 4, 0, A, None) == moe.MOE_E_ARG
    assert L.moe_nf4_dequant(A, A, 4, 100, A, None) == moe.MOE_E_UNSUPPORTED
    assert L.moe_nf4_dequant(A + 4, A, 4, 64, A, None) == moe.MOE_E_ARG     # codes 16-byte aligned
    assert L.moe_nf4_dequant(A, A + 2, 4, 64, A, None) == moe.MOE_E_ARG     # scales 4-byte aligned
    assert L.moe_nf4_dequant(A, A, 4, 64, A + 8, None) == moe.MOE_E_ARG     # out 16-byte aligned
    assert L.moe_nf4_dequant(None, None, 0, 64, None, None) == moe.MOE_OK   # nothing to do


def test_two_gib_limit_is_in_bytes():
    """Every tensor must fit 2^31 bytes (32-bit byte offsets in the kernels):
    the largest GPT-OSS-120B-shaped batch that fits is accepted, one more
    token is refused."""
    F2 = 2 * 2880
    t_max = (1 << 31) // (F2 * 2) // 4   # S = 4 T slots of [2F] bf16
    ok, over = pb(T=t_max, d=2880, E=128, k=4, F=2880, r=32), pb(T=t_max + 1, d=2880, E=128, k=4, F=2880, r=32)
    assert moe.route_workspace(ok) > 0 and moe.saved_bytes(ok, True) > 0
    assert moe.route_workspace(over) == 0 and moe.saved_bytes(over, True) == 0


def test_binding_checks_host_buffers():
    import numpy as np
    p = pb()
    rt = {n: 1 << 20 for n in ("topk_idx", "topk_w", "counts", "offsets", "sorted_slot", "slot_row")}
    for bad in (np.zeros(p.E - 1, np.int32), np.zeros(p.E, np.int64), np.zeros(p.E, np.float32)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_route(p, 1 << 20, rt, host_counts=bad, stream=0)
        assert ei.value.status == moe.MOE_E_ARG
    short = np.zeros(moe.saved_host_bytes(p, False) - 1, np.uint8)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_saved_copy(p, False, False, 1 << 20, short, copy_stream=0)
    assert ei.value.status == moe.MOE_E_ARG
    # the stack calls' host_saved buffers likewise
    A = 1 << 20
    rt = {n: A for n in ("topk_idx", "topk_w", "counts", "offsets", "sorted_slot", "slot_row")}
    w = {n: A for n in ("w_gate", "w_up", "w_down", "a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")}
    layer = {"logits": A, "rt": rt, "w": w, "x": A, "out": A}
    layers = [dict(layer, host_saved=short), dict(layer), dict(layer)]
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_stack_fwd(p, layers, False, [A, 2 * A], 3 * A, [4 * A] * 4, A, stream=0)
    assert ei.value.status == moe.MOE_E_ARG and "host_saved of layer 0" in str(ei.value)


def test_stack_argument_errors_before_launch():
    p, L, A = pb(), moe.lib(), 1 << 20
    assert moe.stack_workspace(pb(k=0), False) == 0
    need = moe.stack_workspace(p, False)
    assert need == max(moe.route_workspace(p), moe.fwd_workspace(p, True, False), moe.bwd_workspace(p))
    rt, w, g = _routing(A), _weights(A), _grads(A)

    def layers(n, host=A):
        arr = (moe.StackLayer * n)()
        for i in range(n):
            arr[i] = moe.StackLayer(A, ctypes.pointer(rt), ctypes.pointer(w), A, A, A, A,
                                    ctypes.pointer(g), None, None, host)
        return arr

    def off(s0=A, s1=2 * A, cs=3 * A, ev=4 * A):
        return moe.Offload((ctypes.c_void_p * 2)(s0, s1), cs, (ctypes.c_void_p * 4)(ev, ev, ev, ev))

    for fn in (L.moe_stack_fwd, L.moe_stack_bwd):
        assert fn(ctypes.byref(p), 0, layers(1), 0, ctypes.byref(off()), A, need, None) == moe.MOE_E_ARG
        assert fn(ctypes.byref(p), 2, layers(2), 0, ctypes.byref(off()), A, need - 1, None) == moe.MOE_E_WORKSPACE
        assert fn(ctypes.byref(p), 2, layers(2), 0, ctypes.byref(off(s1=A)), A, need, None) == moe.MOE_E_ARG
        assert fn(ctypes.byref(p), 3, layers(3), 0, ctypes.byref(off(cs=None)), A, need, None) == moe.MOE_E_ARG
        assert fn(ctypes.byref(p), 3, layers(3), 0, ctypes.byref(off(ev=None)), A, need, None) == moe.MOE_E_ARG
        # host memory of the offloaded layers must be pinned (a fake address is not)
        assert fn(ctypes.byref(p), 3, layers(3), 0, ctypes.byref(off()), A, need, None) == moe.MOE_E_ARG
        assert fn(ctypes.byref(pb(k=0)), 1, layers(1), 0, ctypes.byref(off()), A, need, None) == moe.MOE_E_ARG


def test_nf4_layer_argument_errors_before_launch():
    L, A = moe.lib(), 1 << 20
    p = pb(d=256, F=128)
    rt, w, g = _routing(A), _weights(A), _grads(A)
    q = moe.Nf4Base(A, A, A, A, A, A)
    # fp32 layers and d or F not a multiple of 64 are unsupported
    for bad in (pb(dtype=moe.MOE_F32), pb(d=200), pb(F=136)):
        assert L.moe_fwd_nf4(ctypes.byref(bad), A, ctypes.byref(rt), ctypes.byref(w), ctypes.byref(q), A, A, 0,
                             A, 1 << 40, None, None) == moe.MOE_E_UNSUPPORTED
    assert L.moe_fwd_nf4(ctypes.byref(p), A, ctypes.byref(rt), ctypes.byref(w), None, A, A, 0, A, 1 << 40,
                         None, None) == moe.MOE_E_ARG
    q2 = moe.Nf4Base(A + 8, A, A, A, A, A)   # codes must be 16-byte aligned
    assert L.moe_fwd_nf4(ctypes.byref(p), A, ctypes.byref(rt), ctypes.byref(w), ctypes.byref(q2), A, A, 0, A,
                         1 << 40, None, None) == moe.MOE_E_ARG
    q3 = moe.Nf4Base(A, A, A, A, A + 2, A)   # scales 4-byte aligned
    assert L.moe_bwd_nf4(ctypes.byref(p), A, A, ctypes.byref(rt), ctypes.byref(w), ctypes.byref(q3), A, 1, A,
                         ctypes.byref(g), None, None, A, 1 << 40, None, None) == moe.MOE_E_ARG
    # base-weight pointers are not needed, the LoRA factors are
    w0 = _weights(A)
    w0.w_gate = w0.w_up = w0.w_down = None
    assert L.moe_fwd_nf4(ctypes.byref(p), A, ctypes.byref(rt), ctypes.byref(w0), ctypes.byref(q), A, A, 0, A,
                         0, None, None) == moe.MOE_E_WORKSPACE
    w0.a_up = None
    assert L.moe_fwd_nf4(ctypes.byref(p), A, ctypes.byref(rt), ctypes.byref(w0), ctypes.byref(q), A, A, 0, A,
                         1 << 40, None, None) == moe.MOE_E_ARG
