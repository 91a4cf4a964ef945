"""Python binding of libmoe.so, the gfx950 MoE expert layer with Split-LoRA.

Argument marshalling only: every step of routing, forward and backward runs
in the library's HIP kernels (declared in ``include/moe.h``). PyTorch is
used for device memory and streams. There is no fallback: if the library
is missing the import fails.

The three calls keep the C names:

    moe_route(pb, logits, rt, host_counts=None, ws=None, stream=None, trace=None)
    moe_fwd(pb, x, rt, w, out, saved=None, keep_expert_out=False, ws=None, ...)
    moe_bwd(pb, x, dout, rt, w, saved, keep_expert_out, dx, grads, d_topk_w=None,
            d_logits=None, ws=None, ...)

Tensors may be torch tensors (their data_ptr() is passed) or raw integer
device addresses. ``stream`` is a torch.cuda.Stream, a raw hipStream_t int or
None for torch's current stream.
"""
from __future__ import annotations

import ctypes
import os

try:  # torch first: libmoe.so then binds to the HIP runtime torch already
    import torch  # noqa: F401  # loaded, so both share one runtime and its streams
except ImportError:  # host-only use (size queries, argument checks)
    torch = None

from ._build import LIB_PATH, build  # noqa: F401

MOE_OK, MOE_E_ARG, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1

KERNELS = ["route_topk", "route_scan", "route_scatter", "proj_gu", "gateup", "proj_d", "down",
           "combine", "router_grad", "proj_dout", "down_bwd", "proj_dgu", "gateup_bwd",
           "dx_combine", "lora_grad", "router_logits", "router_dx", "router_dw"]
MOE_K_COUNT = len(KERNELS)

EXPORTS = ["moe_route_workspace", "moe_fwd_workspace", "moe_bwd_workspace", "moe_saved_bytes",
           "moe_route", "moe_fwd", "moe_bwd", "moe_status_str", "moe_router_workspace",
           "moe_router_fwd", "moe_router_bwd", "moe_saved_copy", "moe_nf4_dequant",
           "moe_workspace_part", "moe_route_noalloc", "moe_stack_workspace", "moe_stack_fwd",
           "moe_stack_bwd", "moe_fwd_nf4", "moe_bwd_nf4", "moe_saved_host_bytes"]
MOE_PART_Y, MOE_PART_DGU, MOE_PART_DXP = range(3)


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("F", ctypes.c_int32), ("r", ctypes.c_int32),
                ("lora_scale", ctypes.c_float), ("dtype", ctypes.c_int32)]

    @classmethod
    def from_config(cls, cfg, T=None):
        return cls(cfg.T if T is None else T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.r, cfg.s,
                   MOE_BF16 if cfg.dtype == "bf16" else MOE_F32)

    @property
    def S(self):
        return self.T * self.k


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "counts", "offsets", "sorted_slot", "slot_row")]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_gate", "w_up", "w_down", "a_gate", "b_gate", "a_up", "b_up", "a_down",
                 "b_down")]


class Nf4Base(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("codes_gate", "codes_up", "codes_down", "scales_gate", "scales_up", "scales_down")]


class LoraGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down")]


class StackLayer(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("rt", ctypes.POINTER(Routing)),
                ("w", ctypes.POINTER(Weights)), ("x", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("dout", ctypes.c_void_p), ("dx", ctypes.c_void_p),
                ("grads", ctypes.POINTER(LoraGrads)), ("d_topk_w", ctypes.c_void_p),
                ("d_logits", ctypes.c_void_p), ("host_saved", ctypes.c_void_p)]


class Offload(ctypes.Structure):
    _fields_ = [("saved", ctypes.c_void_p * 2), ("copy_stream", ctypes.c_void_p),
                ("events", ctypes.c_void_p * 4)]


class Trace(ctypes.Structure):
    _fields_ = [("start", ctypes.c_void_p * MOE_K_COUNT), ("stop", ctypes.c_void_p * MOE_K_COUNT)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (or "
                      "python __graft_entry__.py) first")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.POINTER
_vp, _sz, _i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_lib.moe_route_workspace.argtypes = [_P(Problem)]
_lib.moe_fwd_workspace.argtypes = [_P(Problem), _i32, _i32]
_lib.moe_bwd_workspace.argtypes = [_P(Problem)]
_lib.moe_saved_bytes.argtypes = [_P(Problem), _i32]
_lib.moe_saved_host_bytes.argtypes = [_P(Problem), _i32]
for _f in (_lib.moe_route_workspace, _lib.moe_fwd_workspace, _lib.moe_bwd_workspace,
           _lib.moe_saved_bytes, _lib.moe_saved_host_bytes):
    _f.restype = _sz
_lib.moe_route.argtypes = [_P(Problem), _vp, _P(Routing), _vp, _vp, _sz, _vp, _P(Trace)]
_lib.moe_route_noalloc.argtypes = [_P(Problem), _vp, _P(Routing), _vp, _vp, _P(Trace)]
_lib.moe_fwd.argtypes = [_P(Problem), _vp, _P(Routing), _P(Weights), _vp, _vp, _i32, _vp, _sz,
                         _vp, _P(Trace)]
_lib.moe_bwd.argtypes = [_P(Problem), _vp, _vp, _P(Routing), _P(Weights), _vp, _i32, _vp,
                         _P(LoraGrads), _vp, _vp, _vp, _sz, _vp, _P(Trace)]
_lib.moe_workspace_part.argtypes = [_P(Problem), _i32, _i32, _i32]
_lib.moe_workspace_part.restype = _sz
_lib.moe_stack_workspace.argtypes = [_P(Problem), _i32]
_lib.moe_stack_workspace.restype = _sz
_lib.moe_stack_fwd.argtypes = [_P(Problem), _i32, _P(StackLayer), _i32, _P(Offload), _vp, _sz, _vp]
_lib.moe_stack_bwd.argtypes = [_P(Problem), _i32, _P(StackLayer), _i32, _P(Offload), _vp, _sz, _vp]
_lib.moe_stack_fwd.restype = _i32
_lib.moe_stack_bwd.restype = _i32
_lib.moe_fwd_nf4.argtypes = [_P(Problem), _vp, _P(Routing), _P(Weights), _P(Nf4Base), _vp, _vp, _i32, _vp,
                             _sz, _vp, _P(Trace)]
_lib.moe_bwd_nf4.argtypes = [_P(Problem), _vp, _vp, _P(Routing), _P(Weights), _P(Nf4Base), _vp, _i32, _vp,
                             _P(LoraGrads), _vp, _vp, _vp, _sz, _vp, _P(Trace)]
_lib.moe_fwd_nf4.restype = _i32
_lib.moe_bwd_nf4.restype = _i32
_lib.moe_router_workspace.argtypes = [_P(Problem)]
_lib.moe_router_workspace.restype = _sz
_lib.moe_router_fwd.argtypes = [_P(Problem), _vp, _vp, _vp, _vp, _P(Trace)]
_lib.moe_router_bwd.argtypes = [_P(Problem), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _P(Trace)]
_lib.moe_saved_copy.argtypes = [_P(Problem), _i32, _i32, _vp, _vp, _vp, _vp, _vp]
_lib.moe_nf4_dequant.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp]
_lib.moe_nf4_dequant.restype = _i32
for _f in (_lib.moe_route, _lib.moe_route_noalloc, _lib.moe_fwd, _lib.moe_bwd, _lib.moe_router_fwd, _lib.moe_router_bwd,
           _lib.moe_saved_copy):
    _f.restype = _i32
_lib.moe_status_str.argtypes = [_i32]
_lib.moe_status_str.restype = ctypes.c_char_p


class MoeError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {moe_status_str(status)} (status {status})")


def lib():
    return _lib


def moe_status_str(st: int) -> str:
    return _lib.moe_status_str(st).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    if t is None:
        return 0
    if isinstance(t, int):
        raise TypeError("pass a workspace tensor (its size is needed), not a raw address")
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _struct(cls, d):
    return cls(*[_ptr(d.get(n)) for n, _ in cls._fields_])


def route_workspace(pb: Problem) -> int:
    return _lib.moe_route_workspace(ctypes.byref(pb))


def fwd_workspace(pb: Problem, training: bool, keep_expert_out: bool) -> int:
    return _lib.moe_fwd_workspace(ctypes.byref(pb), int(training), int(keep_expert_out))


def bwd_workspace(pb: Problem) -> int:
    return _lib.moe_bwd_workspace(ctypes.byref(pb))


def saved_bytes(pb: Problem, keep_expert_out: bool) -> int:
    return _lib.moe_saved_bytes(ctypes.byref(pb), int(keep_expert_out))


def saved_host_bytes(pb: Problem, keep_expert_out: bool) -> int:
    """Bytes of `saved` an offload moves to host memory (all of it but H)."""
    return _lib.moe_saved_host_bytes(ctypes.byref(pb), int(keep_expert_out))


def _check(st, what):
    if st != MOE_OK:
        raise MoeError(st, what)


def _host_buffer(a, what):
    """(address, bytes, dtype name) of a host numpy array or CPU torch tensor."""
    if hasattr(a, "ctypes"):  # numpy
        return a.ctypes.data, a.nbytes, str(a.dtype)
    if getattr(a, "is_cuda", False):
        raise MoeError(MOE_E_ARG, f"{what}: a host buffer is needed, got a device tensor")
    return a.data_ptr(), a.numel() * a.element_size(), str(a.dtype).replace("torch.", "")


def moe_route(pb, logits, rt: dict, host_counts=None, ws=None, stream=None, trace=None):
    """rt: dict of the six routing tensors; host_counts: CPU int32 tensor/array
    of at least E elements, or None. The library writes E int32 counts there,
    so a shorter or differently typed buffer is refused before the call."""
    hc = None
    if host_counts is not None:
        hc, nbytes, dt = _host_buffer(host_counts, "moe_route host_counts")
        if dt != "int32" or nbytes < 4 * pb.E:
            raise MoeError(MOE_E_ARG, f"moe_route host_counts: need int32[{pb.E}], got {dt} "
                                      f"of {nbytes} bytes")
    st = _lib.moe_route(ctypes.byref(pb), _ptr(logits), ctypes.byref(_struct(Routing, rt)), hc,
                        _ptr(ws), _nbytes(ws), _stream(stream),
                        ctypes.byref(trace) if trace is not None else None)
    _check(st, "moe_route")


def moe_route_noalloc(pb, logits, rt: dict, host_counts=None, stream=None, trace=None):
    """moe_route without a workspace: the library's own device scratch array
    (for callers that cannot allocate). host_counts: None or a pinned CPU int32
    tensor of at least E elements."""
    hc = None
    if host_counts is not None:
        hc, nbytes, dt = _host_buffer(host_counts, "moe_route_noalloc host_counts")
        if dt != "int32" or nbytes < 4 * pb.E:
            raise MoeError(MOE_E_ARG, f"moe_route_noalloc host_counts: need int32[{pb.E}], got {dt} "
                                      f"of {nbytes} bytes")
    st = _lib.moe_route_noalloc(ctypes.byref(pb), _ptr(logits), ctypes.byref(_struct(Routing, rt)), hc,
                                _stream(stream), ctypes.byref(trace) if trace is not None else None)
    _check(st, "moe_route_noalloc")


def moe_fwd(pb, x, rt: dict, w: dict, out, saved=None, keep_expert_out=False, ws=None,
            stream=None, trace=None):
    st = _lib.moe_fwd(ctypes.byref(pb), _ptr(x), ctypes.byref(_struct(Routing, rt)),
                      ctypes.byref(_struct(Weights, w)), _ptr(out), _ptr(saved),
                      int(keep_expert_out), _ptr(ws), _nbytes(ws), _stream(stream),
                      ctypes.byref(trace) if trace is not None else None)
    _check(st, "moe_fwd")


def moe_bwd(pb, x, dout, rt: dict, w: dict, saved, keep_expert_out, dx, grads: dict,
            d_topk_w=None, d_logits=None, ws=None, stream=None, trace=None):
    st = _lib.moe_bwd(ctypes.byref(pb), _ptr(x), _ptr(dout), ctypes.byref(_struct(Routing, rt)),
                      ctypes.byref(_struct(Weights, w)), _ptr(saved), int(keep_expert_out),
                      _ptr(dx), ctypes.byref(_struct(LoraGrads, grads)), _ptr(d_topk_w),
                      _ptr(d_logits), _ptr(ws), _nbytes(ws), _stream(stream),
                      ctypes.byref(trace) if trace is not None else None)
    _check(st, "moe_bwd")


def moe_fwd_nf4(pb, x, rt: dict, w: dict, q4: dict, out, saved=None, keep_expert_out=False, ws=None,
                stream=None, trace=None):
    """moe_fwd with the base weights in NF4: q4 holds codes_gate/up/down and
    scales_gate/up/down; w needs only the LoRA factors."""
    st = _lib.moe_fwd_nf4(ctypes.byref(pb), _ptr(x), ctypes.byref(_struct(Routing, rt)),
                          ctypes.byref(_struct(Weights, w)), ctypes.byref(_struct(Nf4Base, q4)), _ptr(out),
                          _ptr(saved), int(keep_expert_out), _ptr(ws), _nbytes(ws), _stream(stream),
                          ctypes.byref(trace) if trace is not None else None)
    _check(st, "moe_fwd_nf4")


def moe_bwd_nf4(pb, x, dout, rt: dict, w: dict, q4: dict, saved, keep_expert_out, dx, grads: dict,
                d_topk_w=None, d_logits=None, ws=None, stream=None, trace=None):
    """moe_bwd with the base weights in NF4 (see moe_fwd_nf4)."""
    st = _lib.moe_bwd_nf4(ctypes.byref(pb), _ptr(x), _ptr(dout), ctypes.byref(_struct(Routing, rt)),
                          ctypes.byref(_struct(Weights, w)), ctypes.byref(_struct(Nf4Base, q4)), _ptr(saved),
                          int(keep_expert_out), _ptr(dx), ctypes.byref(_struct(LoraGrads, grads)),
                          _ptr(d_topk_w), _ptr(d_logits), _ptr(ws), _nbytes(ws), _stream(stream),
                          ctypes.byref(trace) if trace is not None else None)
    _check(st, "moe_bwd_nf4")


def router_workspace(pb: Problem) -> int:
    return _lib.moe_router_workspace(ctypes.byref(pb))


def moe_router_fwd(pb, x, w_router, logits, stream=None, trace=None):
    """logits [T,E] fp32 = x [T,d] W_r^T (w_router [E,d] in the layer dtype)."""
    st = _lib.moe_router_fwd(ctypes.byref(pb), _ptr(x), _ptr(w_router), _ptr(logits), _stream(stream),
                             ctypes.byref(trace) if trace is not None else None)
    _check(st, "moe_router_fwd")


def moe_router_bwd(pb, x, w_router, d_logits, dx_in=None, dx=None, dw_router=None, ws=None,
                   stream=None, trace=None):
    """dx = dx_in + d_logits W_r (dx may be dx_in); dw_router = d_logits^T x."""
    st = _lib.moe_router_bwd(ctypes.byref(pb), _ptr(x), _ptr(w_router), _ptr(d_logits), _ptr(dx_in),
                             _ptr(dx), _ptr(dw_router), _ptr(ws), _nbytes(ws), _stream(stream),
                             ctypes.byref(trace) if trace is not None else None)
    _check(st, "moe_router_bwd")


def moe_saved_copy(pb, keep_expert_out, to_device, saved, host, wait_event=None, copy_stream=None,
                   done_event=None):
    """Copy a `saved` buffer (all but H) to (to_device=False) or from a
    pinned host tensor of saved_host_bytes on copy_stream, after wait_event (a
    torch.cuda.Event or raw hipEvent_t); a reload then rebuilds H from G and U
    on copy_stream; records done_event on copy_stream."""
    def ev(e):
        if e is None or isinstance(e, int):
            return e
        return e.cuda_event
    if isinstance(host, int):
        hp = host
    else:
        hp, nbytes, _ = _host_buffer(host, "moe_saved_copy host")
        need = saved_host_bytes(pb, keep_expert_out)
        if nbytes < need:
            raise MoeError(MOE_E_ARG, f"moe_saved_copy host: {nbytes} bytes, the offloaded part of "
                                      f"saved is {need}")
    st = _lib.moe_saved_copy(ctypes.byref(pb), int(keep_expert_out), int(to_device), _ptr(saved), hp,
                             ev(wait_event), _stream(copy_stream), ev(done_event))
    _check(st, "moe_saved_copy")


def stack_workspace(pb: Problem, keep_expert_out: bool) -> int:
    return _lib.moe_stack_workspace(ctypes.byref(pb), int(keep_expert_out))


def _stack_args(pb, keep_expert_out, layers, saved, copy_stream, events):
    """ctypes arrays for the stack calls; the returned tuple keeps every
    referenced structure alive for the duration of the call. A host_saved
    buffer shorter than saved_host_bytes is refused here (the C ABI cannot
    see its size)."""
    keep = []
    need = saved_host_bytes(pb, keep_expert_out)
    arr = (StackLayer * len(layers))()
    for i, L in enumerate(layers):
        rt, w = _struct(Routing, L["rt"]), _struct(Weights, L["w"])
        g = _struct(LoraGrads, L["grads"]) if L.get("grads") is not None else None
        keep += [rt, w, g]
        hs = L.get("host_saved")
        if hs is not None and not isinstance(hs, int):
            nbytes = _host_buffer(hs, "host_saved")[1]
            if nbytes < need:
                raise MoeError(MOE_E_ARG, f"host_saved of layer {i}: {nbytes} bytes, need {need}")
        arr[i] = StackLayer(_ptr(L.get("logits")), ctypes.pointer(rt), ctypes.pointer(w), _ptr(L.get("x")),
                            _ptr(L.get("out")), _ptr(L.get("dout")), _ptr(L.get("dx")),
                            ctypes.pointer(g) if g is not None else None, _ptr(L.get("d_topk_w")),
                            _ptr(L.get("d_logits")),
                            hs if (hs is None or isinstance(hs, int)) else _host_buffer(hs, "host_saved")[0])

    def ev(e):
        if e is None or isinstance(e, int):
            return e
        h = e.cuda_event
        if not h:
            raise MoeError(MOE_E_ARG, "stack events: a torch.cuda.Event has no HIP event until it is "
                                      "first recorded; record each once before passing it")
        return h
    off = Offload((ctypes.c_void_p * 2)(_ptr(saved[0]), _ptr(saved[1]) if len(saved) > 1 else None),
                  None if copy_stream is None else _stream(copy_stream),
                  (ctypes.c_void_p * 4)(*[ev(e) for e in events]))
    return arr, off, keep


def moe_stack_fwd(pb, layers: list, keep_expert_out, saved, copy_stream, events, ws, stream=None):
    """Forward of a stack of layers with saved activations offloaded to each
    layer's pinned host_saved through the two device buffers `saved`.
    layers: dicts with logits, rt, w, x, out, host_saved (see moe.h)."""
    arr, off, _keep = _stack_args(pb, keep_expert_out, layers, saved, copy_stream, events)
    st = _lib.moe_stack_fwd(ctypes.byref(pb), len(layers), arr, int(keep_expert_out), ctypes.byref(off),
                            _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "moe_stack_fwd")


def moe_stack_bwd(pb, layers: list, keep_expert_out, saved, copy_stream, events, ws, stream=None):
    """Backward of the stack moe_stack_fwd ran: layers additionally carry dout,
    dx, grads and optionally d_topk_w / d_logits."""
    arr, off, _keep = _stack_args(pb, keep_expert_out, layers, saved, copy_stream, events)
    st = _lib.moe_stack_bwd(ctypes.byref(pb), len(layers), arr, int(keep_expert_out), ctypes.byref(off),
                            _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "moe_stack_bwd")


def moe_nf4_dequant(codes, scales, rows, cols, out, stream=None):
    """bf16 out [rows, cols] = NF4 level[code] * scale (codes [rows, cols/2]
    uint8, low nibble first; scales [rows, cols/64] fp32)."""
    st = _lib.moe_nf4_dequant(_ptr(codes), _ptr(scales), int(rows), int(cols), _ptr(out),
                              _stream(stream))
    _check(st, "moe_nf4_dequant")


# ---------------------------------------------------------------- allocation helpers
def alloc_routing(pb: Problem, device):
    T, E, k = pb.T, pb.E, pb.k
    i32 = torch.int32
    return {"topk_idx": torch.empty((T, k), dtype=i32, device=device),
            "topk_w": torch.empty((T, k), dtype=torch.float32, device=device),
            "counts": torch.empty(E, dtype=i32, device=device),
            "offsets": torch.empty(E + 1, dtype=i32, device=device),
            "sorted_slot": torch.empty(T * k, dtype=i32, device=device),
            "slot_row": torch.empty(T * k, dtype=i32, device=device)}


def alloc_bytes(n: int, device):
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def alloc_grads(pb: Problem, device):
    E, d, F, r = pb.E, pb.d, pb.F, pb.r
    f = torch.float32
    return {"da_gate": torch.empty((E, r, d), dtype=f, device=device),
            "db_gate": torch.empty((E, F, r), dtype=f, device=device),
            "da_up": torch.empty((E, r, d), dtype=f, device=device),
            "db_up": torch.empty((E, F, r), dtype=f, device=device),
            "da_down": torch.empty((E, r, F), dtype=f, device=device),
            "db_down": torch.empty((E, d, r), dtype=f, device=device)}


def workspace_part(pb: Problem, part: int, training: bool = True, keep_expert_out: bool = False):
    """Byte offset of an inspectable intermediate in a workspace (MOE_PART_*), or None."""
    o = _lib.moe_workspace_part(ctypes.byref(pb), int(part), int(training), int(keep_expert_out))
    return None if o == ctypes.c_size_t(-1).value else int(o)


def workspace_views(pb: Problem, ws_fwd=None, ws_bwd=None, training=True,
                    keep_expert_out=False) -> dict:
    """Typed views of the intermediates the workspaces hold after moe_fwd /
    moe_bwd: Y (fwd workspace, if held there), dGU [S,2F] and dXp [S,d]."""
    S, F, d = pb.S, pb.F, pb.d
    dt = torch.bfloat16 if pb.dtype == MOE_BF16 else torch.float32
    es = 2 if pb.dtype == MOE_BF16 else 4
    out = {}
    for name, buf, part, cols in (("Y", ws_fwd, MOE_PART_Y, d), ("dGU", ws_bwd, MOE_PART_DGU, 2 * F),
                                  ("dXp", ws_bwd, MOE_PART_DXP, d)):
        if buf is None:
            continue
        o = workspace_part(pb, part, training, keep_expert_out)
        if o is not None:
            out[name] = buf[o:o + S * cols * es].view(dt).view(S, cols)
    return out


def saved_views(pb: Problem, saved, keep_expert_out: bool) -> dict:
    """Typed views of the `saved` buffer (layout documented in moe.h)."""
    S, F, r, d = pb.S, pb.F, pb.r, pb.d
    bf = pb.dtype == MOE_BF16
    dt = torch.bfloat16 if bf else torch.float32
    es = 2 if bf else 4

    def al(x):
        return (x + 255) // 256 * 256

    parts = [("G", (S, F), dt, es), ("U", (S, F), dt, es),
             ("Zgu", (S, 2 * r), torch.float32, 4), ("Zd", (S, r), torch.float32, 4)]
    ldT = (S + 7) // 8 * 8
    if bf:
        parts += [("ZguT", (2 * r, ldT), torch.bfloat16, 2), ("wZdT", (r, ldT), torch.bfloat16, 2)]
    if keep_expert_out:
        parts += [("Y", (S, d), dt, es)]
    parts += [("H", (S, F), dt, es)]
    out, o = {}, 0
    for name, shape, t, e in parts:
        n = shape[0] * shape[1]
        out[name] = saved[o:o + n * e].view(t).view(*shape)
        o += al(n * e)
    for name in ("ZguT", "wZdT"):
        if name in out:
            out[name] = out[name][:, :S]
    return out
