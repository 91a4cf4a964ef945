"""ctypes front-end of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library. It shares no code with
the HIP path; its inputs come from the ``synth`` generator.

Every function returns numpy float64 (or int32 for routing) arrays computed
in fp64 from the stored inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
             os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layer(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("F", ctypes.c_int32), ("r", ctypes.c_int32),
                ("s", ctypes.c_double), ("dtype", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in ("x", "w_gate", "w_up", "w_down", "a_gate", "b_gate",
                                       "a_up", "b_up", "a_down", "b_down")]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lp = ctypes.POINTER(_Layer)
        lib.orc_route.argtypes = [i32, i32, i32] + [vp] * 7
        lib.orc_fwd.argtypes = [lp] + [vp] * 13
        lib.orc_bwd.argtypes = [lp] + [vp] * 17
        lib.orc_fwd_tokens.argtypes = [lp, vp, vp, i32, vp, vp, vp]
        lib.orc_bwd_tokens.argtypes = [lp, vp, vp, vp, i32, vp, vp, vp, vp]
        lib.orc_lora_grads.argtypes = [lp, vp, vp, vp, vp, vp, i32, vp] + [vp] * 6
        lib.orc_router_fwd.argtypes = [i32, i32, i32, i32, vp, vp, vp]
        lib.orc_router_bwd.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
        for f in (lib.orc_route, lib.orc_fwd, lib.orc_bwd, lib.orc_fwd_tokens,
                  lib.orc_bwd_tokens, lib.orc_lora_grads, lib.orc_router_fwd, lib.orc_router_bwd):
            f.restype = ctypes.c_int
        lib.orc_threads.argtypes = []
        lib.orc_threads.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_threads())


def set_threads(n: int) -> None:
    """Number of OpenMP threads for the oracle's parallel loops."""
    _load().orc_set_threads(int(n))


def _p(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


class Layer:
    """One layer instance: dims, LoRA scale and the stored input tensors.

    ``tensors`` holds x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up,
    a_down, b_down, all in one storage dtype: 'f32' (float32), 'bf16'
    (uint16 bit patterns) or 'f64' (float64, for finite-difference checks).
    """

    NAMES = ("x", "w_gate", "w_up", "w_down", "a_gate", "b_gate", "a_up", "b_up",
             "a_down", "b_down")

    _NP = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}
    _CODE = {"f32": 0, "bf16": 1, "f64": 2}

    def __init__(self, T, d, E, k, F, r, s, dtype, tensors):
        self.T, self.d, self.E, self.k, self.F, self.r = T, d, E, k, F, r
        self.s, self.dtype = float(s), dtype
        want = self._NP[dtype]
        shapes = {"x": (T, d), "w_gate": (E, F, d), "w_up": (E, F, d), "w_down": (E, d, F),
                  "a_gate": (E, r, d), "b_gate": (E, F, r), "a_up": (E, r, d),
                  "b_up": (E, F, r), "a_down": (E, r, F), "b_down": (E, d, r)}
        self.t = {}
        for n in self.NAMES:
            a = np.ascontiguousarray(tensors[n])
            if a.dtype != want or a.shape != shapes[n]:
                raise ValueError(f"{n}: got {a.dtype}{a.shape}, want {want}{shapes[n]}")
            self.t[n] = a
        self._c = _Layer(T, d, E, k, F, r, self.s, self._CODE[dtype],
                         *[self.t[n].ctypes.data for n in self.NAMES])

    @classmethod
    def from_config(cls, cfg, inputs, tokens=None, s=None):
        T = cfg.T if tokens is None else tokens
        return cls(T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.r, cfg.s if s is None else s,
                   cfg.dtype, inputs)

    def store(self, a):
        """Check that a dout-like [T,d] array is in this layer's storage dtype."""
        want = self._NP[self.dtype]
        a = np.ascontiguousarray(a)
        if a.dtype != want or a.shape != (self.T, self.d):
            raise ValueError(f"dout: got {a.dtype}{a.shape}")
        return a


def route(logits: np.ndarray, k: int) -> dict:
    """Top-k by (logit desc, id asc), softmax over the selected, per-expert grouping."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    S = T * k
    out = {"topk_idx": np.empty((T, k), np.int32), "topk_w": np.empty((T, k), np.float64),
           "counts": np.empty(E, np.int32), "offsets": np.empty(E + 1, np.int32),
           "sorted_slot": np.empty(S, np.int32), "slot_row": np.empty(S, np.int32)}
    _check(_load().orc_route(T, E, k, logits.ctypes.data, *[out[n].ctypes.data for n in (
        "topk_idx", "topk_w", "counts", "offsets", "sorted_slot", "slot_row")]), "route")
    return out


def fwd(L: Layer, rt: dict, intermediates: bool = False) -> dict:
    S = L.T * L.k
    out = np.empty((L.T, L.d), np.float64)
    inter = {}
    if intermediates:
        inter = {"G": np.empty((S, L.F)), "U": np.empty((S, L.F)), "H": np.empty((S, L.F)),
                 "Zg": np.empty((S, L.r)), "Zu": np.empty((S, L.r)), "Zd": np.empty((S, L.r)),
                 "Y": np.empty((S, L.d))}
    g = inter.get
    _check(_load().orc_fwd(ctypes.byref(L._c), _p(rt["topk_idx"]), _p(rt["topk_w"]),
                           _p(rt["offsets"]), _p(rt["sorted_slot"]), _p(rt["slot_row"]),
                           out.ctypes.data, _p(g("G")), _p(g("U")), _p(g("H")), _p(g("Zg")),
                           _p(g("Zu")), _p(g("Zd")), _p(g("Y"))), "fwd")
    inter["out"] = out
    return inter


def bwd(L: Layer, rt: dict, dout: np.ndarray, intermediates: bool = False) -> dict:
    dout = L.store(dout)
    T, d, E, k, F, r = L.T, L.d, L.E, L.k, L.F, L.r
    S = T * k
    o = {"dx": np.empty((T, d)), "da_gate": np.empty((E, r, d)), "db_gate": np.empty((E, F, r)),
         "da_up": np.empty((E, r, d)), "db_up": np.empty((E, F, r)),
         "da_down": np.empty((E, r, F)), "db_down": np.empty((E, d, r)),
         "d_topk_w": np.empty((T, k)), "d_logits": np.empty((T, E))}
    if intermediates:
        o.update({"dG": np.empty((S, F)), "dU": np.empty((S, F)), "dXp": np.empty((S, d))})
    g = o.get
    _check(_load().orc_bwd(ctypes.byref(L._c), _p(rt["topk_idx"]), _p(rt["topk_w"]),
                           _p(rt["offsets"]), _p(rt["sorted_slot"]), dout.ctypes.data,
                           *[_p(g(n)) for n in ("dx", "da_gate", "db_gate", "da_up", "db_up",
                                                "da_down", "db_down", "d_topk_w", "d_logits",
                                                "dG", "dU", "dXp")]), "bwd")
    return o


def fwd_tokens(L: Layer, rt: dict, tokens) -> dict:
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n = len(tokens)
    out = np.empty((n, L.d))
    y = np.empty((n, L.k, L.d))
    _check(_load().orc_fwd_tokens(ctypes.byref(L._c), _p(rt["topk_idx"]), _p(rt["topk_w"]),
                                  n, tokens.ctypes.data, out.ctypes.data, y.ctypes.data),
           "fwd_tokens")
    return {"out": out, "y": y}


def bwd_tokens(L: Layer, rt: dict, dout: np.ndarray, tokens) -> dict:
    dout = L.store(dout)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n = len(tokens)
    o = {"dx": np.empty((n, L.d)), "d_topk_w": np.empty((n, L.k)),
         "d_logits": np.empty((n, L.E))}
    _check(_load().orc_bwd_tokens(ctypes.byref(L._c), _p(rt["topk_idx"]), _p(rt["topk_w"]),
                                  dout.ctypes.data, n, tokens.ctypes.data, o["dx"].ctypes.data,
                                  o["d_topk_w"].ctypes.data, o["d_logits"].ctypes.data),
           "bwd_tokens")
    return o


def lora_grads(L: Layer, rt: dict, dout: np.ndarray, experts) -> dict:
    dout = L.store(dout)
    experts = np.ascontiguousarray(experts, dtype=np.int32)
    n, d, F, r = len(experts), L.d, L.F, L.r
    o = {"da_gate": np.empty((n, r, d)), "db_gate": np.empty((n, F, r)),
         "da_up": np.empty((n, r, d)), "db_up": np.empty((n, F, r)),
         "da_down": np.empty((n, r, F)), "db_down": np.empty((n, d, r))}
    _check(_load().orc_lora_grads(ctypes.byref(L._c), _p(rt["topk_idx"]), _p(rt["topk_w"]),
                                  _p(rt["offsets"]), _p(rt["sorted_slot"]), dout.ctypes.data, n,
                                  experts.ctypes.data,
                                  *[o[k].ctypes.data for k in ("da_gate", "db_gate", "da_up",
                                                               "db_up", "da_down", "db_down")]),
           "lora_grads")
    return o


_DTYPE_CODE = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}


def router_fwd(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """Router logits x W_r^T in fp64. x [T,d] and w_r [E,d] in one storage
    dtype (float32, bf16 bits as uint16, or float64)."""
    x, w_r = np.ascontiguousarray(x), np.ascontiguousarray(w_r)
    if x.dtype != w_r.dtype or x.ndim != 2 or w_r.ndim != 2 or x.shape[1] != w_r.shape[1]:
        raise ValueError(f"router_fwd: x {x.dtype}{x.shape}, w_r {w_r.dtype}{w_r.shape}")
    T, d = x.shape
    E = w_r.shape[0]
    out = np.empty((T, E))
    _check(_load().orc_router_fwd(T, d, E, _DTYPE_CODE[x.dtype], x.ctypes.data, w_r.ctypes.data,
                                  out.ctypes.data), "router_fwd")
    return out


def router_bwd(x: np.ndarray, w_r: np.ndarray, d_logits: np.ndarray) -> dict:
    """The router projection's backward for a gradient d_logits [T,E] of its
    output: {"dx": d_logits W_r [T,d], "dw_r": d_logits^T x [E,d]}, fp64."""
    x, w_r = np.ascontiguousarray(x), np.ascontiguousarray(w_r)
    d_logits = np.ascontiguousarray(d_logits, dtype=np.float64)
    T, d = x.shape
    E = w_r.shape[0]
    if x.dtype != w_r.dtype or w_r.shape[1] != d or d_logits.shape != (T, E):
        raise ValueError("router_bwd: shape or dtype mismatch")
    o = {"dx": np.empty((T, d)), "dw_r": np.empty((E, d))}
    _check(_load().orc_router_bwd(T, d, E, _DTYPE_CODE[x.dtype], x.ctypes.data, w_r.ctypes.data,
                                  d_logits.ctypes.data, o["dx"].ctypes.data,
                                  o["dw_r"].ctypes.data), "router_bwd")
    return o
