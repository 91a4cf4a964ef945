"""Seeded synthetic inputs for the MoE expert layer.

A module of its own: it draws numbers and nothing else (no routing, no GEMM,
no activation). Both the CPU oracle's tests and the HIP library's tests and
benchmark take their inputs from here, so both sides see identical bytes.

The generator is counter-based (splitmix64 + Box-Muller, defined in
``synth.c``): value ``i`` of tensor ``tau`` depends only on (seed, tau, i),
so any prefix of a tensor (the first T' tokens, say) is the same whether the
whole tensor or only the prefix is drawn.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import CONFIGS, LayerConfig, get_config  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

# tensor ids of the counter-based generator
TENSOR_IDS = {
    "x": 0, "logits": 1, "w_gate": 2, "w_up": 3, "w_down": 4,
    "a_gate": 5, "b_gate": 6, "a_up": 7, "b_up": 8, "a_down": 9, "b_down": 10,
    "dout": 11, "w_router": 12, "d_logits": 13,
}


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
             os.path.join(_HERE, "synth.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, u32, i64, dbl, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.synth_normal_f32.argtypes = [u64, u32, dbl, vp, i64]
        lib.synth_normal_bf16.argtypes = [u64, u32, dbl, vp, i64]
        lib.synth_f32_to_bf16.argtypes = [vp, vp, i64]
        lib.synth_add_rank_bias.argtypes = [vp, i64, i64, dbl]
        for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_f32_to_bf16,
                  lib.synth_add_rank_bias):
            f.restype = None
        _lib = lib
    return _lib


def normal(seed: int, tensor: int, sigma: float, shape, dtype: str) -> np.ndarray:
    """N(0, sigma^2) draws of ``shape``; ``dtype`` 'f32' -> float32, 'bf16' -> uint16 bits."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        lib.synth_normal_f32(seed, tensor, sigma, out.ctypes.data, n)
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        lib.synth_normal_bf16(seed, tensor, sigma, out.ctypes.data, n)
    else:
        raise ValueError(dtype)
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even); returns the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def add_rank_bias(logits: np.ndarray, c: float) -> None:
    """In place: logits[t, e] += (float)(c * ln(1/(e+1))) in fp32."""
    assert logits.dtype == np.float32 and logits.flags.c_contiguous and logits.ndim == 2
    _load().synth_add_rank_bias(logits.ctypes.data, logits.shape[0], logits.shape[1], c)


def make_inputs(cfg: LayerConfig, seed: int = 0, tokens: int | None = None,
                with_dout: bool = True) -> dict:
    """All inputs of one layer instance, in storage format.

    x, W, A, B and dout are in the layer's dtype ('f32' -> float32, 'bf16' ->
    uint16 bf16 bits); logits are always float32. ``tokens`` draws only the
    first ``tokens`` rows of x / logits / dout (a prefix of the same tensors).
    """
    T = cfg.T if tokens is None else int(tokens)
    d, E, F, r, dt = cfg.d, cfg.E, cfg.F, cfg.r, cfg.dtype
    sw = cfg.sigma_w
    out = {
        "x": normal(seed, TENSOR_IDS["x"], sw, (T, d), dt),
        "logits": normal(seed, TENSOR_IDS["logits"], 1.0, (T, E), "f32"),
        "w_gate": normal(seed, TENSOR_IDS["w_gate"], sw, (E, F, d), dt),
        "w_up": normal(seed, TENSOR_IDS["w_up"], sw, (E, F, d), dt),
        "w_down": normal(seed, TENSOR_IDS["w_down"], sw, (E, d, F), dt),
        "a_gate": normal(seed, TENSOR_IDS["a_gate"], sw, (E, r, d), dt),
        "b_gate": normal(seed, TENSOR_IDS["b_gate"], sw, (E, F, r), dt),
        "a_up": normal(seed, TENSOR_IDS["a_up"], sw, (E, r, d), dt),
        "b_up": normal(seed, TENSOR_IDS["b_up"], sw, (E, F, r), dt),
        "a_down": normal(seed, TENSOR_IDS["a_down"], sw, (E, r, F), dt),
        "b_down": normal(seed, TENSOR_IDS["b_down"], sw, (E, d, r), dt),
    }
    if cfg.skew_bias:
        add_rank_bias(out["logits"], cfg.skew_bias)
    if with_dout:
        out["dout"] = normal(seed, TENSOR_IDS["dout"], 1.0, (T, d), dt)
    return out


def make_router(cfg: LayerConfig, seed: int = 0, tokens: int | None = None) -> dict:
    """Inputs of the router projection in front of the layer: w_router [E,d]
    in the layer's dtype, with sigma 1 / (sigma_w sqrt(d)) so that x W_r^T has
    unit variance like the workloads' N(0,1) logits; and a logit gradient
    d_logits [T,E] float32 ~ N(0,1) for the backward on its own."""
    T = cfg.T if tokens is None else int(tokens)
    sr = 1.0 / (cfg.sigma_w * float(np.sqrt(cfg.d)))
    return {"w_router": normal(seed, TENSOR_IDS["w_router"], sr, (cfg.E, cfg.d), cfg.dtype),
            "d_logits": normal(seed, TENSOR_IDS["d_logits"], 1.0, (T, cfg.E), "f32")}


def make_nf4(rows: int, cols: int, seed: int = 0, tensor: int = 20, sigma: float = 0.02) -> dict:
    """A 4-bit NormalFloat weight [rows, cols] (cols a multiple of 64) as stored:
    uniform random codes packed two per byte ({"codes": [rows, cols/2] uint8})
    and one positive scale per 64 weights ({"scales": [rows, cols/64] float32})
    drawn as sigma * 1.9 * (0.5 + u), u uniform in [0, 1), so the weights'
    standard deviation is about sigma (uniform codes give level RMS ~ 0.53)."""
    rng = np.random.default_rng([seed, tensor])
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = (sigma * 1.9 * (0.5 + rng.random((rows, cols // 64)))).astype(np.float32)
    return {"codes": codes, "scales": scales}


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a stored tensor (float32, or bf16 bits) to float64."""
    if dtype == "bf16" and a.dtype == np.uint16:
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)
