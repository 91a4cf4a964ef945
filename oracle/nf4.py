"""4-bit NormalFloat (NF4) frozen base weights: the codebook and the
dequantisation, in fp64.

TEST INFRASTRUCTURE ONLY (like the rest of this package): imported by the
test suite and the benchmark, never by the library.

The pages name 4-bit QLoRA as the frozen-base variant of MoE fine-tuning
(Unsloth 2026 wiki chapter, model-support table) and QLoRA's NF4 code (GPU
MODE lecture 32 notes, closing open questions) without giving the format. The reading taken is the NormalFloat
code of the QLoRA paper (Dettmers et al., 2023, section 3): 16 levels that
are quantiles of N(0, 1), built asymmetrically so that zero is exact, and
scaled into [-1, 1]; each block of 64 consecutive weights along a row has
its own positive scale (the block's absolute maximum when quantising), and
a weight is level[code] * scale.

Levels (ascending, code q indexes them):
  q = 0 .. 6   : -Q(0.5 + j/7 * (p - 0.5)) / Q(p) for j = 7 .. 1
  q = 7        : 0
  q = 8 .. 15  : +Q(0.5 + j/8 * (p - 0.5)) / Q(p) for j = 1 .. 8
with Q the standard normal quantile, so level 0 is -1 and level 15 is +1.
The paper's text leaves the top probability p open; its appendix prints the
16 resulting values, and p = 0.9677083 (about 1 - (1/64 + 1/60), between the
half-bin offsets of 16 and of 15 bins) reproduces them to float32 rounding.
That p is used here, so weights quantised with the published code
dequantise unchanged.

Packing: codes [rows, cols/2] uint8, element 2i of a row in the low nibble of
byte i and element 2i+1 in the high nibble; scales [rows, cols/64] float32.
"""
from __future__ import annotations

import numpy as np
from scipy.stats import norm

P_TOP = 0.9677083
BLOCK = 64


def levels() -> np.ndarray:
    """The 16 NF4 levels in fp64, ascending."""
    qmax = norm.ppf(P_TOP)
    neg = [-norm.ppf(0.5 + j / 7.0 * (P_TOP - 0.5)) / qmax for j in range(7, 0, -1)]
    pos = [norm.ppf(0.5 + j / 8.0 * (P_TOP - 0.5)) / qmax for j in range(1, 9)]
    return np.array(neg + [0.0] + pos, dtype=np.float64)


def unpack_codes(codes: np.ndarray, cols: int) -> np.ndarray:
    """[rows, cols/2] uint8 -> [rows, cols] codes 0..15 (low nibble first)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], cols), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def dequant(codes: np.ndarray, scales: np.ndarray, cols: int) -> np.ndarray:
    """fp64 weights [rows, cols] = level[code] * scale of the element's block."""
    q = unpack_codes(codes, cols)
    s = np.repeat(np.asarray(scales, dtype=np.float64), BLOCK, axis=1)[:, :cols]
    return levels()[q] * s


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest, ties to even), returned as fp64 values: the
    storage precision the layer's GEMMs read the weights in."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)  # inputs here are exact in fp32 or rounded once
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)
