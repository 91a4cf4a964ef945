"""The five layer workloads (shapes, dtypes, input distributions).

Shapes and distributions are the five MoE layer instances the method is
measured on; where a workload leaves a value open the plain reading is taken:
weights and activations N(0, 0.02) (0.02 = standard deviation), router logits
N(0, 1), upstream gradient N(0, 1), LoRA scale s = alpha / r = 2 everywhere
(alpha = 2r, the ratio of the tiny workload), LoRA on gate, up and down.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int          # tokens
    d: int          # model width
    E: int          # experts
    k: int          # experts per token
    F: int          # expert FFN width
    r: int          # LoRA rank
    dtype: str      # 'f32' or 'bf16' storage of x, W, A, B, activations
    alpha: float    # LoRA alpha; s = alpha / r
    backward: bool = True
    router_grad: bool = False     # also d_topk_w and d_logits
    skew_bias: float = 0.0        # c in logits[t, e] += c * ln(1/(e+1))
    sigma_w: float = 0.02

    @property
    def S(self) -> int:
        return self.T * self.k

    @property
    def s(self) -> float:
        return self.alpha / self.r

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    def gemm_flops(self) -> dict:
        """Algorithmic GEMM flops of one pass (base W frozen; W+BA never formed)."""
        S, d, F, r = self.S, self.d, self.F, self.r
        fwd = S * (6 * d * F + 6 * r * (d + F))
        bwd = S * (6 * d * F + 12 * r * (d + F)) if self.backward else 0
        return {"fwd": fwd, "bwd": bwd, "total": fwd + bwd}


CONFIGS = {
    # tiny fp32 layer: fwd + bwd on the CPU in seconds
    "tiny_fp32": LayerConfig("tiny_fp32", T=256, d=128, E=8, k=2, F=256, r=8,
                             dtype="f32", alpha=16.0),
    # GPT-OSS-20B-shaped layer, forward only
    "gptoss20b": LayerConfig("gptoss20b", T=4096, d=2880, E=32, k=4, F=2880, r=16,
                             dtype="bf16", alpha=32.0, backward=False),
    # Qwen3-30B-A3B-shaped layer, forward + backward (the headline workload)
    "qwen3_30b_a3b": LayerConfig("qwen3_30b_a3b", T=8192, d=2048, E=128, k=8, F=768,
                                 r=16, dtype="bf16", alpha=32.0),
    # same shapes, Zipf-like skewed routing
    "qwen3_30b_a3b_skewed": LayerConfig("qwen3_30b_a3b_skewed", T=8192, d=2048, E=128,
                                        k=8, F=768, r=16, dtype="bf16", alpha=32.0,
                                        skew_bias=3.0),
    # GPT-OSS-120B-shaped layer, forward + backward + router-weight gradient
    "gptoss120b": LayerConfig("gptoss120b", T=16384, d=2880, E=128, k=4, F=2880, r=32,
                              dtype="bf16", alpha=64.0, router_grad=True),
}

HEADLINE = "qwen3_30b_a3b"


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]
