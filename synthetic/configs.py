"""The five layer workloads, in the pages' notation.

T tokens, d_model, E_r routed experts, K picks per token, E_s shared experts,
d_ffn (expert hidden width), router score function, bias recipe and bias step
gamma.  Sizes follow the Mixtral-8x7B and DeepSeek-V3 shapes that the pages
describe (Mixture of Experts designs page, section on expert granularity;
Sparse MoE routing-math page, section 6 comparison table).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    index: int            # stable small integer used in the token seed keys
    T: int
    d_model: int
    E_r: int
    K: int
    E_s: int
    d_ffn: int
    dtype: str            # "f32" or "bf16": tokens, weights and outputs
    score: str            # "sigmoid" or "softmax"
    bias: str             # "none" (no bias), "zero" (b = 0), "uniform" (b ~ U(-r, r))
    bias_range: float = 0.0
    gamma: float = 0.0    # bias step used by the training-style configs
    steps: int = 1        # forward + count + update steps (skewed config: 20)
    mixture: int = 0      # >0: tokens from a Gaussian mixture with this many components
    mixture_scale: float = 4.0
    hot_experts: int = 0  # experts whose centroids are aligned with mixture components
    layer_index: int = -1  # seed index of the layer's parameters (-1: same as index)

    @property
    def param_index(self) -> int:
        return self.index if self.layer_index < 0 else self.layer_index

    @property
    def rows(self) -> int:
        return self.T * self.K

    def with_tokens(self, T: int) -> "LayerConfig":
        return replace(self, T=T)

    def weight_bytes(self) -> int:
        per = 3 * self.d_model * self.d_ffn * (4 if self.dtype == "f32" else 2)
        return per * (self.E_r + self.E_s)


CONFIGS = {
    # Tiny fp32 layer: sigmoid router, b = 0 then one update with gamma = 0.1.
    "tiny_fp32": LayerConfig("tiny_fp32", 0, T=64, d_model=128, E_r=8, K=2, E_s=0,
                             d_ffn=256, dtype="f32", score="sigmoid", bias="zero",
                             gamma=0.1),
    # Mixtral-8x7B shape: softmax top-2, no bias.
    "mixtral_8x7b": LayerConfig("mixtral_8x7b", 1, T=4096, d_model=4096, E_r=8, K=2,
                                E_s=0, d_ffn=14336, dtype="bf16", score="softmax",
                                bias="none"),
    # DeepSeek-V3 prefill shape: sigmoid, b ~ U(-0.01, 0.01) for selection only.
    "dsv3_prefill": LayerConfig("dsv3_prefill", 2, T=4096, d_model=7168, E_r=256, K=8,
                                E_s=1, d_ffn=2048, dtype="bf16", score="sigmoid",
                                bias="uniform", bias_range=0.01, gamma=0.001),
    # Decode-sized batch through the same DeepSeek-V3 layer (same parameters).
    "dsv3_decode": LayerConfig("dsv3_decode", 3, T=64, d_model=7168, E_r=256, K=8,
                               E_s=1, d_ffn=2048, dtype="bf16", score="sigmoid",
                               bias="uniform", bias_range=0.01, gamma=0.001,
                               layer_index=2),
    # Skewed-load training steps through the same DeepSeek-V3 expert weights:
    # 4-component mixture tokens, 8 hot experts, b0 = 0, gamma = 0.001, 20 steps.
    "dsv3_skewed": LayerConfig("dsv3_skewed", 4, T=16384, d_model=7168, E_r=256, K=8,
                               E_s=1, d_ffn=2048, dtype="bf16", score="sigmoid",
                               bias="zero", gamma=0.001, steps=20, mixture=4,
                               mixture_scale=4.0, hot_experts=8, layer_index=2),
}


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]
