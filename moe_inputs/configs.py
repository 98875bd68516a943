"""Workload shapes for the mixture-of-experts feed-forward layer.

Each entry is a layer shape taken from the pages plus the seeded synthetic-value recipe
used to fill it.  Nothing here computes any part of the layer.

Shape sources (page title, where on the page):
  * Inkling (d = 6,144; 256 routed + 2 shared SwiGLU experts of intermediate 3,072; top-6;
    sigmoid router with a per-expert selection bias, weights normalized over the 8 active
    experts then x8): "Qwen3.8-2.4T-A95B vs Inkling", component table, residual-stream and
    router rows; "Inkling vs Gemma 4 31B", component table, routed-expert and
    shared-expert rows.
  * Qwen3.8-2.4T-A95B (hidden 8,192; 512 experts; moe_intermediate_size 2,048; top-10
    softmax renormalized; dtype bfloat16; initializer_range 0.02): "Qwen3.8 2.4T A95B"
    atlas page, key facts and raw config fields; "Qwen3.8-2.4T-A95B vs Inkling",
    component table, router row.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens in the batch
    d: int            # model width (d_model)
    E: int            # routed experts
    S: int            # shared (always-active) experts
    I: int            # expert intermediate size (d_ff)
    k: int            # routed experts kept per token
    router: str       # "softmax" (top-k, renormalized) or "sigmoid" (shared-expert sink)
    dtype: str        # "f32" or "bf16": x, router weight and expert weights
    x_std: float      # hidden-state std of the synthetic inputs
    w_std: float      # router / expert weight std (initializer_range)
    bias_std: float   # selection-bias std (sigmoid router only; 0 otherwise)
    zipf_s: float     # Zipf exponent of the per-expert logit offset (0: none)
    zipf_hot_share: float  # target share of assignments on the 8 hottest experts
    seed: int
    bias_on_logits: bool = False  # selection bias on the score (False) or on the logit
    prenorm: bool = False         # x is the raw hidden state; the layer input is RMSNorm(x)
    norm_zero_centred: bool = False  # RMSNorm scale is 1 + g (stored g) instead of g
    norm_eps: float = 1e-6
    weight_format: str = "dense"  # routed experts' weights: "dense" (dtype) or "mxfp4"

    @property
    def route_scale(self) -> float:
        """Multiplier after the joint normalization: the active-expert count k + S for the
        sigmoid router, 1 for softmax renormalization."""
        return float(self.k + self.S) if self.router == "sigmoid" else 1.0

    @property
    def router_rows(self) -> int:
        """Rows of the router weight: E + S for the sigmoid router (shared experts score
        too); E for the softmax router, whose shared experts are ungated."""
        return self.E + self.S if self.router == "sigmoid" else self.E

    @property
    def n_active(self) -> int:
        return self.k + self.S

    @property
    def rows(self) -> int:
        """Expert-input rows after grouping: k routed + S shared per token."""
        return self.T * (self.k + self.S)

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


_INKLING = dict(d=6144, E=256, S=2, I=3072, k=6, router="sigmoid", dtype="bf16",
                x_std=1.0, w_std=0.02, bias_std=0.1, zipf_s=0.0, zipf_hot_share=0.0)

CONFIGS: dict[str, MoEConfig] = {
    # Tiny fp32 layer: softmax top-2 of 16, everything ~N(0, 0.02^2).
    "tiny_fp32": MoEConfig(name="tiny_fp32", T=64, d=256, E=16, S=0, I=128, k=2,
                           router="softmax", dtype="f32", x_std=0.02, w_std=0.02,
                           bias_std=0.0, zipf_s=0.0, zipf_hot_share=0.0, seed=0),
    # Inkling-shaped layer, decode batch.
    "inkling_decode": MoEConfig(name="inkling_decode", T=32, seed=1, **_INKLING),
    # Inkling-shaped layer, prefill batch.
    "inkling_prefill": MoEConfig(name="inkling_prefill", T=8192, seed=2, **_INKLING),
    # Qwen3.8-shaped layer: softmax top-10 of 512, no shared expert.
    "qwen38": MoEConfig(name="qwen38", T=4096, d=8192, E=512, S=0, I=2048, k=10,
                        router="softmax", dtype="bf16", x_std=1.0, w_std=0.02,
                        bias_std=0.0, zipf_s=0.0, zipf_hot_share=0.0, seed=3),
    # Qwen3.8-shaped layer with its ungated shared expert (I = 2,048, weight 1).
    "qwen38_shared": MoEConfig(name="qwen38_shared", T=4096, d=8192, E=512, S=1, I=2048,
                               k=10, router="softmax", dtype="bf16", x_std=1.0,
                               w_std=0.02, bias_std=0.0, zipf_s=0.0, zipf_hot_share=0.0,
                               seed=5),
    # Inkling shape with a Zipf(1.2) per-expert logit offset: ~30% of assignments on
    # the 8 hottest experts.
    "inkling_skewed": MoEConfig(name="inkling_skewed", T=16384, seed=4,
                                **{**_INKLING, "zipf_s": 1.2, "zipf_hot_share": 0.30}),
    # Inkling decode batch with MXFP4 routed-expert weights (shared experts stay bf16).
    "inkling_decode_mxfp4": MoEConfig(name="inkling_decode_mxfp4", T=32, seed=7,
                                      weight_format="mxfp4", **_INKLING),
    # Kimi K3-style latent experts: sigmoid 16-of-896 in a 3,584-wide latent, RMSNorm
    # before the experts' up-projection (plain gains); I = 3,072 is a reading (the pages
    # give none; 2.8T parameters over 93 layers of 896 x 3 x 3,584 x I suggest ~3,100).
    "kimi_k3_latent": MoEConfig(name="kimi_k3_latent", T=8192, d=3584, E=896, S=0, I=3072,
                                k=16, router="sigmoid", dtype="bf16", x_std=1.0,
                                w_std=0.02, bias_std=0.1, zipf_s=0.0, zipf_hot_share=0.0,
                                seed=6, prenorm=True),
    # One GPU's share of the Inkling prefill layer under 8-way expert parallelism: the 32
    # routed experts it would own receive ~49,152 rows (8,192 tokens x 6 per GPU, spread
    # over 8 owners), plus the replicated shared experts on its own 8,192 tokens.  Routing
    # 8,192 local tokens over the 32 local experts gives the grouped GEMMs that shape.
    "inkling_ep8_share": MoEConfig(name="inkling_ep8_share", T=8192, seed=8,
                                   **{**_INKLING, "E": 32}),
}

# The order in which the five workloads are listed everywhere.
CONFIG_ORDER = ["tiny_fp32", "inkling_decode", "inkling_prefill", "qwen38", "inkling_skewed"]
# Workloads beyond the five above: Qwen3.8 with its ungated shared expert; Kimi K3-style
# latent experts behind a pre-norm RMSNorm; the Inkling decode batch with MXFP4 weights;
# one GPU's expert-parallel share of the Inkling prefill layer.
EXTRA_ORDER = ["qwen38_shared", "kimi_k3_latent", "inkling_decode_mxfp4", "inkling_ep8_share"]
