"""Workload table for the routed MoE layer: shapes and input distributions.

Each entry is a synthetic stand-in for one of the model layers the pages describe
(the real checkpoints are not available).  Only sizes and distributions live here;
nothing in this file computes any part of the layer.

Sources for the shapes (pages: "rabbit" README, "Ran Moonshot's 2.8T-parameter Kimi K3
on a GPU-less mini-PC"):
  * Qwen3.8-Max: softmax top-10 of 512 routed experts plus a gated shared expert,
    OCP MXFP4 experts of about 27 MB each (rabbit README, design section and the
    architecture table).  An intermediate width of 2368 at hidden 7168 gives
    3*7168*2368*17/32 = 27,052,032 bytes per expert.
  * Kimi K3: Stable LatentMoE, routed experts computed at a narrower latent width,
    896 experts per layer, MXFP4 (Kimi K3 article, architecture section and run log).
  * GLM-5.2: noaux_tc sigmoid routing, FP8 E4M3 with block scales, one shared expert
    (rabbit README architecture table; Kimi K3 article architecture table).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class LayerConfig:
    name: str
    tag: int            # stream tag for tokens / router / biases
    wtag: int           # stream tag for expert weights (shared between configs that reuse a layer)
    T: int              # tokens per step
    H: int              # hidden width (router input, layer output)
    I: int              # routed expert intermediate width
    E: int              # routed experts
    k: int              # experts per token
    score: str = "softmax"          # "softmax" | "sigmoid"
    renormalize: bool = True
    routed_scaling: float = 1.0
    wfmt: str = "mxfp4"             # "mxfp4" | "fp8b128"
    act: str = "float"              # "float" (W4A16 style) | "mxfp4" (both operands MX-quantised)
    latent: int | None = None       # latent width for the routed experts (LatentMoE), else None
    shared: str | None = None       # None | "gated" | "ungated"
    shared_K: int = 0               # shared expert input width (hidden)
    shared_I: int = 0               # shared expert intermediate width
    router_std: float = 0.02
    logit_bias: str | None = None   # None | "zipf1.1" | "hot10"
    select_bias_std: float = 0.0    # per-expert selection bias (sigmoid path), N(0, std^2)
    scale_lo: int = 119             # E8M0 scale bytes uniform in [scale_lo, scale_hi]  (2^-8 .. 2^-4)
    scale_hi: int = 123
    fp8_exp_lo: int = -8            # FP8 block scales 2^u, u uniform in [lo, hi]
    fp8_exp_hi: int = -4
    notes: str = field(default="", compare=False)

    @property
    def d_model(self) -> int:
        """Input width of the routed experts (the latent width for LatentMoE)."""
        return self.latent if self.latent else self.H

    @property
    def pairs(self) -> int:
        return self.T * self.k

    def expert_bytes(self, K: int | None = None, I: int | None = None) -> int:
        K = self.d_model if K is None else K
        I = self.I if I is None else I
        if self.wfmt == "mxfp4":
            return 3 * K * I * 17 // 32
        # FP8: one byte per weight + fp32 scale per 128x128 tile, for gate, up ([I][K]) and down ([K][I])
        return 3 * K * I + 3 * (K // 128) * (I // 128) * 4


CONFIGS: dict[str, LayerConfig] = {}


def _add(c: LayerConfig) -> None:
    CONFIGS[c.name] = c


# Small layer the oracle finishes in well under a second.
_add(LayerConfig(name="tiny", tag=0, wtag=0, T=4, H=256, I=128, E=8, k=2,
                 notes="hidden 256, intermediate 128, 8 experts, softmax top-2 renormalised, no shared expert"))
# Qwen3.8-Max-like decode layer: one token.
_add(LayerConfig(name="qwen38max_decode", tag=1, wtag=1, T=1, H=7168, I=2368, E=512, k=10,
                 shared="gated", shared_K=7168, shared_I=2368,
                 notes="512 experts, softmax top-10 renormalised, gated MXFP4 shared expert"))
# Kimi-K3-like LatentMoE decode layer: 4 tokens, routed experts at latent width 2048.
_add(LayerConfig(name="kimik3_latent_decode", tag=2, wtag=2, T=4, H=7168, I=2048, E=896, k=8,
                 latent=2048, shared="ungated", shared_K=7168, shared_I=2048,
                 notes="896 experts, softmax top-8 renormalised, bf16 latent projections, ungated MXFP4 shared expert"))
# Qwen3.8-Max-like prefill: 512 tokens through the decode layer's experts, Zipf-skewed routing.
_add(LayerConfig(name="qwen38max_prefill", tag=3, wtag=1, T=512, H=7168, I=2368, E=512, k=10,
                 act="mxfp4", shared="gated", shared_K=7168, shared_I=2368,
                 router_std=7168 ** -0.5, logit_bias="zipf1.1",
                 notes="512 tokens, router logits ~N(0,1) plus a Zipf(1.1) popularity bias, MX-quantised activations"))
# Compute-bound slice of the prefill: every token routed to the same 10 experts.
_add(LayerConfig(name="qwen38max_prefill_hot", tag=4, wtag=1, T=512, H=7168, I=2368, E=512, k=10,
                 act="mxfp4", shared="gated", shared_K=7168, shared_I=2368,
                 router_std=7168 ** -0.5, logit_bias="hot10",
                 notes="as the prefill, with a +100 logit bias on 10 fixed experts (512 tokens per expert)"))
# The Zipf prefill with unquantised bf16 activations (weight-only quantisation).
_add(LayerConfig(name="qwen38max_prefill_float", tag=3, wtag=1, T=512, H=7168, I=2368, E=512, k=10,
                 act="float", shared="gated", shared_K=7168, shared_I=2368,
                 router_std=7168 ** -0.5, logit_bias="zipf1.1",
                 notes="as the prefill, with bf16 activations and float32 h (MXFP4 weights only)"))
# The hot prefill with unquantised bf16 activations (weight-only quantisation): the same
# tokens, routing and experts, the products on the bf16 matrix cores.
_add(LayerConfig(name="qwen38max_prefill_hot_float", tag=4, wtag=1, T=512, H=7168, I=2368, E=512, k=10,
                 act="float", shared="gated", shared_K=7168, shared_I=2368,
                 router_std=7168 ** -0.5, logit_bias="hot10",
                 notes="as the hot prefill, with bf16 activations and float32 h (MXFP4 weights only)"))
# GLM-5.2-like block-FP8 layer.
_add(LayerConfig(name="glm52_fp8", tag=5, wtag=5, T=64, H=6144, I=2048, E=256, k=8,
                 score="sigmoid", wfmt="fp8b128", shared="ungated", shared_K=6144, shared_I=2048,
                 select_bias_std=0.01,
                 notes="256 FP8 E4M3 experts with 128x128 fp32 block scales, noaux_tc sigmoid + selection bias, top-8"))


def get(name: str) -> LayerConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
