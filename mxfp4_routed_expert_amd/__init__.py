"""Routed MoE FFN over block-quantised (OCP MXFP4 / FP8 block-128) experts on MI355X.

The compute lives in the HIP library libmoe.so (C ABI in include/moe.h); `binding`
exposes each entry point with the same name, `layer` composes one layer step.
"""
from . import binding  # noqa: F401  (raises ImportError when the library is not built)
from .binding import (ExpertWeights, MoeError, decode_step_sync, moe_combine, moe_dense_bf16, moe_dequant, moe_dequant_bf16,  # noqa: F401
                      moe_decode_step, moe_expert_down, moe_expert_down_combine, moe_expert_ffn, moe_expert_gateup,
                      moe_expert_gateup_shared, moe_mx_quantize, moe_permute, moe_route, moe_route_permute,
                      moe_route_permute_noalloc, moe_router_logits, moe_topk_gateup_shared)
from .layer import LayerWeights, MoELayer  # noqa: F401
