"""Move one layer's seeded inputs into device memory (torch tensors).

Small tensors (tokens, router, biases, projections) are drawn on the host and copied;
the expert stacks are filled on the device by the torch twin of the byte streams.
"""
from __future__ import annotations

import numpy as np

from . import LayerConfig, experts_torch, layer_inputs_np, tokens_np


def bf16_tensor(bits: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f32_tensor(a, device):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def layer_tensors(cfg: LayerConfig, device, seed: int = 0, inst: int = 0, batch: int = 0, experts=None,
                  shared=None):
    """(dict of device tensors, host LayerInputs).  Pass `experts` / `shared` to reuse stacks."""
    inp = layer_inputs_np(cfg, seed, inst, batch)
    d = dict(
        x=bf16_tensor(inp.x, device),
        w_router=bf16_tensor(inp.w_router, device),
        logit_bias=f32_tensor(inp.logit_bias, device),
        select_bias=f32_tensor(inp.select_bias, device),
        w_shared_gate=bf16_tensor(inp.w_shared_gate, device) if inp.w_shared_gate is not None else None,
        p_down=bf16_tensor(inp.p_down, device) if inp.p_down is not None else None,
        p_up=bf16_tensor(inp.p_up, device) if inp.p_up is not None else None,
    )
    d["experts"] = experts if experts is not None else experts_torch(cfg, device, seed, inst)
    if cfg.shared:
        d["shared"] = shared if shared is not None else experts_torch(cfg, device, seed, inst, shared=True)
    else:
        d["shared"] = None
    return d, inp


def token_batch(cfg: LayerConfig, device, seed: int = 0, inst: int = 0, batch: int = 0):
    return bf16_tensor(tokens_np(cfg, seed, inst, batch), device)
