"""The no-allocation routing entry point against the workspace form (GPU).

moe_route_permute_noalloc keeps its scratch in a static device array; two calls in a row
(the second smaller, so it reads scratch the first one left behind) must give exactly what
moe_route_permute gives with a caller workspace: the same kernels run on the same inputs.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import synth
from synth.device import bf16_tensor, f32_tensor

pytestmark = pytest.mark.gpu


def _args(cfg, dev, seed):
    inp = synth.layer_inputs_np(cfg, seed)
    wsg = inp.w_shared_gate if cfg.shared == "gated" else None
    return (bf16_tensor(inp.x, dev), bf16_tensor(inp.w_router, dev), cfg.k, cfg.score, cfg.renormalize,
            cfg.routed_scaling, f32_tensor(inp.logit_bias, dev), f32_tensor(inp.select_bias, dev),
            bf16_tensor(wsg, dev) if wsg is not None else None)


def test_route_permute_noalloc_matches_workspace_form():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mxfp4_routed_expert_amd as M
    dev = torch.device("cuda:0")
    decode = synth.get("qwen38max_decode")
    # first a 48-token batch (tiled router: logits and float64 partials in the scratch), then a
    # 3-token one (fused permutation), then a sigmoid-scored layer with a selection bias
    cases = [(dataclasses.replace(decode, T=48), 1), (dataclasses.replace(decode, T=3), 2),
             (dataclasses.replace(synth.get("glm52_fp8"), T=5), 3)]
    for cfg, seed in cases:
        a = _args(cfg, dev, seed)
        got = M.moe_route_permute_noalloc(*a)
        ref = M.moe_route_permute(*a)
        torch.cuda.synchronize()
        names = ["topk_ids", "topk_w", "shared_gate", "expert_offsets", "sorted_pairs", "pair_to_row"]
        for n, g, r in zip(names, got, ref):
            if r is None:
                assert g is None, n
                continue
            np.testing.assert_array_equal(g.cpu().numpy(), r.cpu().numpy(), err_msg=f"{cfg.name} T={cfg.T} {n}")
        print(f"  {cfg.name} T={cfg.T}: no-allocation call equals the workspace call", flush=True)
