"""GPU properties of whole layer steps: the library against itself.

  * two runs of one step give the same bits;
  * permuting the tokens of a step permutes its outputs, bit for bit: every output row
    is computed by the same instructions in the same order wherever its token sits in
    the batch (the K order of each product is fixed by the K-steps, the combine sums a
    token's slots in slot order);
  * a batch equals its tokens (or sub-batches) run as separate steps of the same path:
    routing bit for bit, outputs within float32 reassociation (a smaller batch can pick
    another split of the decode work, which reorders float32 sums);
  * an expert that no token selects changes nothing: overwriting its weights leaves the
    output bit for bit the same, while overwriting a selected expert changes it.

The cases cover the fused decode calls (three calls and the single launch), the decode GEMV
over FP8 weights, the per-slot GEMV in its wide form, the bf16 matrix-core prefill and the
FP4 matrix-core prefill.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_common import build, layer_weights, say, to_np

pytestmark = pytest.mark.gpu

REASSOC_REL_L2 = 2e-5      # float32 reassociation of the same sums in another order


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mxfp4_routed_expert_amd  # noqa: F401  (fails loudly when libmoe.so is missing)
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def M():
    import mxfp4_routed_expert_amd as m
    return m


def tiny(**kw):
    return dataclasses.replace(synth.get("tiny"), **kw)


# name -> (config, sub-batch size for "batched = token-by-token")
CASES = {
    # fused decode: router logits, gate/up with routing in its prologue, down-combine
    "decode_fused": (tiny(name="pd", wtag=110, T=4, k=3, E=16, shared="gated", shared_K=256, shared_I=128), 1),
    # the same decode step as one launch (moe_decode_step)
    "decode_single": (tiny(name="pd", wtag=110, T=4, k=3, E=16, shared="gated", shared_K=256, shared_I=128), 1),
    # decode GEMV over FP8 weights with sigmoid scoring, staged calls
    "decode_fp8": (tiny(name="pf", wtag=111, wfmt="fp8b128", score="sigmoid", select_bias_std=0.01, I=256, T=7, k=3,
                        E=24, shared="ungated", shared_K=256, shared_I=128), 1),
    # per-slot GEMV over FP8 weights in its wide form (8 token rows of 6 KB per chunk, two
    # chunks for experts with more rows), staged calls
    "mid_fp8_wide": (tiny(name="pw", wtag=114, wfmt="fp8b128", score="sigmoid", select_bias_std=0.01, T=40, H=3072,
                          I=512, E=64, k=4, shared="ungated", shared_K=3072, shared_I=256), 20),
    # bf16 matrix-core grouped GEMM (float activations)
    "prefill_float": (tiny(name="pp", wtag=112, T=192, H=512, I=160, E=256, k=2, shared="gated", shared_K=512,
                           shared_I=192), 64),
    # FP4 matrix-core grouped GEMM (MX activations)
    "prefill_mx": (tiny(name="pm", wtag=113, act="mxfp4", T=192, H=512, I=160, E=256, k=2, shared="gated",
                        shared_K=512, shared_I=192), 64),
}


SINGLE = {"decode_single"}                 # cases that run the single-launch decode step


def _layer(M, cfg, t, T, dev, name):
    layer = M.MoELayer(layer_weights(cfg, t), T, dev, single_launch=name in SINGLE)
    assert layer.single == (name in SINGLE and layer.fused)
    return layer


def _step(M, cfg, t, x, name):
    layer = _layer(M, cfg, t, x.shape[0], x.device, name)
    out = layer.forward(x).clone()
    torch.cuda.synchronize()
    return out, to_np(layer.ids), to_np(layer.topk_w)


@pytest.mark.parametrize("name", list(CASES))
def test_two_runs_give_the_same_bits(dev, M, name):
    cfg, _ = CASES[name]
    t, _ = build(cfg, dev)
    layer = _layer(M, cfg, t, cfg.T, dev, name)
    a = layer.forward(t["x"]).clone()
    b = layer.forward(t["x"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b), name


@pytest.mark.parametrize("name", list(CASES))
def test_token_permutation_permutes_outputs(dev, M, name):
    cfg, _ = CASES[name]
    t, _ = build(cfg, dev)
    perm = np.random.default_rng(7).permutation(cfg.T)
    pt = torch.from_numpy(perm).to(dev)
    out, ids, tw = _step(M, cfg, t, t["x"], name)
    out_p, ids_p, tw_p = _step(M, cfg, t, t["x"][pt].contiguous(), name)
    np.testing.assert_array_equal(ids_p, ids[perm])
    np.testing.assert_array_equal(tw_p, tw[perm])
    assert torch.equal(out_p, out[pt]), name


@pytest.mark.parametrize("name", list(CASES))
def test_batch_equals_its_parts(dev, M, name):
    cfg, part = CASES[name]
    t, _ = build(cfg, dev)
    out, ids, tw = _step(M, cfg, t, t["x"], name)
    outs, idss, tws = [], [], []
    for s in range(0, cfg.T, part):
        cs = dataclasses.replace(cfg, T=min(part, cfg.T - s))
        o, i, w = _step(M, cs, t, t["x"][s:s + part].contiguous(), name)
        outs.append(to_np(o))
        idss.append(i)
        tws.append(w)
    np.testing.assert_array_equal(np.concatenate(idss), ids)
    np.testing.assert_array_equal(np.concatenate(tws), tw)
    a, b = to_np(out).astype(np.float64), np.concatenate(outs).astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(a)
    say(f"  {name}: batch vs parts of {part}: rel_l2={rel:.3e} bit-equal={np.array_equal(a, b)}")
    assert rel <= REASSOC_REL_L2, (name, rel)


def _with_expert_overwritten(ex, e):
    """A copy of the expert stack with expert e's code bytes inverted and its scales changed."""
    c = {f.name: getattr(ex, f.name) for f in dataclasses.fields(ex)}
    for m in ("gate", "up", "down"):
        codes, sc = c[m].clone(), c[m + "_s"].clone()
        codes[e] = codes[e] ^ 0x77
        if sc.dtype == torch.uint8:
            sc[e] = sc[e] + 1
        else:
            sc[e] = sc[e] * 2
        c[m], c[m + "_s"] = codes, sc
    return type(ex)(**c)


@pytest.mark.parametrize("name", list(CASES))
def test_unrouted_expert_changes_nothing(dev, M, name):
    cfg, _ = CASES[name]
    t, _ = build(cfg, dev)
    out, ids, _ = _step(M, cfg, t, t["x"], name)
    used = set(ids.reshape(-1).tolist())
    idle = [e for e in range(cfg.E) if e not in used]
    assert idle, f"{name}: every expert is selected; the case needs more experts"
    t_idle = dict(t, experts=_with_expert_overwritten(t["experts"], idle[0]))
    out_idle, ids_idle, _ = _step(M, cfg, t_idle, t["x"], name)
    np.testing.assert_array_equal(ids_idle, ids)
    assert torch.equal(out_idle, out), name
    # control: the same overwrite of a selected expert does change the output
    t_used = dict(t, experts=_with_expert_overwritten(t["experts"], int(ids[0, 0])))
    out_used, _, _ = _step(M, cfg, t_used, t["x"], name)
    assert not torch.equal(out_used, out), name
