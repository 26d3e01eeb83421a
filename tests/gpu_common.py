"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from synth import device as sdev

REL_L2 = 1e-4          # relative L2 error bound for float32 outputs
MAX_REL_RMS = 2e-3     # per-element bound, as a fraction of the reference RMS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(gpu, ref, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    nref = np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    diff = gpu - ref
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    mx = np.abs(diff).max() / rms if rms > 0 else np.abs(diff).max()
    say(f"  {what}: rel_l2={rel:.3e} max_err/rms={mx:.3e}")
    assert rel <= REL_L2, f"{what}: relative L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_REL_RMS, f"{what}: max error {mx:.3e} x RMS > {MAX_REL_RMS}"
    return rel, mx


def layer_weights(cfg, t):
    from mxfp4_routed_expert_amd import ExpertWeights, LayerWeights
    ex = ExpertWeights.from_arrays(t["experts"])
    sh = ExpertWeights.from_arrays(t["shared"]) if t["shared"] is not None else None
    return LayerWeights(score=cfg.score, k=cfg.k, renormalize=cfg.renormalize, routed_scaling=cfg.routed_scaling,
                        act=cfg.act, w_router=t["w_router"], experts=ex, logit_bias=t["logit_bias"],
                        select_bias=t["select_bias"], shared=sh,
                        w_shared_gate=t["w_shared_gate"] if cfg.shared == "gated" else None,
                        p_down=t["p_down"], p_up=t["p_up"])


_EXPERT_CACHE = {}


def device_experts(cfg, dev, seed=0, inst=0):
    """Expert stacks per (weight stream, instance), kept for the test session."""
    key = (cfg.wtag, cfg.wfmt, cfg.d_model, cfg.I, cfg.E, cfg.shared_K, cfg.shared_I, seed, inst)
    if key not in _EXPERT_CACHE:
        ex = synth.experts_torch(cfg, dev, seed, inst)
        sh = synth.experts_torch(cfg, dev, seed, inst, shared=True) if cfg.shared else None
        _EXPERT_CACHE[key] = (ex, sh)
    return _EXPERT_CACHE[key]


def build(cfg, dev, seed=0, inst=0, batch=0):
    ex, sh = device_experts(cfg, dev, seed, inst)
    t, inp = sdev.layer_tensors(cfg, dev, seed, inst, batch, experts=ex, shared=sh)
    return t, inp


def host_expert_getter(cfg, seed=0, inst=0):
    return (lambda e: synth.expert_np(cfg, e, seed, inst)), (lambda: synth.expert_np(cfg, synth.SHARED, seed, inst))


def to_np(t):
    return t.detach().cpu().numpy()
