"""Pins for oracle.layer: brute force, library routines, closed forms and invariants.

A plausible slip in the oracle (a dropped term, a sign, a transposed operand, a wrong
index or tie rule) breaks at least one of these:
  * top-k against brute-force subset enumeration with constructed exact ties;
  * softmax weights against scipy.special.softmax; renormalised weights sum to 1;
  * sigmoid selection bias changes the selection only, never the weights;
  * router logits against exact integer arithmetic and the float32 rounding rule;
  * permutation against numpy's stable argsort;
  * the expert FFN against torch.nn.functional (linear, silu) on non-square shapes;
  * one-hot routing reduces the layer to one dense SwiGLU FFN; identical experts make the
    routed sum independent of routing; +1 on every down-scale byte doubles the output;
  * LatentMoE with identity projections equals the plain layer;
  * sizes against the numbers the pages print.
"""
import dataclasses
import itertools
import os

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import formats as F
from oracle import layer as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(v):
    return synth.to_bf16_bits(np.asarray(v, dtype=np.float64))


# ------------------------------------------------------------------ router + top-k

def _brute_topk(key_row, k):
    E = len(key_row)
    valid = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if not rest or min(key_row[list(S)]) >= max(key_row[rest]):
            valid.append(S)
    S = min(valid)                              # among equally valid sets, the lowest indices
    return sorted(S, key=lambda e: (-key_row[e], e))


def test_topk_bruteforce_random_and_ties():
    rng = np.random.default_rng(0)
    for trial in range(200):
        E = 8
        k = 2 + trial % 3
        key = rng.integers(-3, 4, E).astype(np.float64) if trial % 2 else rng.normal(size=E)
        got = L.topk_ids(key[None, :], k)[0]
        assert list(got) == _brute_topk(key, k), (key, k)


def test_router_logits_exact_and_rounded_once():
    # small integers: the dot product is an exact integer
    x = _bf16([[1, 2, -3, 4] + [0] * 28])
    W = _bf16([[5, -6, 7, 8] + [0] * 28, [1, 1, 1, 1] + [0] * 28])
    l = L.router_logits(x, W)
    assert l[0, 0] == 1 * 5 - 2 * 6 - 3 * 7 + 4 * 8 and l[0, 1] == 4
    # 1 + 2^-30 is not a float32: the logit is rounded once, to 1.0
    x = _bf16([[1.0, 2.0 ** -30]])
    W = _bf16([[1.0, 1.0]])
    assert L.router_logits(x, W)[0, 0] == 1.0
    # 1 + 3*2^-24 rounds to 1 + 2^-22 (nearest float32), not via two roundings
    x = _bf16([[1.0, 2.0 ** -23, 2.0 ** -24]])
    W = _bf16([[1.0, 1.0, 1.0]])
    assert L.router_logits(x, W)[0, 0] == np.float32(1 + 2.0 ** -22)
    # the logit bias is added after rounding
    assert L.router_logits(_bf16([[1.0]]), _bf16([[1.0]]), np.array([0.5], np.float32))[0, 0] == 1.5


def _rand_route_inputs(rng, T, H, E):
    x = _bf16(rng.normal(size=(T, H)))
    W = _bf16(0.05 * rng.normal(size=(E, H)))
    return x, W


def test_softmax_renormalised_matches_scipy_and_sums_to_one():
    rng = np.random.default_rng(1)
    x, W = _rand_route_inputs(rng, 5, 64, 16)
    r = L.route(x, W, 4)
    for t in range(5):
        sel = r.logits[t, r.ids[t]]
        np.testing.assert_allclose(r.weights[t], scipy.special.softmax(sel), rtol=1e-14)
        assert abs(r.weights[t].sum() - 1.0) < 1e-15
        assert (np.diff(sel) <= 0).all()          # descending order


def test_softmax_without_renorm_is_global_probability():
    rng = np.random.default_rng(2)
    x, W = _rand_route_inputs(rng, 3, 64, 16)
    r = L.route(x, W, 4, renormalize=False, routed_scaling=2.5)
    for t in range(3):
        p = scipy.special.softmax(r.logits[t])
        np.testing.assert_allclose(r.weights[t], 2.5 * p[r.ids[t]], rtol=1e-14)


def test_sigmoid_bias_affects_selection_only():
    rng = np.random.default_rng(3)
    x, W = _rand_route_inputs(rng, 6, 64, 16)
    r0 = L.route(x, W, 3, score="sigmoid")
    # without bias, the selection is the plain top-k of the logits (sigmoid is monotone)
    np.testing.assert_array_equal(r0.ids, L.topk_ids(r0.logits, 3))
    for t in range(6):
        s = scipy.special.expit(r0.logits[t, r0.ids[t]])
        np.testing.assert_allclose(r0.weights[t], s / s.sum(), rtol=1e-14)
    # a large bias on expert 5 forces it in; the weights are still sigmoid-of-logit ratios
    beta = np.zeros(16, np.float32)
    beta[5] = 10.0
    r1 = L.route(x, W, 3, score="sigmoid", select_bias=beta)
    assert (r1.ids[:, 0] == 5).all()
    for t in range(6):
        s = scipy.special.expit(r1.logits[t, r1.ids[t]])
        np.testing.assert_allclose(r1.weights[t], s / s.sum(), rtol=1e-14)
    # a bias that does not change the selection does not change the weights
    r2 = L.route(x, W, 3, score="sigmoid", select_bias=np.full(16, 0.25, np.float32))
    np.testing.assert_array_equal(r2.ids, r0.ids)
    np.testing.assert_array_equal(r2.weights, r0.weights)


def _golden_fields(name):
    d = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            key, *vals = line.split()
            d[key] = vals
    return d


def test_sigmoid_without_renorm_hand_case():
    """Sigmoid scoring, selection bias, no renormalisation, routed_scaling 2.5: the hand-worked
    case in tests/golden/sigmoid_no_renorm_case.txt.  Dividing by the selected sum, dropping
    routed_scaling, selecting without the bias or adding the bias to the weights all fail it."""
    g = _golden_fields("sigmoid_no_renorm_case.txt")
    logits = [float(v) for v in g["logits"]]
    E, H = len(logits), 32
    x = _bf16([[1.0] + [0.0] * (H - 1)])
    W = np.zeros((E, H))
    W[:, 0] = logits
    r = L.route(x, _bf16(W), int(g["k"][0]), score="sigmoid", renormalize=False,
                routed_scaling=float(g["routed_scaling"][0]), select_bias=np.array(g["beta"], np.float32))
    assert r.ids[0].tolist() == [int(v) for v in g["ids"]]
    np.testing.assert_allclose(r.weights[0], [float(v) for v in g["weights"]], rtol=1e-15)
    # with renormalisation the same selection gets the ratios (the two branches differ)
    r2 = L.route(x, _bf16(W), 3, score="sigmoid", renormalize=True, routed_scaling=2.5,
                 select_bias=np.array(g["beta"], np.float32))
    assert r2.ids[0].tolist() == r.ids[0].tolist()
    np.testing.assert_allclose(r2.weights[0], 2.5 * r.weights[0] / r.weights[0].sum(), rtol=1e-14)


def test_shared_gate_is_sigmoid_of_rounded_logit():
    rng = np.random.default_rng(4)
    x, W = _rand_route_inputs(rng, 3, 64, 8)
    wsg = _bf16(0.1 * rng.normal(size=64))
    r = L.route(x, W, 2, w_shared_gate_bits=wsg)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()
    wf = torch.from_numpy(wsg.view(np.int16)).view(torch.bfloat16).double()
    lg = (xf @ wf).float().double()
    np.testing.assert_allclose(r.shared_gate, torch.sigmoid(lg).numpy(), rtol=1e-15)


# ------------------------------------------------------------------ permutation

def test_permute_matches_stable_argsort():
    rng = np.random.default_rng(5)
    for T, k, E in [(1, 1, 1), (4, 2, 8), (33, 3, 5), (64, 8, 256)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
        p = L.permute(ids, E)
        flat = ids.reshape(-1)
        np.testing.assert_array_equal(p.sorted_pairs, np.argsort(flat, kind="stable"))
        np.testing.assert_array_equal(p.expert_offsets, np.r_[0, np.cumsum(np.bincount(flat, minlength=E))])
        np.testing.assert_array_equal(p.sorted_pairs[p.pair_to_row], np.arange(T * k))
        for e in range(E):
            rows = p.sorted_pairs[p.expert_offsets[e]:p.expert_offsets[e + 1]]
            assert (flat[rows] == e).all()


# ------------------------------------------------------------------ expert FFN + combine

def test_silu_closed_forms():
    assert L.silu(np.float64(0.0)) == 0.0
    assert L.silu(np.float64(1.0)) == pytest.approx(1.0 / (1.0 + np.exp(-1.0)), rel=1e-16)
    assert L.silu(np.float64(-1000.0)) == 0.0 and L.silu(np.float64(1000.0)) == 1000.0
    v = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(L.silu(v), torch.nn.functional.silu(torch.from_numpy(v)).numpy(), rtol=1e-14,
                               atol=1e-300)


def _tiny_cfg(**kw):
    base = dict(name="t", tag=90, wtag=90, T=5, H=64, I=96, E=6, k=2)
    base.update(kw)
    return synth.LayerConfig(**base)


def _torch_ffn(a, G, U, D):
    import torch.nn.functional as Fn
    a, G, U, D = (torch.from_numpy(np.asarray(t, np.float64)) for t in (a, G, U, D))
    return Fn.linear(Fn.silu(Fn.linear(a, G)) * Fn.linear(a, U), D).numpy()


def test_ffn_matches_torch_functional_nonsquare():
    cfg = _tiny_cfg()
    es = synth.expert_np(cfg, 3)
    G, U, D = L.dequant_expert(es)
    assert G.shape == (96, 64) and D.shape == (64, 96)
    a = F.bf16_value(synth.tokens_np(cfg))
    np.testing.assert_allclose(L.ffn(a, G, U, D), _torch_ffn(a, G, U, D), rtol=1e-12, atol=1e-300)


def test_one_hot_routing_equals_dense_ffn():
    cfg = _tiny_cfg(k=1)
    inp = synth.layer_inputs_np(cfg)
    res = L.layer(cfg, inp, lambda e: synth.expert_np(cfg, e))
    x = F.bf16_value(inp.x)
    assert np.allclose(res.routing.weights, 1.0)
    for t in range(cfg.T):
        e = int(res.routing.ids[t, 0])
        G, U, D = L.dequant_expert(synth.expert_np(cfg, e))
        ref = _torch_ffn(x[t:t + 1], G, U, D)[0]
        np.testing.assert_allclose(res.out[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_identical_experts_make_routing_irrelevant():
    cfg = _tiny_cfg(k=3, E=5)
    inp = synth.layer_inputs_np(cfg)
    same = synth.expert_np(cfg, 0)
    res = L.layer(cfg, inp, lambda e: same)
    x = F.bf16_value(inp.x)
    ref = _torch_ffn(x, *L.dequant_expert(same))
    np.testing.assert_allclose(res.out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_single_expert_layer_is_dense_ffn_plus_gated_shared():
    cfg = _tiny_cfg(E=1, k=1, shared="gated", shared_K=64, shared_I=32)
    inp = synth.layer_inputs_np(cfg)
    res = L.layer(cfg, inp, lambda e: synth.expert_np(cfg, e), lambda: synth.expert_np(cfg, synth.SHARED))
    x = F.bf16_value(inp.x)
    y0 = _torch_ffn(x, *L.dequant_expert(synth.expert_np(cfg, 0)))
    ys = _torch_ffn(x, *L.dequant_expert(synth.expert_np(cfg, synth.SHARED)))
    g = res.routing.shared_gate
    ref = y0 + g[:, None] * ys
    np.testing.assert_allclose(res.out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_down_scale_plus_one_doubles_output():
    cfg = _tiny_cfg()
    es = synth.expert_np(cfg, 1)
    a = F.bf16_value(synth.tokens_np(cfg))
    y = L.ffn(a, *L.dequant_expert(es))
    es2 = dataclasses.replace(es, down_s=es.down_s + 1)
    np.testing.assert_array_equal(L.ffn(a, *L.dequant_expert(es2)), 2 * y)


def test_combine_hand_example():
    y_rows = np.array([[1.0, 2.0], [3.0, 4.0]])
    out = L.combine(y_rows, np.array([1, 0]), np.array([[0.25, 0.75]]), 2,
                    y_shared=np.array([[10.0, 20.0]]), shared_gate=np.array([0.5]))
    np.testing.assert_array_equal(out, [[0.25 * 3 + 0.75 * 1 + 5.0, 0.25 * 4 + 0.75 * 2 + 10.0]])


@pytest.mark.parametrize("shared", ["ungated", "gated"])
def test_latent_identity_projection_equals_plain_layer(shared):
    plain = _tiny_cfg(k=2, shared=shared, shared_K=64, shared_I=32)
    lat = dataclasses.replace(plain, latent=64)
    inp = synth.layer_inputs_np(plain)
    eye = _bf16(np.eye(64))
    inp_l = dataclasses.replace(inp, p_down=eye, p_up=eye)
    ge = lambda e: synth.expert_np(plain, e)
    gs = lambda: synth.expert_np(plain, synth.SHARED)
    a = L.layer(plain, inp, ge, gs)
    b = L.layer(lat, inp_l, ge, gs)
    np.testing.assert_allclose(b.out, a.out, rtol=1e-13, atol=1e-13 * np.abs(a.out).max())


def test_mxfp4_activation_mode_quantises_both_operands():
    cfg = _tiny_cfg(act="mxfp4")
    es = synth.expert_np(cfg, 2)
    G, U, D = L.dequant_expert(es)
    a = F.bf16_value(synth.tokens_np(cfg))
    aq = F.mx_dequantize(*F.mx_quantize(a))
    h = L.silu(aq @ G.T) * (aq @ U.T)
    hq = F.mx_dequantize(*F.mx_quantize(h))
    ref = torch.nn.functional.linear(torch.from_numpy(hq), torch.from_numpy(D)).numpy()
    np.testing.assert_allclose(L.ffn(a, G, U, D, "mxfp4"), ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    # and the quantised activations are on the E2M1 grid times a power of two per block
    assert not np.array_equal(aq, a)


# ------------------------------------------------------------------ sizes the pages print

def _page_numbers():
    d = {}
    for line in open(os.path.join(GOLDEN, "page_sizes.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            d[k] = float(v)
    return d


def test_sizes_agree_with_pages():
    p = _page_numbers()
    cfg = synth.get("qwen38max_decode")
    per_expert = cfg.expert_bytes()
    assert per_expert == 3 * 7168 * 2368 * 17 // 32 == 27_052_032
    assert round(per_expert / 1e6) == p["expert_mb"]
    assert p["layers"] * p["experts_per_layer"] == p["experts_total"]
    assert cfg.E == p["experts_per_layer"] and cfg.k == p["topk"]
    # 46.3e9 routed params per token over 92 layers x top-10 -> params per expert; at
    # 17/32 byte per weight this reproduces the per-token read and the total expert bytes
    per_expert_params = p["routed_params_per_token"] / (p["layers"] * p["topk"])
    mb = per_expert_params * 17 / 32 / 1e6
    assert abs(mb - p["expert_mb"]) < 0.5
    assert abs(p["layers"] * p["topk"] * mb / 1e3 - p["per_token_gb"]) < 0.05
    assert abs(p["experts_total"] * mb / 1e6 - p["experts_tb"]) < 0.01
    # the synthetic intermediate width keeps the same parameter count within 1.5 %
    assert abs(3 * 7168 * 2368 - per_expert_params) / per_expert_params < 0.015


# ------------------------------------------------------------------ group-limited selection

def _brute_groups(key_row, n_group, topk_group, score):
    """Kept groups by enumeration: a valid set's lowest score is at least the highest score
    outside it; among valid sets, the lowest group indices."""
    gs = len(key_row) // n_group
    g = np.where(np.isnan(key_row), -np.inf, key_row).reshape(n_group, gs)
    gscore = np.array([sorted(r)[-1] + (sorted(r)[-2] if score == "sigmoid" else 0.0) for r in g])
    valid = []
    for S in itertools.combinations(range(n_group), topk_group):
        rest = [x for x in range(n_group) if x not in S]
        if not rest or min(gscore[list(S)]) >= max(gscore[rest]):
            valid.append(S)
    return set(min(valid))


def test_group_limit_hand_cases():
    n = 0
    for line in open(os.path.join(GOLDEN, "group_routing_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        head, keys, want = (part.split() for part in line.split("|"))
        score, ng, tg, k = head[0], int(head[1]), int(head[2]), int(head[3])
        key = np.array([float(v) for v in keys])[None, :]
        got = L.topk_ids(L.group_limit(key, ng, tg, score), k)[0]
        assert list(got) == [int(v) for v in want], line
        n += 1
    assert n == 5


def test_group_limit_bruteforce():
    rng = np.random.default_rng(11)
    for trial in range(300):
        ng = [2, 4, 8][trial % 3]
        gs = 2 + trial % 3
        E = ng * gs
        tg = 1 + trial % ng
        k = 1 + trial % min(4, tg * gs)
        score = "sigmoid" if trial % 2 else "softmax"
        key = rng.integers(-3, 4, E).astype(np.float64) if trial % 4 < 2 else rng.normal(size=E)
        kept = _brute_groups(key, ng, tg, score)
        masked = np.array([key[e] if e // gs in kept else -np.inf for e in range(E)])
        got = L.topk_ids(L.group_limit(key[None, :], ng, tg, score), k)[0]
        assert list(got) == _brute_topk(masked, k), (key, ng, tg, k, score)
        assert all(e // gs in kept for e in got)


def test_group_limit_reduces_to_plain_selection():
    rng = np.random.default_rng(12)
    x, W = _rand_route_inputs(rng, 5, 64, 32)
    for score in ("softmax", "sigmoid"):
        r0 = L.route(x, W, 4, score=score)
        for ng, tg in ((1, 1), (4, 4), (8, 8)):
            r1 = L.route(x, W, 4, score=score, n_group=ng, topk_group=tg)
            np.testing.assert_array_equal(r1.ids, r0.ids)
            np.testing.assert_array_equal(r1.weights, r0.weights)
        # a limit changes the selection only through the groups, never the weight formula
        r2 = L.route(x, W, 4, score=score, n_group=8, topk_group=2)
        if score == "sigmoid":
            for t in range(5):
                s = scipy.special.expit(r2.logits[t, r2.ids[t]])
                np.testing.assert_allclose(r2.weights[t], s / s.sum(), rtol=1e-14)
