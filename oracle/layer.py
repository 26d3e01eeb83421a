"""The routed MoE layer, step by step, in float64.

What the pages fix (all prior art, whole-model engines):
  * the layer keeps the dense part resident, picks routed experts per token and sums
    their outputs with routing weights, next to shared experts (rabbit README, design
    section; Kimi K3 article, "how it works" list);
  * routing schemes: "softmax top-10 of 512 + gated shared expert" (Qwen3.8-Max),
    "noaux_tc sigmoid" (GLM-5.2), Stable LatentMoE with routed experts at a narrower
    latent width (Kimi K3) (rabbit README architecture table; Kimi K3 article,
    architecture section and table);
  * the expert activation is listed for Kimi K3 as "SituAndMul" (rabbit README source
    tree; Kimi K3 article source tree), a garbled name read here as SiLU-and-multiply,
    i.e. a SwiGLU expert: h = silu(gate x) * (up x), y = down h.

Readings where the pages are silent (each is repeated at the function that uses it):
  * router logits are the float32 rounding of the exact dot product of bf16 x and bf16
    router rows; an optional float32 logit bias is then added (in float64);
  * top-k order is by descending key, ties to the lower expert index; the softmax path
    selects on the logits (softmax is monotone), the sigmoid path on sigmoid(l) + beta,
    where beta is used for selection only;
  * renormalisation divides each selected weight by the sum of the selected weights;
    the result is multiplied by routed_scaling;
  * the shared gate is sigmoid of the float32-rounded logit x . w_sg;
  * tokens are grouped by expert with a stable order (ascending pair index p = t*k + j
    within an expert);
  * the expert FFN is float64 throughout (the GPU accumulates in float32); in the
    MX-quantised activation mode, x and h are passed through the OCP MX quantiser;
  * combine sums the k routed rows in order j = 0..k-1, then adds the gated shared row.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import bf16_value, dequant, mx_dequantize, mx_quantize


def _f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def router_logits(x_bits, w_bits, logit_bias=None):
    """l[t,e] = RN_fp32(sum_h x[t,h] W[e,h]) (+ logit_bias[e] in float64).

    Products of two bf16 values are exact in float64 and the float64 sum is rounded once
    to float32, so the logits are the float32 rounding of the exact dot product up to a
    float64 rounding error far below a float32 unit.  Routing follows the rabbit README
    architecture table ("MoE routing" row)."""
    x = bf16_value(x_bits)
    W = bf16_value(w_bits)
    l = _f32(x @ W.T)
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, dtype=np.float32).astype(np.float64)[None, :]
    return l


def sigmoid(v):
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def topk_ids(key, k):
    """First k experts of each row ordered by (-key, expert index)."""
    key = np.asarray(key, dtype=np.float64)
    T, E = key.shape
    ids = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-key[t, e], e))
        ids[t] = order[:k]
    return ids


@dataclass
class Routing:
    logits: np.ndarray        # [T][E] float64 (float32 values plus the optional bias)
    ids: np.ndarray           # [T][k] int64
    weights: np.ndarray       # [T][k] float64
    shared_gate: np.ndarray | None   # [T] float64


def group_limit(key, n_group, topk_group, score):
    """Group-limited selection ("grouped routing", Kimi Linear; noaux_tc: rabbit README,
    architecture table; the pages give no rule, the reading is the published noaux_tc one).
    Experts e are in group e // (E / n_group).  A group's score is the sum of its two
    largest keys (sigmoid) or its largest key (softmax); NaN keys count as -inf.  The
    topk_group best groups per token are kept, ties to the lower group; the keys of every
    other expert become -inf so that they are never selected."""
    key = np.array(key, dtype=np.float64)
    T, E = key.shape
    gs = E // n_group
    for t in range(T):
        kt = np.where(np.isnan(key[t]), -np.inf, key[t]).reshape(n_group, gs)
        best = np.sort(kt, axis=1)[:, ::-1]
        gscore = best[:, 0] + best[:, 1] if score == "sigmoid" else best[:, 0]
        order = sorted(range(n_group), key=lambda g: (-gscore[g], g))
        keep = set(order[:topk_group])
        for g in range(n_group):
            if g not in keep:
                key[t, g * gs:(g + 1) * gs] = -np.inf
    return key


def route(x_bits, w_router_bits, k, score="softmax", renormalize=True, routed_scaling=1.0,
          logit_bias=None, select_bias=None, w_shared_gate_bits=None, n_group=1, topk_group=1):
    """Scoring, top-k and renormalisation.

    softmax ("softmax top-10 of 512", rabbit README architecture table): select the k
    largest logits; weights are softmax probabilities of the selected experts, divided
    by their sum when renormalising (equal to a softmax over the selected logits).
    sigmoid ("noaux_tc sigmoid", same table): s = sigmoid(l); select on s + beta with a
    per-expert bias beta used for selection only; weights s_j, divided by their sum when
    renormalising.  Weights are then multiplied by routed_scaling.  The gated shared
    expert ("gated shared expert", same table) gets weight sigmoid(x . w_sg).  With
    n_group > 1 the selection is group-limited first (group_limit)."""
    l = router_logits(x_bits, w_router_bits, logit_bias)
    T, E = l.shape
    if score == "softmax":
        key = l
    elif score == "sigmoid":
        s = sigmoid(l)
        key = s + (np.asarray(select_bias, np.float32).astype(np.float64)[None, :]
                   if select_bias is not None else 0.0)
    else:
        raise ValueError(score)
    if n_group > 1:
        key = group_limit(key, n_group, topk_group, score)
    ids = topk_ids(key, k)
    rows = np.arange(T)[:, None]
    if score == "softmax":
        if renormalize:
            sel = l[rows, ids]
            p = np.exp(sel - sel.max(axis=1, keepdims=True))
            w = p / p.sum(axis=1, keepdims=True)
        else:
            p = np.exp(l - l.max(axis=1, keepdims=True))
            w = (p / p.sum(axis=1, keepdims=True))[rows, ids]
    else:
        sel = sigmoid(l[rows, ids])
        w = sel / sel.sum(axis=1, keepdims=True) if renormalize else sel
    w = w * float(np.float32(routed_scaling))
    g = None
    if w_shared_gate_bits is not None:
        g = sigmoid(router_logits(x_bits, np.asarray(w_shared_gate_bits)[None, :])[:, 0])
    return Routing(l, ids, w, g)


@dataclass
class Permutation:
    expert_offsets: np.ndarray   # [E+1]
    sorted_pairs: np.ndarray     # [T*k], pair p = t*k + j, grouped by expert, ascending p within
    pair_to_row: np.ndarray      # [T*k], inverse of sorted_pairs


def permute(ids, E):
    """Group the T*k (token, slot) pairs by expert: a stable sort on the expert id.

    The pages process experts one at a time as their bytes arrive (rabbit README,
    features list, per-expert early drain) and run a step's routed experts as one launch
    (Rulith Inference README, engine section); both need tokens grouped per expert."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = flat.size
    order = sorted(range(P), key=lambda p: (int(flat[p]), p))
    counts = np.bincount(flat, minlength=E) if P else np.zeros(E, np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    sorted_pairs = np.asarray(order, dtype=np.int64)
    pair_to_row = np.empty(P, dtype=np.int64)
    pair_to_row[sorted_pairs] = np.arange(P)
    return Permutation(offsets, sorted_pairs, pair_to_row)


def silu(g):
    """silu(g) = g / (1 + exp(-g)), evaluated in the form that stays finite for large |g|."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def ffn(a, G, U, D, act="float"):
    """One SwiGLU expert on activation rows a [M][K] (float64) with dequantised G, U [I][K], D [K][I].

    act == "mxfp4": a and h are passed through the OCP MX quantiser first (both operands
    of a block-scaled FP4 product are MX-encoded)."""
    if act == "mxfp4":
        a = mx_dequantize(*mx_quantize(a))
    g = a @ G.T
    u = a @ U.T
    h = silu(g) * u
    if act == "mxfp4":
        h = mx_dequantize(*mx_quantize(h))
    return h @ D.T


def dequant_expert(es, i=0):
    """(G, U, D) float64 for the i-th expert of a synth.ExpertSet."""
    return (dequant(es.fmt, es.gate[i], es.gate_s[i]), dequant(es.fmt, es.up[i], es.up_s[i]),
            dequant(es.fmt, es.down[i], es.down_s[i]))


def expert_rows(get_expert, a, perm, k, act="float", E=None):
    """y_rows [T*k][d_out]: row r is expert e's FFN of token sorted_pairs[r] // k.

    get_expert(e) returns a synth.ExpertSet holding expert e (index 0)."""
    offs = perm.expert_offsets
    E = len(offs) - 1 if E is None else E
    P = len(perm.sorted_pairs)
    y = None
    for e in range(E):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r0 == r1:
            continue
        G, U, D = dequant_expert(get_expert(e))
        toks = perm.sorted_pairs[r0:r1] // k
        ye = ffn(a[toks], G, U, D, act)
        if y is None:
            y = np.zeros((P, ye.shape[1]))
        y[r0:r1] = ye
    return y


def combine(y_rows, pair_to_row, weights, k, y_shared=None, shared_gate=None):
    """out[t] = sum_{j<k} w[t,j] * y_rows[pair_to_row[t*k+j]]  (+ g[t] * y_shared[t]).

    The weighted sum of routed expert outputs plus the shared expert (rabbit README,
    design section).  An ungated shared expert has weight 1."""
    T = weights.shape[0]
    d = y_rows.shape[1] if y_rows is not None else y_shared.shape[1]
    out = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            out[t] += weights[t, j] * y_rows[pair_to_row[t * k + j]]
        if y_shared is not None:
            out[t] += (1.0 if shared_gate is None else shared_gate[t]) * y_shared[t]
    return out


def dense_bf16(a, w_bits):
    """a [T][K] float64 times a bf16 weight [N][K]: a @ W^T (LatentMoE projections)."""
    return a @ bf16_value(w_bits).T


@dataclass
class LayerResult:
    routing: Routing
    perm: Permutation
    x_expert: np.ndarray        # activations the routed experts read ([T][d_model])
    y_rows: np.ndarray          # [T*k][d_model]
    y_shared: np.ndarray | None  # [T][H]
    z: np.ndarray               # routed sum (latent width for LatentMoE)
    out: np.ndarray             # [T][H]


def layer(cfg, inp, get_expert, get_shared=None):
    """One routed MoE layer step in float64.

    cfg: synth.LayerConfig; inp: synth.LayerInputs; get_expert(e) / get_shared() return
    synth.ExpertSet objects.  LatentMoE (Kimi K3 article, architecture section: routed
    experts compute in a narrower latent width): the router reads the full-width x,
    the routed experts read x_lat = P_d x, their weighted sum z is projected back with
    P_u, and the full-width shared expert's output, times its gate when it has one, is
    added after that."""
    x = bf16_value(inp.x)
    r = route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling,
              inp.logit_bias, inp.select_bias, inp.w_shared_gate if cfg.shared == "gated" else None)
    perm = permute(r.ids, cfg.E)
    xe = dense_bf16(x, inp.p_down) if cfg.latent else x
    y_rows = expert_rows(get_expert, xe, perm, cfg.k, cfg.act, cfg.E)
    y_s = None
    if cfg.shared:
        G, U, D = dequant_expert(get_shared())
        y_s = ffn(x, G, U, D, cfg.act)
    if cfg.latent:
        z = combine(y_rows, perm.pair_to_row, r.weights, cfg.k)
        out = dense_bf16(z, inp.p_up)
        if y_s is not None:
            out = out + (1.0 if r.shared_gate is None else r.shared_gate[:, None]) * y_s
    else:
        z = combine(y_rows, perm.pair_to_row, r.weights, cfg.k, y_s, r.shared_gate)
        out = z
    return LayerResult(r, perm, xe, y_rows, y_s, z, out)
