"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Bit-exact: decoded weights, MX-quantised activations, expert ids, the permutation.
Within tolerance (relative L2 <= 1e-4 and max error <= 2e-3 x RMS of the reference):
routing weights, shared gate, expert rows, layer outputs.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_common import assert_close, build, host_expert_getter, layer_weights, say, to_np
from synth.device import bf16_tensor, f32_tensor
from oracle import formats as OF
from oracle import layer as OL

pytestmark = pytest.mark.gpu


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


# ------------------------------------------------------------------ formats

def test_device_generator_matches_host(dev):
    for cfg in (tiny(), tiny(name="tfp8", wtag=77, wfmt="fp8b128", score="sigmoid", I=256, shared="ungated",
                             shared_K=256, shared_I=128)):
        es = synth.experts_torch(cfg, dev)
        for e in range(cfg.E):
            h = synth.expert_np(cfg, e)
            for n in ("gate", "gate_s", "up", "up_s", "down", "down_s"):
                np.testing.assert_array_equal(to_np(getattr(es, n)[e]), getattr(h, n)[0], err_msg=f"{cfg.name} {n}")
        if cfg.shared:
            s = synth.experts_torch(cfg, dev, shared=True)
            h = synth.expert_np(cfg, synth.SHARED)
            np.testing.assert_array_equal(to_np(s.down), h.down)


def _bits_equal(gpu_f32, ref_f64):
    ref = ref_f64.astype(np.float32)
    g = np.asarray(gpu_f32, np.float32)
    nan = np.isnan(ref)
    assert (np.isnan(g) == nan).all()
    np.testing.assert_array_equal(g[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_dequant_mxfp4_every_code_and_scale_bitexact(dev, M):
    # row b: scale byte b on each of its 16 blocks, code bytes 0..255 across the row
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)
    g = M.moe_dequant("mxfp4", torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
    _bits_equal(to_np(g), OF.dequant_mxfp4(codes, scales))


def test_dequant_bf16_product_decode_every_code_and_scale_bitexact(dev, M):
    """The scaled FP4 -> bf16 conversion that every matrix-core kernel multiplies, over all 16
    codes x 256 scale bytes, against the oracle's exact value rounded to bf16: E2M1(code) times a
    power of two is a bf16 value unless it leaves bf16's range, which only scale byte 254 with
    |value| >= 2 reaches (rounded to infinity); byte 255 is NaN."""
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)
    g = M.moe_dequant_bf16(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
    ref64 = OF.dequant_mxfp4(codes, scales)
    ref = torch.from_numpy(ref64).to(torch.bfloat16)
    finite = np.isfinite(ref.float().numpy())
    # the oracle values are bf16 values wherever bf16 holds them (no rounding happened)
    np.testing.assert_array_equal(ref.double().numpy()[finite], ref64[finite])
    gb, rb = g.cpu().view(torch.int16).numpy(), ref.view(torch.int16).numpy()
    nan = np.isnan(ref64)
    assert (np.isnan(g.cpu().float().numpy()) == nan).all()
    bad = np.argwhere((gb != rb) & ~nan)
    assert bad.size == 0, f"{len(bad)} values differ, first (scale byte, element): {bad[:8].tolist()}"


def test_dequant_fp8_every_code_bitexact(dev, M):
    r = np.arange(256)
    codes = ((r[:, None] + r[None, :]) % 256).astype(np.uint8)
    scales = np.array([[2.0 ** -6, 0.7], [3.0, 2.0 ** -20]], np.float32)
    g = M.moe_dequant("fp8b128", torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
    _bits_equal(to_np(g), OF.dequant_fp8_b128(codes, scales))


def _mx_rows():
    rng = np.random.default_rng(7)
    rows = [rng.normal(0, s, 256) for s in (1.0, 1e-3, 1e3, 1e-30, 1e30)]
    rows.append(np.zeros(256))
    r = rng.normal(size=256); r[5] = np.nan; rows.append(r)
    r = rng.normal(size=256); r[100] = np.inf; rows.append(r)
    # exact E2M1 midpoints at several scales
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    r = np.tile(np.concatenate([mids, -mids]), 16) * 2.0 ** -3
    rows.append(r)
    r = rng.normal(size=256); r[::32] = 1e-40; rows.append(r)     # float32 subnormals
    rows.append(np.full(256, 3e38))
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mx_quantize_bitexact(dev, M, dtype):
    v = _mx_rows()
    if dtype == "bf16":
        bits = synth.to_bf16_bits(v.astype(np.float64))
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        ref_in = OF.bf16_value(bits)
    else:
        x = torch.from_numpy(v).to(dev)
        ref_in = v.astype(np.float64)
    q, s = M.moe_mx_quantize(x)
    rq, rs = OF.mx_quantize(ref_in)
    np.testing.assert_array_equal(to_np(s), rs)
    np.testing.assert_array_equal(to_np(q), rq)


# ------------------------------------------------------------------ routing

ROUTE_CASES = {
    "tiny": (tiny(), 0),
    "tiny_sigmoid": (tiny(score="sigmoid", select_bias_std=0.01, k=3), 0),
    "decode_router": (synth.get("qwen38max_decode"), 0),
    "decode_router_16tok": (dataclasses.replace(synth.get("qwen38max_decode"), T=16), 0),
    "latent_router": (synth.get("kimik3_latent_decode"), 0),
    "prefill_router_zipf": (synth.get("qwen38max_prefill"), 0),
    "fp8_router_sigmoid": (synth.get("glm52_fp8"), 0),
    "tiny_no_renorm": (tiny(renormalize=False, routed_scaling=2.5), 0),
    "tiny_sigmoid_no_renorm": (tiny(score="sigmoid", select_bias_std=0.01, k=3, renormalize=False,
                                    routed_scaling=2.5), 0),
    # tiled float64 router (T >= 32, H a multiple of 512): ragged token and row tiles
    "tiled_ragged_gated": (tiny(name="rt", T=300, H=1024, E=200, k=6, shared="gated"), 3),
    "tiled_min_tokens": (tiny(name="rt32", T=32, H=512, E=130, k=4), 4),
}


@pytest.mark.parametrize("name", list(ROUTE_CASES))
def test_route_matches_oracle(dev, M, name):
    cfg, seed = ROUTE_CASES[name]
    inp = synth.layer_inputs_np(cfg, seed)
    wsg = inp.w_shared_gate if cfg.shared == "gated" else None
    ids, w, sg = M.moe_route(bf16_tensor(inp.x, dev), bf16_tensor(inp.w_router, dev), cfg.k, cfg.score,
                             cfg.renormalize, cfg.routed_scaling, f32_tensor(inp.logit_bias, dev),
                             f32_tensor(inp.select_bias, dev),
                             bf16_tensor(wsg, dev) if wsg is not None else None)
    r = OL.route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling, inp.logit_bias,
                 inp.select_bias, wsg)
    np.testing.assert_array_equal(to_np(ids), r.ids)
    assert_close(to_np(w), r.weights, f"{name} topk_w")
    if cfg.renormalize:
        np.testing.assert_allclose(to_np(w).astype(np.float64).sum(1), cfg.routed_scaling, rtol=cfg.k * 2.0 ** -23)
    if wsg is not None:
        assert_close(to_np(sg), r.shared_gate, f"{name} shared_gate")


def test_route_ties_and_zero_logits(dev, M):
    """Exact ties (identical router rows) and a zero row, through the route kernel and the
    gate/up prologue: ids as the oracle's (larger key first, a tie to the lower expert),
    softmax and sigmoid with a selection bias."""
    for score in ("softmax", "sigmoid"):
        cfg = tiny(name="tie", wtag=107, E=16, k=6, T=4, score=score, shared="gated", shared_K=256, shared_I=128,
                   select_bias_std=0.01 if score == "sigmoid" else 0.0)
        inp = synth.layer_inputs_np(cfg, 0)
        W = inp.w_router.copy()             # bf16 bits
        for r in (5, 9, 12):
            W[r] = W[2]                     # four experts with the same logit for every token
        W[7] = W[3]
        W[14] = 0                           # zero logits
        wsg = inp.w_shared_gate
        sbias = inp.select_bias if score == "sigmoid" else None
        x = bf16_tensor(inp.x, dev)
        wr = bf16_tensor(W, dev)
        sb = f32_tensor(sbias, dev) if sbias is not None else None
        ids, w, sg = M.moe_route(x, wr, cfg.k, score, True, 1.0, None, sb, bf16_tensor(wsg, dev))
        r = OL.route(inp.x, W, cfg.k, score, True, 1.0, None, sbias, wsg)
        np.testing.assert_array_equal(to_np(ids), r.ids, err_msg=score)
        assert_close(to_np(w), r.weights, f"ties {score} topk_w")
        if score == "softmax":
            tied = sum(len(set(row) & {2, 5, 9, 12}) >= 2 for row in r.ids.tolist())
            assert tied > 0, "the case must select tied experts"
        # the gate/up prologue's selection on the same logits
        t, _ = build(cfg, dev)
        lw = layer_weights(cfg, t)
        lg = M.moe_router_logits(x, wr, cfg.k, score, bf16_tensor(wsg, dev))
        got = M.moe_topk_gateup_shared(lg, x, cfg.k, lw.experts, lw.shared, score, True, 1.0, None, sb, True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(got[0]), r.ids, err_msg=f"{score} prologue")


GROUP_CASES = {
    # noaux_tc-like: sigmoid + selection bias, 256 experts in 8 groups, 4 kept, top-8
    "glm_groups_decode": (dataclasses.replace(synth.get("glm52_fp8"), T=3), 8, 4),
    "glm_groups_64tok": (synth.get("glm52_fp8"), 8, 4),
    # softmax with group maxima (grouped routing), 512 experts in 16 groups, 2 kept
    "qwen_groups_decode": (synth.get("qwen38max_decode"), 16, 2),
    "qwen_groups_tiled": (dataclasses.replace(synth.get("qwen38max_prefill"), T=40), 16, 3),
    # the kept groups hold exactly k experts: topk_group * group size == k
    "tiny_groups_exact": (tiny(score="sigmoid", select_bias_std=0.01, k=4), 4, 2),
}


@pytest.mark.parametrize("name", list(GROUP_CASES))
def test_group_limited_route_matches_oracle(dev, M, name):
    cfg, ng, tg = GROUP_CASES[name]
    inp = synth.layer_inputs_np(cfg, 5)
    wsg = inp.w_shared_gate if cfg.shared == "gated" else None
    args = (bf16_tensor(inp.x, dev), bf16_tensor(inp.w_router, dev), cfg.k, cfg.score, cfg.renormalize,
            cfg.routed_scaling, f32_tensor(inp.logit_bias, dev), f32_tensor(inp.select_bias, dev),
            bf16_tensor(wsg, dev) if wsg is not None else None)
    ids, w, sg = M.moe_route(*args, n_group=ng, topk_group=tg)
    r = OL.route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling, inp.logit_bias,
                 inp.select_bias, wsg, n_group=ng, topk_group=tg)
    np.testing.assert_array_equal(to_np(ids), r.ids)
    assert_close(to_np(w), r.weights, f"{name} topk_w")
    gs = cfg.E // ng
    assert max(len(set(row // gs)) for row in r.ids) <= tg
    # the fused entry point selects the same experts and places them the same way
    ids2, w2, _, offs, sp, p2r = M.moe_route_permute(*args, n_group=ng, topk_group=tg)
    np.testing.assert_array_equal(to_np(ids2), r.ids)
    np.testing.assert_array_equal(to_np(w2), to_np(w))
    ref = OL.permute(r.ids, cfg.E)
    np.testing.assert_array_equal(to_np(offs), ref.expert_offsets)
    np.testing.assert_array_equal(to_np(sp), ref.sorted_pairs)
    np.testing.assert_array_equal(to_np(p2r), ref.pair_to_row)
    # without the limit the selection differs somewhere (the cases are chosen so)
    r0 = OL.route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling, inp.logit_bias,
                  inp.select_bias, wsg)
    assert (r0.ids != r.ids).any()


# ------------------------------------------------------------------ permutation

@pytest.mark.parametrize("name", list(ROUTE_CASES))
def test_route_permute_equals_route_then_permute(dev, M, name):
    """The fused entry point (one launch fewer for T <= 4, T*k <= 64) gives exactly what the
    two calls give, and the oracle's permutation of the oracle's ids."""
    cfg, seed = ROUTE_CASES[name]
    inp = synth.layer_inputs_np(cfg, seed)
    wsg = inp.w_shared_gate if cfg.shared == "gated" else None
    args = (bf16_tensor(inp.x, dev), bf16_tensor(inp.w_router, dev), cfg.k, cfg.score, cfg.renormalize,
            cfg.routed_scaling, f32_tensor(inp.logit_bias, dev), f32_tensor(inp.select_bias, dev),
            bf16_tensor(wsg, dev) if wsg is not None else None)
    ids, w, sg, offs, sp, p2r = M.moe_route_permute(*args)
    ids2, w2, sg2 = M.moe_route(*args)
    offs2, sp2, p2r2 = M.moe_permute(ids2, cfg.E)
    for a, b in [(ids, ids2), (w, w2), (offs, offs2), (sp, sp2), (p2r, p2r2)]:
        np.testing.assert_array_equal(to_np(a), to_np(b))
    if sg is not None:
        np.testing.assert_array_equal(to_np(sg), to_np(sg2))
    r = OL.route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling, inp.logit_bias,
                 inp.select_bias, wsg)
    ref = OL.permute(r.ids, cfg.E)
    np.testing.assert_array_equal(to_np(offs), ref.expert_offsets)
    np.testing.assert_array_equal(to_np(sp), ref.sorted_pairs)
    np.testing.assert_array_equal(to_np(p2r), ref.pair_to_row)


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (1, 10, 512), (4, 2, 8), (64, 8, 256), (513, 10, 512),
                                   (2000, 16, 2048), (4, 8, 896), (7, 10, 512),
                                   (819, 10, 896), (820, 10, 64)])
def test_permute_matches_oracle(dev, M, T, k, E):
    rng = np.random.default_rng(T * 131 + k * 7 + E)
    # skewed choice so some experts are empty and some are hot
    p = rng.zipf(1.3, size=E * 4) % E
    ids = np.stack([rng.choice(E, k, replace=False, p=np.bincount(p, minlength=E) / len(p)) if E > k * 2
                    else rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    offs, sp, p2r = M.moe_permute(torch.from_numpy(ids).to(dev), E)
    ref = OL.permute(ids, E)
    np.testing.assert_array_equal(to_np(offs), ref.expert_offsets)
    np.testing.assert_array_equal(to_np(sp), ref.sorted_pairs)
    np.testing.assert_array_equal(to_np(p2r), ref.pair_to_row)


def test_permute_drops_out_of_range_ids(dev, M):
    ids = np.array([[0, 3], [-1, 1], [3, 7]], np.int32)        # -1 and 7 are outside [0, 4)
    offs, sp, p2r = M.moe_permute(torch.from_numpy(ids).to(dev), 4)
    assert to_np(offs).tolist() == [0, 1, 2, 2, 4]
    assert to_np(sp).tolist() == [0, 3, 1, 4, -1, -1]
    assert to_np(p2r).tolist() == [0, 2, -1, 1, 3, -1]


# ------------------------------------------------------------------ expert FFN

FFN_CASES = {
    "mxfp4_tiny": tiny(T=37),
    "mxfp4_ragged": tiny(name="rag", wtag=81, T=29, H=1024, I=416, E=6, k=3),
    "mxfp4_wide": tiny(name="wide", wtag=82, T=5, H=2368, I=7168 // 4, E=4, k=2),
    "fp8": tiny(name="f8", wtag=83, wfmt="fp8b128", T=19, H=384, I=256, E=5, k=2),
    # >= 64 tokens over MXFP4 weights take the bf16 matrix-core GEMM: K tails of one MX block
    # (544 = 8.5 x 64, 416 = 6.5 x 64), ragged 128-column tiles, experts over several row tiles
    "mxfp4_prefill_ragged": tiny(name="fg1", wtag=95, T=150, H=544, I=416, E=6, k=3),
    "mxfp4_prefill_multitile": tiny(name="fg2", wtag=96, T=300, H=256, I=160, E=2, k=1),
}


@pytest.mark.parametrize("name", list(FFN_CASES))
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_expert_ffn_float_matches_oracle(dev, M, name, xdt):
    cfg = FFN_CASES[name]
    t, inp = build(cfg, dev)
    r = OL.route(inp.x, inp.w_router, cfg.k)
    perm = OL.permute(r.ids, cfg.E)
    x = OF.bf16_value(inp.x)
    if xdt == "f32":
        # float32 activations that are not bf16 values
        x = (x * (1.0 + 2.0 ** -12)).astype(np.float32).astype(np.float64)
        xg = torch.from_numpy(x.astype(np.float32)).to(dev)
    else:
        xg = t["x"]
    w = layer_weights(cfg, t)
    y = M.moe_expert_ffn(w.experts, xg, "float", cfg.k, torch.from_numpy(perm.expert_offsets.astype(np.int32)).to(dev),
                         torch.from_numpy(perm.sorted_pairs.astype(np.int32)).to(dev))
    ge, _ = host_expert_getter(cfg)
    ref = OL.expert_rows(ge, x, perm, cfg.k)
    assert_close(to_np(y), ref, f"{name}/{xdt} y_rows")


@pytest.mark.parametrize("groups", [(8, 0, 0, 0), (5, 0, 3, 0)])
def test_expert_ffn_rows_beyond_register_tile(dev, M, groups):
    """A grouping in which an expert owns more rows than a decode launch's register tile of
    token rows (2 tokens, 4 pairs each: the launches hold up to 2 rows of an expert at once,
    so rows are taken in chunks).  Against the oracle on the same grouping."""
    cfg = tiny(name="rbt", wtag=102, T=2, k=4, E=4, H=256, I=128)
    t, inp = build(cfg, dev)
    counts = np.array(groups)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    sorted_pairs = np.arange(cfg.T * cfg.k, dtype=np.int64)
    perm = OL.Permutation(offsets, sorted_pairs, sorted_pairs.copy())
    w = layer_weights(cfg, t)
    y = M.moe_expert_ffn(w.experts, t["x"], "float", cfg.k, torch.from_numpy(offsets.astype(np.int32)).to(dev),
                         torch.from_numpy(sorted_pairs.astype(np.int32)).to(dev))
    ge, _ = host_expert_getter(cfg)
    ref = OL.expert_rows(ge, OF.bf16_value(inp.x), perm, cfg.k)
    assert_close(to_np(y), ref, f"groups {groups} y_rows")


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_expert_ffn_identity_form_prefill_float(dev, M, xdt):
    """The shared expert's form (NULL offsets, one expert) at a prefill size: the bf16
    matrix-core GEMM without the permutation, with a ragged row tile and K tail."""
    cfg = tiny(name="fid", wtag=99, T=130, H=544, I=416, E=4, k=2, shared="ungated", shared_K=544, shared_I=416)
    t, inp = build(cfg, dev)
    x = OF.bf16_value(inp.x)
    if xdt == "f32":
        x = (x * (1.0 + 2.0 ** -12)).astype(np.float32).astype(np.float64)
        xg = torch.from_numpy(x.astype(np.float32)).to(dev)
    else:
        xg = t["x"]
    w = layer_weights(cfg, t)
    y = M.moe_expert_ffn(w.shared, xg, "float", 1, None, None)
    _, gs = host_expert_getter(cfg)
    ref = OL.ffn(x, *OL.dequant_expert(gs()))
    assert_close(to_np(y), ref, f"identity form/{xdt} y")


def test_dense_bf16_matches_oracle(dev, M):
    rng = np.random.default_rng(11)
    T, n, kd = 5, 200, 448
    w = synth.to_bf16_bits(0.05 * rng.normal(size=(n, kd)))
    xb = synth.to_bf16_bits(rng.normal(size=(T, kd)))
    res = rng.normal(size=(T, n)).astype(np.float32)
    y1 = M.moe_dense_bf16(bf16_tensor(xb, dev), bf16_tensor(w, dev))
    assert_close(to_np(y1), OL.dense_bf16(OF.bf16_value(xb), w), "dense bf16 x")
    xf = rng.normal(size=(T, kd)).astype(np.float32)
    y2 = M.moe_dense_bf16(torch.from_numpy(xf).to(dev), bf16_tensor(w, dev), torch.from_numpy(res).to(dev))
    assert_close(to_np(y2), OL.dense_bf16(xf.astype(np.float64), w) + res, "dense f32 x + residual")


def test_combine_matches_oracle(dev, M):
    rng = np.random.default_rng(12)
    T, k, d = 7, 3, 260
    y_rows = rng.normal(size=(T * k, d)).astype(np.float32)
    p2r = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    ys = rng.normal(size=(T, d)).astype(np.float32)
    g = rng.random(T).astype(np.float32)
    tt = lambda a: torch.from_numpy(a).to(dev)
    out = M.moe_combine(tt(y_rows), tt(p2r), tt(w), tt(ys), tt(g))
    ref = OL.combine(y_rows.astype(np.float64), p2r, w.astype(np.float64), k, ys.astype(np.float64),
                     g.astype(np.float64))
    assert_close(to_np(out), ref, "combine")


# ------------------------------------------------------------------ whole layers, small

LAYER_CASES = {
    "tiny": tiny(),
    "tiny_gated_shared": tiny(name="tg", wtag=84, shared="gated", shared_K=256, shared_I=96),
    "tiny_sigmoid_fp8": tiny(name="tf", wtag=85, wfmt="fp8b128", score="sigmoid", select_bias_std=0.01,
                             I=256, T=9, k=3, shared="ungated", shared_K=256, shared_I=128),
    "tiny_latent": tiny(name="tl", wtag=86, latent=128, H=512, I=96, shared="ungated", shared_K=512,
                        shared_I=64),
    # LatentMoE with a gated shared expert: the gate scales the shared output added after P_u
    "tiny_latent_gated": tiny(name="tlg", wtag=89, latent=128, H=512, I=96, shared="gated", shared_K=512,
                              shared_I=64),
    # decode fusion (T <= 4, shared d_ff == d_ff): fused gate/up + down-combine calls
    "tiny_fused_gated": tiny(name="tfg", wtag=87, T=3, k=3, shared="gated", shared_K=256, shared_I=128),
    "tiny_fused_fp8_ungated": tiny(name="tff", wtag=88, wfmt="fp8b128", score="sigmoid", select_bias_std=0.01,
                                   I=256, T=2, k=4, shared="ungated", shared_K=256, shared_I=256),
    # an odd number of 32-value blocks per down row (the down-combine reads the two scale bytes
    # of a lane one by one)
    "tiny_fused_odd_blocks": tiny(name="tfo", wtag=101, T=2, k=2, I=96, shared="ungated", shared_K=256, shared_I=96),
    # FP8 with 40 tokens and 6 KB activation rows: the per-slot GEMV's wide form (8 rows of a
    # chunk in LDS, 512-thread workgroups), two chunks per routed expert, five for the shared
    "fp8_wide_chunks": tiny(name="fw", wtag=102, wfmt="fp8b128", score="sigmoid", select_bias_std=0.01, T=40,
                            H=3072, I=512, E=16, k=4, shared="ungated", shared_K=3072, shared_I=256),
    # prefill sizes on the bf16 matrix-core GEMM: the shared expert in the identity form, and
    # the latent form (float32 x_lat split into two bf16 terms)
    "prefill_gated_shared": tiny(name="pgs", wtag=97, T=160, H=512, I=160, E=8, k=2, shared="gated",
                                 shared_K=512, shared_I=192),
    "prefill_latent": tiny(name="plt", wtag=98, latent=128, H=512, I=96, T=96, shared="ungated", shared_K=512,
                           shared_I=64),
}


GRAPH_CASES = ["tiny_gated_shared", "tiny_fused_gated", "tiny_fused_gated/single", "tiny_latent",
               "tiny_sigmoid_fp8", "prefill_gated_shared"]


@pytest.mark.parametrize("name", GRAPH_CASES)
def test_graph_replays_match_eager(dev, M, name):
    """One layer step captured as a HIP graph (with the shared expert's second stream where the
    layer uses one; "/single": the single-launch decode step) and replayed three times over
    three inputs, with eager copies and synchronisations between the replays: every replay
    gives the eager output bit for bit."""
    cfg = LAYER_CASES[name.split("/")[0]]
    t, _ = build(cfg, dev)
    layer = M.MoELayer(layer_weights(cfg, t), cfg.T, dev, single_launch=name.endswith("/single"))
    if name.endswith("/single"):
        assert layer.single
    x0 = t["x"]
    xs = [x0, (x0.float() * 0.5).to(torch.bfloat16), x0.roll(1, dims=1).contiguous()]
    eager = [layer.forward(x).clone() for x in xs]
    torch.cuda.synchronize()
    x_static = x0.clone()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        layer.forward(x_static)
        st.synchronize()
        with torch.cuda.graph(g, stream=st):
            out = layer.forward(x_static)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, x in enumerate(xs):
            x_static.copy_(x)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager[i]), (name, rep, i)


def _run_layer(M, cfg, dev, seed=0, inst=0):
    t, inp = build(cfg, dev, seed, inst)
    layer = M.MoELayer(layer_weights(cfg, t), cfg.T, dev)
    out = layer.forward(t["x"])
    torch.cuda.synchronize()
    return layer, out, inp


@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_layer_matches_oracle(dev, M, name):
    cfg = LAYER_CASES[name]
    layer, out, inp = _run_layer(M, cfg, dev)
    ge, gs = host_expert_getter(cfg)
    ref = OL.layer(cfg, inp, ge, gs)
    np.testing.assert_array_equal(to_np(layer.ids), ref.routing.ids)
    np.testing.assert_array_equal(to_np(layer.sp), ref.perm.sorted_pairs)
    if layer.y_rows is not None:          # the down-combine calls never write y_rows
        assert_close(to_np(layer.y_rows), ref.y_rows, f"{name} y_rows")
    assert_close(to_np(out), ref.out, f"{name} out")


FUSED_CASES = ["tiny", "tiny_fused_gated", "tiny_fused_fp8_ungated", "tiny_fused_odd_blocks"]


@pytest.mark.parametrize("name", FUSED_CASES)
def test_fused_decode_calls_match_unfused(dev, M, name):
    """moe_expert_gateup_shared + moe_expert_down_combine against moe_expert_ffn (routed and
    shared) + moe_combine on the same routing: h rows equal, output within tolerance."""
    cfg = LAYER_CASES[name]
    layer, out, inp = _run_layer(M, cfg, dev)
    assert layer.fused
    w = layer.w
    t, _ = build(cfg, dev)
    x = t["x"]
    h, _, _ = M.moe_expert_gateup(w.experts, x, "float", w.k, layer.offs, layer.sp)
    assert_close(to_np(layer.h), to_np(h), f"{name} h")
    y = M.moe_expert_ffn(w.experts, x, "float", w.k, layer.offs, layer.sp)
    ys = M.moe_expert_ffn(w.shared, x, "float", 1, None, None) if w.shared is not None else None
    if w.shared is not None:
        hs, _, _ = M.moe_expert_gateup(w.shared, x, "float", 1, None, None)
        assert_close(to_np(layer.h_sh), to_np(hs), f"{name} shared h")
    ref = M.moe_combine(y, layer.p2r, layer.topk_w, ys, layer.sg)
    assert_close(to_np(out), to_np(ref), f"{name} out")


# routing in the gate/up launch (moe_router_logits + moe_topk_gateup_shared) against
# moe_route_permute + moe_expert_gateup_shared: (config, n_group, topk_group)
TOPK_GATEUP_CASES = {
    "tiny": (tiny(), 1, 1),
    "tiny_fused_gated": (LAYER_CASES["tiny_fused_gated"], 1, 1),
    "tiny_sigmoid_fp8": (LAYER_CASES["tiny_fused_fp8_ungated"], 1, 1),
    "tiny_groups": (tiny(name="tgk", wtag=103, score="sigmoid", select_bias_std=0.01, k=4, T=3, E=16,
                         shared="gated", shared_K=256, shared_I=128), 4, 2),
    "decode_full": (synth.get("qwen38max_decode"), 1, 1),
    # more experts than the in-launch selection holds: the route kernel selects first
    "tiny_many_experts": (tiny(name="tme", wtag=104, E=640, k=3, T=2, shared="gated", shared_K=256, shared_I=128),
                          1, 1),
}


@pytest.mark.parametrize("name", list(TOPK_GATEUP_CASES))
def test_topk_gateup_equals_route_then_gateup(dev, M, name):
    """The three-kernel decode step's first two calls give the routing, the permutation, h and
    h_shared of moe_route_permute followed by moe_expert_gateup_shared, bit for bit."""
    cfg, ng, tg = TOPK_GATEUP_CASES[name]
    t, inp = build(cfg, dev)
    w = layer_weights(cfg, t)
    x = t["x"]
    wsg = t["w_shared_gate"] if cfg.shared == "gated" else None
    ref = M.moe_route_permute(x, t["w_router"], cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling,
                              t["logit_bias"], t["select_bias"], wsg, n_group=ng, topk_group=tg)
    ids, tw, sg, offs, sp, p2r = ref
    h_ref, hs_ref = M.moe_expert_gateup_shared(w.experts, w.shared, x, cfg.k, offs, sp)
    lg = M.moe_router_logits(x, t["w_router"], cfg.k, cfg.score, wsg, n_group=ng, topk_group=tg)
    got = M.moe_topk_gateup_shared(lg, x, cfg.k, w.experts, w.shared, cfg.score, cfg.renormalize, cfg.routed_scaling,
                                   t["logit_bias"], t["select_bias"], wsg is not None, n_group=ng, topk_group=tg)
    torch.cuda.synchronize()
    names = ["topk_ids", "topk_w", "shared_gate", "expert_offsets", "sorted_pairs", "pair_to_row"]
    for nm, a, b in zip(names, got[:6], ref):
        if b is None:
            assert a is None, nm
            continue
        np.testing.assert_array_equal(to_np(a), to_np(b), err_msg=f"{name} {nm}")
    np.testing.assert_array_equal(to_np(got[6]), to_np(h_ref), err_msg=f"{name} h")
    if hs_ref is not None:
        np.testing.assert_array_equal(to_np(got[7]), to_np(hs_ref), err_msg=f"{name} h_shared")
    say(f"  {name}: routing, permutation, h equal")


# the single-launch decode step (moe_decode_step) against its three calls:
# (config, n_group, topk_group, whether the shapes take the single launch)
DECODE_STEP_CASES = {
    "tiny": (tiny(), 1, 1, True),
    "tiny_fused_gated": (LAYER_CASES["tiny_fused_gated"], 1, 1, True),
    "tiny_fused_odd_blocks": (LAYER_CASES["tiny_fused_odd_blocks"], 1, 1, True),
    "tiny_groups": (TOPK_GATEUP_CASES["tiny_groups"][0], 4, 2, True),
    "tiny_4tok_sigmoid": (tiny(name="t4s", wtag=105, score="sigmoid", select_bias_std=0.01, k=6, T=4, E=32,
                               shared="gated", shared_K=256, shared_I=128), 1, 1, True),
    "decode_full": (synth.get("qwen38max_decode"), 1, 1, True),
    # one expert per token; a layer of a single routed expert (every token selects it)
    "tiny_k1": (tiny(name="tk1", wtag=108, k=1, T=3, shared="ungated", shared_K=256, shared_I=128), 1, 1, True),
    "tiny_one_expert": (tiny(name="t1e", wtag=109, E=1, k=1, T=2, shared="gated", shared_K=256, shared_I=128),
                        1, 1, True),
    # shapes the single launch does not take run as the three calls
    "tiny_sigmoid_fp8": (LAYER_CASES["tiny_fused_fp8_ungated"], 1, 1, False),
    "tiny_many_experts": (TOPK_GATEUP_CASES["tiny_many_experts"][0], 1, 1, False),
    "tiny_6tok": (tiny(name="t6", wtag=106, T=6, shared="gated", shared_K=256, shared_I=128), 1, 1, False),
}


@pytest.mark.parametrize("name", list(DECODE_STEP_CASES))
def test_decode_step_equals_three_calls(dev, M, name):
    """moe_decode_step gives the logits, routing, permutation, h rows and output of
    moe_router_logits + moe_topk_gateup_shared + moe_expert_down_combine bit for bit, on three
    inputs in a row with one sync buffer; the buffer counts the single launches and its error
    word stays 0."""
    cfg, ng, tg, single = DECODE_STEP_CASES[name]
    t, inp = build(cfg, dev)
    w = layer_weights(cfg, t)
    wsg = t["w_shared_gate"] if cfg.shared == "gated" else None
    sync = M.decode_step_sync(dev)
    x0 = t["x"]
    xs = [x0, (x0.float() * 0.5).to(torch.bfloat16), x0.roll(1, dims=1).contiguous()]
    names = ["logits", "topk_ids", "topk_w", "shared_gate", "expert_offsets", "sorted_pairs", "pair_to_row", "h",
             "h_shared", "out"]
    for i, x in enumerate(xs):
        lg = M.moe_router_logits(x, t["w_router"], cfg.k, cfg.score, wsg, n_group=ng, topk_group=tg)
        r = M.moe_topk_gateup_shared(lg, x, cfg.k, w.experts, w.shared, cfg.score, cfg.renormalize,
                                     cfg.routed_scaling, t["logit_bias"], t["select_bias"], wsg is not None,
                                     n_group=ng, topk_group=tg)
        ids, tw, sg, offs, sp, p2r, h, hs = r
        o = M.moe_expert_down_combine(w.experts, w.shared, h, hs, ids, tw, p2r, sg)
        ref = (lg, ids, tw, sg, offs, sp, p2r, h, hs, o)
        got = M.moe_decode_step(x, t["w_router"], cfg.k, w.experts, w.shared, cfg.score, cfg.renormalize,
                                cfg.routed_scaling, t["logit_bias"], t["select_bias"], wsg, sync=sync, n_group=ng,
                                topk_group=tg)
        torch.cuda.synchronize()
        for nm, a, b in zip(names, got, ref):
            if b is None:
                assert a is None, nm
                continue
            np.testing.assert_array_equal(to_np(a), to_np(b), err_msg=f"{name} input {i} {nm}")
    sv = to_np(sync)
    assert sv[1] == 0, f"{name}: a hand-off wait gave up"
    assert sv[0] == (len(xs) if single else 0), (name, sv[0])
    say(f"  {name}: {'single launch' if single else 'three calls'}, every output equal")


def test_decode_step_layer_matches_oracle_after_other_steps(dev, M):
    """A decode layer whose sync buffer has served other layers' steps (the launch count is
    well past zero, with a different grid of experts in between) still matches the oracle."""
    cfg = LAYER_CASES["tiny_fused_gated"]
    other = DECODE_STEP_CASES["tiny_4tok_sigmoid"][0]
    t, inp = build(cfg, dev)
    t2, _ = build(other, dev)
    layer = M.MoELayer(layer_weights(cfg, t), cfg.T, dev, single_launch=True)
    layer2 = M.MoELayer(layer_weights(other, t2), other.T, dev, single_launch=True)
    assert layer.single and layer2.single
    layer2.sync = layer.sync                              # one stream, one sync buffer
    for _ in range(5):
        layer2.forward(t2["x"])
        layer.forward(t["x"])
    out = layer.forward(t["x"])
    torch.cuda.synchronize()
    ge, gs = host_expert_getter(cfg)
    ref = OL.layer(cfg, inp, ge, gs)
    np.testing.assert_array_equal(to_np(layer.ids), ref.routing.ids)
    assert_close(to_np(out), ref.out, "decode step after other steps")
    sv = to_np(layer.sync)
    assert sv[0] == 11 and sv[1] == 0, sv[:2]


def test_down_combine_drops_invalid_pairs(dev, M):
    """A pair with id -1 or row -1 adds nothing; the rest is the weighted sum."""
    cfg = LAYER_CASES["tiny_fused_gated"]
    layer, out, inp = _run_layer(M, cfg, dev)
    w = layer.w
    ids = layer.ids.clone()
    p2r = layer.p2r.clone()
    ids[0, 1] = -1                       # slot 1 of token 0 dropped by id
    p2r[1 * w.k + 2] = -1                # slot 2 of token 1 dropped by row
    o = M.moe_expert_down_combine(w.experts, w.shared, layer.h, layer.h_sh, ids, layer.topk_w, p2r, layer.sg)
    tw = layer.topk_w.clone()
    tw[0, 1] = 0.0
    tw[1, 2] = 0.0
    ref = M.moe_expert_down_combine(w.experts, w.shared, layer.h, layer.h_sh, layer.ids, tw, layer.p2r, layer.sg)
    assert_close(to_np(o), to_np(ref), "dropped pairs")


# ------------------------------------------------------------------ MX activation mode, stage by stage

E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
FLIP_BOUND = 2.0 ** -16


def _mx_flip_distances(h_ref, hq, hs):
    """Where the GPU's MX codes of h (hq, hs) decode to another value than the oracle's own
    quantisation of its float64 h_ref: the relative distance of the quantity that decided the
    code from its rounding boundary.  A different scale byte is decided by the block maximum
    against a power of two (the exponent is floor(log2 amax) - 2); a different element with the
    same scale by |v| / 2^X against the nearest E2M1 rounding midpoint."""
    rq, rs = OF.mx_quantize(h_ref)
    diff = OF.mx_dequantize(hq, hs) != OF.mx_dequantize(rq, rs)
    d = []
    for r, c in zip(*np.nonzero(diff)):
        b = c // 32
        if hs[r, b] != rs[r, b]:
            amax = np.abs(h_ref[r, 32 * b:32 * b + 32]).max()
            p2 = 2.0 ** np.round(np.log2(amax))
            d.append(abs(amax - p2) / p2)
        else:
            a = abs(h_ref[r, c]) / 2.0 ** (int(rs[r, b]) - 127)
            m = E2M1_MIDPOINTS[np.argmin(np.abs(E2M1_MIDPOINTS - a))]
            d.append(abs(a - m) / m)
    return np.array(d)


def _check_flips(h_ref, hq, hs, what):
    d = _mx_flip_distances(h_ref, hq, hs)
    say(f"  {what}: {len(d)} h values differ from the oracle's own quantisation, "
        f"max distance from the rounding boundary {d.max() if len(d) else 0.0:.2e} (bound 2^-16)")
    assert (d < FLIP_BOUND).all(), f"{what}: a code differs {d.max():.3e} away from its rounding boundary"
    return len(d)



def _stagewise_mx(M, cfg, dev, tokens=None):
    """Stage-wise parity of the MX-activation FFN (codes of x exact; g/u within tolerance; oracle's
    quantiser on the GPU's h gives the GPU's h codes; down within tolerance on the GPU's h codes;
    every h code that differs from the oracle's own quantisation lies within 2^-16 of a rounding
    boundary).  `tokens`: check the h and y rows of these tokens only (the codes of every row are
    still checked against the oracle's quantiser)."""
    t, inp = build(cfg, dev)
    w = layer_weights(cfg, t)
    r = OL.route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling, inp.logit_bias)
    perm = OL.permute(r.ids, cfg.E)
    offs = torch.from_numpy(perm.expert_offsets.astype(np.int32)).to(dev)
    sp = torch.from_numpy(perm.sorted_pairs.astype(np.int32)).to(dev)
    x = OF.bf16_value(inp.x)
    xq, xs = M.moe_mx_quantize(t["x"])
    rq, rs = OF.mx_quantize(x)
    np.testing.assert_array_equal(to_np(xq), rq)
    np.testing.assert_array_equal(to_np(xs), rs)
    h, hq, hs = M.moe_expert_gateup(w.experts, t["x"], "mxfp4", cfg.k, offs, sp, want_h=True)
    y = M.moe_expert_down(w.experts, cfg.T, "mxfp4", cfg.k, offs, h_codes=hq, h_scales=hs)
    torch.cuda.synchronize()
    h, hq, hs, y = to_np(h), to_np(hq), to_np(hs), to_np(y)
    # oracle quantiser on the GPU's float32 h reproduces the GPU's codes exactly
    oq, os_ = OF.mx_quantize(h.astype(np.float64))
    np.testing.assert_array_equal(hq, oq)
    np.testing.assert_array_equal(hs, os_)
    aq = OF.mx_dequantize(rq, rs)
    rows = np.arange(len(perm.sorted_pairs))
    if tokens is not None:
        rows = rows[np.isin(perm.sorted_pairs // cfg.k, tokens)]
    hdeq = OF.mx_dequantize(hq, hs)
    ge, _ = host_expert_getter(cfg)
    h_ref = np.zeros((len(rows), cfg.I))
    y_ref = np.zeros((len(rows), cfg.d_model))
    for e in np.unique(np.searchsorted(perm.expert_offsets, rows, side="right") - 1):
        sel = np.where((rows >= perm.expert_offsets[e]) & (rows < perm.expert_offsets[e + 1]))[0]
        G, U, D = OL.dequant_expert(ge(int(e)))
        a = aq[perm.sorted_pairs[rows[sel]] // cfg.k]
        h_ref[sel] = OL.silu(a @ G.T) * (a @ U.T)
        y_ref[sel] = hdeq[rows[sel]] @ D.T
    assert_close(h[rows], h_ref, f"{cfg.name} mx h")
    assert_close(y[rows], y_ref, f"{cfg.name} mx y_rows (on GPU h codes)")
    # end to end against the oracle's own h codes: a differing code is a near-tie
    return _check_flips(h_ref, hq[rows], hs[rows], f"{cfg.name} h codes")


def test_mx_activation_tiny_stagewise(dev, M):
    _stagewise_mx(M, tiny(name="tmx", wtag=87, act="mxfp4", T=33, H=512, I=256), dev)


# Shapes that take the block-scaled FP4 GEMM (>= 64 tokens): ragged K-steps (K/32 not a
# multiple of 4), ragged 128-column tiles, experts spanning several 128-row tiles.
MX_GEMM_CASES = {
    "ragged_k_and_n": tiny(name="g1", wtag=91, act="mxfp4", T=160, H=544, I=320, E=4, k=2),
    "multi_tile_rows": tiny(name="g2", wtag=92, act="mxfp4", T=300, H=256, I=128, E=2, k=1),
    "many_experts": tiny(name="g3", wtag=93, act="mxfp4", T=128, H=512, I=256, E=64, k=6),
    # K = 640 (gate/up) and 768 (down): dword-aligned scale rows, an odd number of K-steps, so the
    # last two-step scale window is moved back to end at the row's last byte
    "odd_steps_aligned_scales": tiny(name="g4", wtag=94, act="mxfp4", T=200, H=640, I=768, E=8, k=2),
}


@pytest.mark.parametrize("name", list(MX_GEMM_CASES))
def test_mx_gemm_stagewise(dev, M, name):
    _stagewise_mx(M, MX_GEMM_CASES[name], dev)


def _mx_layer_end_to_end(M, cfg, dev):
    """A whole MX-activation layer step: ids exact; the output within tolerance of the oracle's
    layer with the GPU's h codes (routed and shared) substituted for its own; every h code that
    differs from the oracle's own quantisation a near-tie (within 2^-16 of its boundary)."""
    layer, out, inp = _run_layer(M, cfg, dev)
    ge, gs = host_expert_getter(cfg)
    ref = OL.layer(cfg, inp, ge, gs)
    np.testing.assert_array_equal(to_np(layer.ids), ref.routing.ids)
    hq, hs = to_np(layer.hq), to_np(layer.hs)
    perm, r = ref.perm, ref.routing
    aq = OF.mx_dequantize(*OF.mx_quantize(OF.bf16_value(inp.x)))
    hdeq = OF.mx_dequantize(hq, hs)
    y_rows = np.zeros((len(perm.sorted_pairs), cfg.d_model))
    h_ref = np.zeros((len(perm.sorted_pairs), cfg.I))
    for e in range(cfg.E):
        r0, r1 = int(perm.expert_offsets[e]), int(perm.expert_offsets[e + 1])
        if r0 == r1:
            continue
        G, U, D = OL.dequant_expert(ge(e))
        a = aq[perm.sorted_pairs[r0:r1] // cfg.k]
        h_ref[r0:r1] = OL.silu(a @ G.T) * (a @ U.T)
        y_rows[r0:r1] = hdeq[r0:r1] @ D.T
    nflip = _check_flips(h_ref, hq, hs, f"{cfg.name} routed h")
    y_s = None
    if cfg.shared:
        G, U, D = OL.dequant_expert(gs())
        hsq, hss = (to_np(layer.hq_sh), to_np(layer.hs_sh)) if layer.hq_sh is not None else (None, None)
        if hsq is None:                      # decode-sized steps run the shared expert in the fused call
            y_s = ref.y_shared
        else:
            nflip += _check_flips(OL.silu(aq @ G.T) * (aq @ U.T), hsq, hss, f"{cfg.name} shared h")
            y_s = OF.mx_dequantize(hsq, hss) @ D.T
    want = OL.combine(y_rows, perm.pair_to_row, r.weights, cfg.k, y_s, r.shared_gate)
    assert_close(to_np(out), want, f"{cfg.name} out (oracle on the GPU's h codes)")
    if nflip == 0:
        assert_close(to_np(out), ref.out, f"{cfg.name} out (oracle's own h codes)")


def test_mx_gemm_layer_with_gated_shared_end_to_end(dev, M):
    _mx_layer_end_to_end(M, tiny(name="g4", wtag=94, act="mxfp4", T=96, H=256, I=128, E=8, k=2, shared="gated",
                                 shared_K=256, shared_I=160), dev)


def test_mx_activation_layer_tiny_end_to_end(dev, M):
    _mx_layer_end_to_end(M, tiny(name="tmx2", wtag=88, act="mxfp4", shared="gated", shared_K=256, shared_I=128),
                         dev)


# ------------------------------------------------------------------ full-size workloads

def test_decode_layer_full_size(dev, M):
    cfg = synth.get("qwen38max_decode")
    say("building qwen38max_decode (13.85 GB of experts)")
    layer, out, inp = _run_layer(M, cfg, dev)
    say("oracle over the 11 touched experts")
    ge, gs = host_expert_getter(cfg)
    ref = OL.layer(cfg, inp, ge, gs)
    np.testing.assert_array_equal(to_np(layer.ids), ref.routing.ids)
    assert_close(to_np(layer.topk_w), ref.routing.weights, "decode topk_w")
    if not layer.fused:
        assert_close(to_np(layer.y_rows), ref.y_rows, "decode y_rows")
        assert_close(to_np(layer.y_s), ref.y_shared, "decode shared")
    assert_close(to_np(out), ref.out, "decode out")
    # a second step on the same buffers is bitwise identical (no atomics in value paths)
    first = to_np(out).copy()
    out2 = to_np(layer.forward(bf16_tensor(inp.x, dev)))
    np.testing.assert_array_equal(out2, first)
    # the single launch and the three calls give the same bits
    assert layer.fused and not layer.single
    one = M.MoELayer(layer.w, cfg.T, dev, single_launch=True)
    assert one.single
    out1 = to_np(one.forward(bf16_tensor(inp.x, dev)))
    np.testing.assert_array_equal(out1, first)


def test_latent_layer_full_size(dev, M):
    cfg = synth.get("kimik3_latent_decode")
    say("building kimik3_latent_decode")
    layer, out, inp = _run_layer(M, cfg, dev)
    ge, gs = host_expert_getter(cfg)
    ref = OL.layer(cfg, inp, ge, gs)
    np.testing.assert_array_equal(to_np(layer.ids), ref.routing.ids)
    assert_close(to_np(layer.x_lat), ref.x_expert, "latent x_lat")
    if layer.y_rows is not None:
        assert_close(to_np(layer.y_rows), ref.y_rows, "latent y_rows")
    assert_close(to_np(layer.z), ref.z, "latent z (routed sum at the latent width)")
    assert_close(to_np(layer.y_s), ref.y_shared, "latent shared")
    assert_close(to_np(out), ref.out, "latent out")


def test_fp8_layer_full_size_sampled_tokens(dev, M):
    cfg = synth.get("glm52_fp8")
    say("building glm52_fp8")
    layer, out, inp = _run_layer(M, cfg, dev)
    r = OL.route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling, None,
                 inp.select_bias)
    np.testing.assert_array_equal(to_np(layer.ids), r.ids)
    assert_close(to_np(layer.topk_w), r.weights, "fp8 topk_w")
    ge, gs = host_expert_getter(cfg)
    x = OF.bf16_value(inp.x)
    G, U, D = OL.dequant_expert(gs())
    sample = [0, 17, 63]
    ys = OL.ffn(x[sample], G, U, D)
    ref = np.zeros((len(sample), cfg.H))
    for i, tkn in enumerate(sample):
        for j in range(cfg.k):
            ref[i] += r.weights[tkn, j] * OL.ffn(x[tkn:tkn + 1], *OL.dequant_expert(ge(int(r.ids[tkn, j]))))[0]
        ref[i] += ys[i]
    assert_close(to_np(out)[sample], ref, "fp8 out (sampled tokens)")


def test_prefill_mx_full_size_stagewise_sampled(dev, M):
    cfg = synth.get("qwen38max_prefill")
    say("prefill, MX activations, stage-wise on sampled tokens")
    _stagewise_mx(M, cfg, dev, tokens=[3, 300])


def test_prefill_hot_mx_full_size_stagewise(dev, M):
    """The compute-bound prefill slice at full size (512 tokens on the same 10 experts, 512 rows
    each): the codes of every h row against the oracle's quantiser, and h and y of tokens
    200 .. 327 -- 128 consecutive rows of every expert, across the boundary between its two
    256-row tiles -- against the oracle."""
    cfg = synth.get("qwen38max_prefill_hot")
    say("hot prefill, MX activations, stage-wise on 128 rows of every expert")
    _stagewise_mx(M, cfg, dev, tokens=list(range(200, 328)))


@pytest.mark.parametrize("name,sample", [("qwen38max_prefill_hot_float", [0, 129, 511]),
                                         ("qwen38max_prefill_float", [5, 300])])
def test_prefill_float_full_size_sampled_tokens(dev, M, name, sample):
    cfg = synth.get(name)
    say(f"building {name}")
    layer, out, inp = _run_layer(M, cfg, dev)
    r = OL.route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling, inp.logit_bias,
                 None, inp.w_shared_gate)
    np.testing.assert_array_equal(to_np(layer.ids), r.ids)
    ge, gs = host_expert_getter(cfg)
    x = OF.bf16_value(inp.x)
    ref = np.zeros((len(sample), cfg.H))
    for e in np.unique(r.ids[sample]):
        G, U, D = OL.dequant_expert(ge(int(e)))
        for i, tkn in enumerate(sample):
            for j in np.where(r.ids[tkn] == e)[0]:
                ref[i] += r.weights[tkn, j] * OL.ffn(x[tkn:tkn + 1], G, U, D)[0]
    G, U, D = OL.dequant_expert(gs())
    ys = OL.ffn(x[sample], G, U, D)
    ref += r.shared_gate[sample][:, None] * ys
    assert_close(to_np(out)[sample], ref, "prefill float out (sampled tokens)")


def test_zero_tokens_is_a_no_op(dev, M):
    cfg = tiny()
    t, _ = build(cfg, dev)
    w = layer_weights(cfg, t)
    x0 = t["x"][:0]
    ids, tw, _ = M.moe_route(x0, w.w_router, cfg.k)
    assert ids.shape == (0, cfg.k)
    offs, sp, p2r = M.moe_permute(ids, cfg.E)
    assert to_np(offs).tolist() == [0] * (cfg.E + 1)
