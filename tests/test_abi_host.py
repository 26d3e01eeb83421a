"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/moe.h declares, and reject bad
arguments on the host, before anything is enqueued.  Only argument combinations that
fail validation are passed here (with dummy non-NULL pointers that are never touched),
so no HIP call is made.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

B = pytest.importorskip("mxfp4_routed_expert_amd.binding",
                        reason="libmoe.so not built (python mxfp4_routed_expert_amd/build.py)")
lib = B.lib
DUMMY = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 15, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"
    assert set(names) == set(B.EXPORTS)


def test_abi_version():
    src = open(HEADER).read()
    v = int(re.search(r"#define MOE_ABI_VERSION (\d+)", src).group(1))
    assert lib.moe_abi_version() == v


def _desc(**kw):
    d = dict(T=4, H=256, E=8, k=2, score=0, renormalize=1, routed_scaling=1.0)
    d.update(kw)
    return B.RouteDesc(**d)


@pytest.mark.parametrize("kw,msg", [
    (dict(T=-1), "T = -1"),
    (dict(H=100), "H = 100"),
    (dict(E=0), "E = 0"),
    (dict(E=5000), "E = 5000"),
    (dict(k=0), "k = 0"),
    (dict(k=9), "k = 9"),
    (dict(k=17, E=64), "k = 17"),
    (dict(score=7), "unknown score"),
])
def test_route_rejects_bad_descriptor(kw, msg):
    d = _desc(**kw)
    st = lib.moe_route(ctypes.byref(d), DUMMY, DUMMY, None, None, None, DUMMY, DUMMY, None, DUMMY, 1 << 20, None)
    assert st == B.MOE_ERR_INVALID_ARG
    assert msg in B.last_error()


@pytest.mark.parametrize("kw,msg", [
    (dict(n_group=3), "n_group = 3"),                                   # does not divide E = 8
    (dict(n_group=128, E=256), "n_group = 128"),                        # more than 64 groups
    (dict(n_group=4, topk_group=0), "topk_group = 0"),
    (dict(n_group=4, topk_group=5), "topk_group = 5"),
    (dict(n_group=4, topk_group=1, k=3), "topk_group = 1"),             # 1 group of 2 < k
    (dict(n_group=8, topk_group=4, score=1), "at least 2 experts"),     # sigmoid, groups of 1
    (dict(n_group=-2), "n_group = -2"),
])
def test_route_rejects_bad_groups(kw, msg):
    d = _desc(**kw)
    st = lib.moe_route(ctypes.byref(d), DUMMY, DUMMY, None, None, None, DUMMY, DUMMY, None, DUMMY, 1 << 20, None)
    assert st == B.MOE_ERR_INVALID_ARG and msg in B.last_error(), B.last_error()


def test_route_null_pointers_and_workspace():
    d = _desc()
    assert lib.moe_route(ctypes.byref(d), None, DUMMY, None, None, None, DUMMY, DUMMY, None, DUMMY, 1 << 20,
                         None) == B.MOE_ERR_INVALID_ARG
    need = lib.moe_route_workspace(ctypes.byref(d))
    assert need >= 4 * 9 * 4
    assert lib.moe_route(ctypes.byref(d), DUMMY, DUMMY, None, None, None, DUMMY, DUMMY, None, DUMMY, need - 1,
                         None) == B.MOE_ERR_WORKSPACE
    assert "workspace" in B.last_error()
    # shared gate pointers must come together
    assert lib.moe_route(ctypes.byref(d), DUMMY, DUMMY, None, None, DUMMY, DUMMY, DUMMY, None, DUMMY, need,
                         None) == B.MOE_ERR_INVALID_ARG
    # a selection bias only exists for the sigmoid score
    assert lib.moe_route(ctypes.byref(d), DUMMY, DUMMY, None, DUMMY, None, DUMMY, DUMMY, None, DUMMY, need,
                         None) == B.MOE_ERR_INVALID_ARG


def test_route_permute_checks():
    d = _desc()
    need = lib.moe_route_workspace(ctypes.byref(d))
    # expert_offsets is required
    assert lib.moe_route_permute(ctypes.byref(d), DUMMY, DUMMY, None, None, None, DUMMY, DUMMY, None, None, DUMMY,
                                 DUMMY, DUMMY, need, None) == B.MOE_ERR_INVALID_ARG
    # the route workspace rule applies
    assert lib.moe_route_permute(ctypes.byref(d), DUMMY, DUMMY, None, None, None, DUMMY, DUMMY, None, DUMMY, DUMMY,
                                 DUMMY, DUMMY, need - 1, None) == B.MOE_ERR_WORKSPACE
    # a bad descriptor is refused before anything else
    bad = _desc(k=0)
    assert lib.moe_route_permute(ctypes.byref(bad), DUMMY, DUMMY, None, None, None, DUMMY, DUMMY, None, DUMMY, DUMMY,
                                 DUMMY, DUMMY, need, None) == B.MOE_ERR_INVALID_ARG


def test_route_zero_tokens_is_a_no_op():
    d = _desc(T=0)
    assert lib.moe_route(ctypes.byref(d), None, None, None, None, None, None, None, None, None, 0, None) == B.MOE_OK


def test_permute_rejects_bad_sizes():
    assert lib.moe_permute(4, 3, 2, DUMMY, DUMMY, DUMMY, DUMMY, None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(-1, 1, 2, DUMMY, DUMMY, DUMMY, DUMMY, None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(4, 2, 8, None, DUMMY, DUMMY, DUMMY, None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(4, 2, 8, DUMMY, None, DUMMY, DUMMY, None, 0, None) == B.MOE_ERR_INVALID_ARG


def _weights(fmt=0, E=8, K=256, I=128, null=None):
    p = {n: 0x1000 for n in ("gate", "up", "down", "gate_s", "up_s", "down_s")}
    if null:
        p[null] = None
    return B.ExpertWeightsC(fmt, E, K, I, p["gate"], p["up"], p["down"], p["gate_s"], p["up_s"], p["down_s"])


@pytest.mark.parametrize("w,act,status", [
    (_weights(K=100), 0, B.MOE_ERR_INVALID_ARG),            # MXFP4 width not a multiple of 32
    (_weights(fmt=1, K=256, I=96), 0, B.MOE_ERR_INVALID_ARG),  # FP8 widths not multiples of 128
    (_weights(fmt=3), 0, B.MOE_ERR_INVALID_ARG),
    (_weights(E=0), 0, B.MOE_ERR_INVALID_ARG),
    (_weights(null="down_s"), 0, B.MOE_ERR_INVALID_ARG),
    (_weights(), 5, B.MOE_ERR_INVALID_ARG),
    (_weights(fmt=1), 1, B.MOE_ERR_UNSUPPORTED),             # MX activations need MXFP4 weights
])
def test_expert_ffn_rejects(w, act, status):
    st = lib.moe_expert_ffn(ctypes.byref(w), act, 4, 2, DUMMY, 0, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 30, None)
    assert st == status, B.last_error()


def test_expert_ffn_row_checks_and_workspace():
    w = _weights()
    # routed form needs 1 <= k <= min(E, 16) and sorted_pairs
    assert lib.moe_expert_ffn(ctypes.byref(w), 0, 4, 9, DUMMY, 0, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 30,
                              None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(ctypes.byref(w), 0, 4, 2, DUMMY, 0, DUMMY, None, DUMMY, DUMMY, 1 << 30,
                              None) == B.MOE_ERR_INVALID_ARG
    # identity form needs exactly one expert
    assert lib.moe_expert_ffn(ctypes.byref(w), 0, 4, 1, DUMMY, 0, None, None, DUMMY, DUMMY, 1 << 30,
                              None) == B.MOE_ERR_INVALID_ARG
    # unknown activation dtype
    assert lib.moe_expert_ffn(ctypes.byref(w), 0, 4, 2, DUMMY, 9, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 30,
                              None) == B.MOE_ERR_INVALID_ARG
    need = lib.moe_expert_ffn_workspace(ctypes.byref(w), 0, 4, 2)
    assert need >= 4 * 2 * 128 * 4          # float32 h for T*k rows
    assert lib.moe_expert_ffn(ctypes.byref(w), 0, 4, 2, DUMMY, 0, DUMMY, DUMMY, DUMMY, DUMMY, need - 1,
                              None) == B.MOE_ERR_WORKSPACE
    need_mx = lib.moe_expert_ffn_workspace(ctypes.byref(w), 1, 4, 2)
    assert need_mx > need                   # plus MX codes of x and h
    assert lib.moe_expert_ffn(ctypes.byref(w), 0, 0, 2, None, 0, DUMMY, None, None, None, 0, None) == B.MOE_OK


def test_gateup_and_down_require_their_outputs():
    w = _weights()
    assert lib.moe_expert_gateup(ctypes.byref(w), 0, 4, 2, DUMMY, 0, DUMMY, DUMMY, None, None, None, DUMMY,
                                 1 << 20, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_gateup(ctypes.byref(w), 1, 4, 2, DUMMY, 0, DUMMY, DUMMY, DUMMY, None, None, DUMMY,
                                 1 << 20, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_down(ctypes.byref(w), 0, 4, 2, None, None, None, DUMMY, DUMMY,
                               None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_down(ctypes.byref(w), 1, 4, 2, DUMMY, DUMMY, None, DUMMY, DUMMY,
                               None) == B.MOE_ERR_INVALID_ARG


def test_fused_decode_calls_validation():
    w, sh = _weights(), _weights(E=1)
    gu, dc = lib.moe_expert_gateup_shared, lib.moe_expert_down_combine
    ok_args = (4, 2, DUMMY, 0, DUMMY, DUMMY, DUMMY, DUMMY, None)
    # the shared set holds one expert of the routed format and d_model
    assert gu(ctypes.byref(w), ctypes.byref(_weights(E=2)), *ok_args) == B.MOE_ERR_INVALID_ARG
    assert gu(ctypes.byref(w), ctypes.byref(_weights(fmt=1, E=1)), *ok_args) == B.MOE_ERR_INVALID_ARG
    assert gu(ctypes.byref(w), ctypes.byref(_weights(E=1, K=512)), *ok_args) == B.MOE_ERR_INVALID_ARG
    # routed rows need expert_offsets and sorted_pairs; h_shared is required with a shared set
    assert gu(ctypes.byref(w), None, 4, 2, DUMMY, 0, None, DUMMY, DUMMY, None, None) == B.MOE_ERR_INVALID_ARG
    assert gu(ctypes.byref(w), ctypes.byref(sh), 4, 2, DUMMY, 0, DUMMY, DUMMY, DUMMY, None,
              None) == B.MOE_ERR_INVALID_ARG
    assert gu(ctypes.byref(w), ctypes.byref(sh), 4, 2, DUMMY, 7, DUMMY, DUMMY, DUMMY, DUMMY,
              None) == B.MOE_ERR_INVALID_ARG
    assert gu(ctypes.byref(w), ctypes.byref(sh), 0, 2, None, 0, DUMMY, None, None, None, None) == B.MOE_OK
    dc_args = (DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, DUMMY, None)
    # down-combine: the shared d_ff must equal d_ff; k + 1 rows of d_ff must fit in LDS
    assert dc(ctypes.byref(w), ctypes.byref(_weights(E=1, I=256)), 4, 2, *dc_args) == B.MOE_ERR_INVALID_ARG
    big = _weights(E=16, I=4096)
    assert dc(ctypes.byref(big), None, 4, 10, *dc_args) == B.MOE_ERR_UNSUPPORTED
    assert dc(ctypes.byref(w), None, 4, 9, *dc_args) == B.MOE_ERR_INVALID_ARG          # k > E
    assert dc(ctypes.byref(w), ctypes.byref(sh), 4, 2, DUMMY, None, DUMMY, DUMMY, DUMMY, None, DUMMY,
              None) == B.MOE_ERR_INVALID_ARG                                           # h_shared missing
    assert dc(ctypes.byref(w), None, 4, 2, DUMMY, None, DUMMY, DUMMY, None, None, DUMMY,
              None) == B.MOE_ERR_INVALID_ARG                                           # pair_to_row missing
    assert dc(ctypes.byref(w), None, 0, 2, None, None, None, None, None, None, None, None) == B.MOE_OK


def test_combine_dense_dequant_quantize_validation():
    assert lib.moe_combine(4, 17, 64, DUMMY, DUMMY, DUMMY, None, None, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(4, 2, 0, DUMMY, DUMMY, DUMMY, None, None, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(4, 2, 64, DUMMY, DUMMY, DUMMY, None, DUMMY, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(0, 2, 64, None, None, None, None, None, None, None) == B.MOE_OK
    assert lib.moe_dense_bf16(4, 64, 30, DUMMY, 0, DUMMY, None, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_dense_bf16(4, 64, 32, DUMMY, 7, DUMMY, None, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_dequant(0, 4, 48, DUMMY, DUMMY, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_dequant(1, 100, 128, DUMMY, DUMMY, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_dequant(2, 4, 64, DUMMY, DUMMY, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_quantize(4, 48, DUMMY, 0, DUMMY, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_quantize(4, 64, None, 0, DUMMY, DUMMY, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_mx_quantize(0, 64, None, 0, None, None, None) == B.MOE_OK


def test_product_path_has_no_oracle_dependency():
    # the package never imports the oracle (test infrastructure) nor the input generator
    pkg = os.path.join(ROOT, "mxfp4_routed_expert_amd")
    pat = re.compile(r"^\s*(import|from)\s+(oracle|synth)\b|#include\s+\S*oracle", re.M)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not pat.search(src), os.path.join(dirpath, f)


def test_layer_fusion_rule():
    from types import SimpleNamespace as NS
    from mxfp4_routed_expert_amd.layer import fuses
    ex = NS(fmt="mxfp4", d_model=7168, d_ff=2368)
    base = dict(act="float", p_down=None, p_up=None, k=10, experts=ex, shared=NS(fmt="mxfp4", d_model=7168, d_ff=2368))
    w = lambda **kw: NS(**{**base, **kw})
    assert fuses(w(), 1) and fuses(w(), 4) and fuses(w(shared=None), 2)
    assert not fuses(w(), 5)                                            # prefill-sized batch
    assert not fuses(w(act="mxfp4"), 1)                                  # MX activations
    assert not fuses(w(p_down=object(), p_up=object()), 1)               # LatentMoE
    assert not fuses(w(shared=NS(fmt="mxfp4", d_model=7168, d_ff=1024)), 1)
    assert not fuses(w(shared=NS(fmt="fp8b128", d_model=7168, d_ff=2368)), 1)
    assert not fuses(w(k=16, experts=NS(fmt="mxfp4", d_model=7168, d_ff=4096), shared=None), 1)  # LDS


def test_route_permute_noalloc_refuses_more_than_its_scratch():
    """A request whose routing scratch exceeds the static array is refused on the host, before
    anything touches the GPU (here 5000 x 2049 float32 logits, about 41 MB)."""
    d = _desc(T=5000, H=512, E=2048, k=8)
    st = lib.moe_route_permute_noalloc(ctypes.byref(d), DUMMY, DUMMY, None, None, None, DUMMY, DUMMY, None, DUMMY,
                                       DUMMY, DUMMY, None)
    assert st == B.MOE_ERR_UNSUPPORTED
    assert "scratch" in B.last_error()


def _decode_step(d, w, sync=DUMMY, shared=None, wsg=None, sg=None):
    return lib.moe_decode_step(ctypes.byref(d), DUMMY, DUMMY, wsg, None, None, ctypes.byref(w),
                               ctypes.byref(shared) if shared is not None else None, DUMMY, DUMMY, DUMMY, sg,
                               DUMMY, DUMMY, DUMMY, DUMMY, DUMMY if shared is not None else None, DUMMY, sync, None)


def test_decode_step_checks():
    # counters, 1024 workgroup flags, tagged logits of 4 tokens x 520 rows (64-bit words)
    assert lib.moe_decode_step_sync_bytes() == 4 * (64 + 1024 + 2 * 4 * 520)
    w = _weights()
    # a sync buffer is required
    assert _decode_step(_desc(), w, sync=None) == B.MOE_ERR_INVALID_ARG and "sync" in B.last_error()
    # more than 8 tokens is not a decode step
    assert _decode_step(_desc(T=9), w) == B.MOE_ERR_INVALID_ARG and "T = 9" in B.last_error()
    # the router's E and H must be the experts'
    assert _decode_step(_desc(E=16), w) == B.MOE_ERR_INVALID_ARG
    assert _decode_step(_desc(H=512), w) == B.MOE_ERR_INVALID_ARG
    # a shared gate needs its output
    assert _decode_step(_desc(), w, wsg=DUMMY, sg=None) == B.MOE_ERR_INVALID_ARG
    # k + 1 rows of a wide d_ff do not fit the down-combine's LDS
    wide = _weights(E=16, K=256, I=8192)
    assert _decode_step(_desc(E=16, k=8), wide, shared=_weights(E=1, K=256, I=8192)) == B.MOE_ERR_UNSUPPORTED
    # a bad descriptor is refused first; zero tokens with NULL outputs is a no-op
    assert _decode_step(_desc(k=0), w) == B.MOE_ERR_INVALID_ARG
