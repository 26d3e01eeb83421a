"""ctypes binding of libmoe.so: one Python function per C entry point, same names.

Argument marshalling only: tensors are checked for device, dtype and layout, outputs and
workspaces are allocated with torch (device memory plumbing), and every computation runs
in the HIP library on torch's current stream.  If the library is missing, importing this
module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
SCORE = {"softmax": 0, "sigmoid": 1}
WFMT = {"mxfp4": 0, "fp8b128": 1}
ACT = {"float": 0, "mxfp4": 1}
DT = {torch.bfloat16: 0, torch.float32: 1}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                          "(run `python mxfp4_routed_expert_amd/build.py`)")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_p, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float


class RouteDesc(ctypes.Structure):
    _fields_ = [("T", _i32), ("H", _i32), ("E", _i32), ("k", _i32), ("score", _i32),
                ("renormalize", _i32), ("routed_scaling", _f32), ("n_group", _i32), ("topk_group", _i32)]


class ExpertWeightsC(ctypes.Structure):
    _fields_ = [("format", _i32), ("num_experts", _i32), ("d_model", _i32), ("d_ff", _i32),
                ("gate", _p), ("up", _p), ("down", _p), ("gate_s", _p), ("up_s", _p), ("down_s", _p)]


def _sig(name, res, *args):
    f = getattr(lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("moe_last_error", ctypes.c_char_p)
_sig("moe_abi_version", _i32)
_sig("moe_route", _i32, ctypes.POINTER(RouteDesc), _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p)
_sig("moe_route_workspace", _sz, ctypes.POINTER(RouteDesc))
_sig("moe_permute", _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p)
_sig("moe_route_permute", _i32, ctypes.POINTER(RouteDesc), _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p)
_sig("moe_permute_workspace", _sz, _i32, _i32, _i32)
_sig("moe_route_permute_noalloc", _i32, ctypes.POINTER(RouteDesc), _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p)
_sig("moe_expert_ffn", _i32, ctypes.POINTER(ExpertWeightsC), _i32, _i32, _i32, _p, _i32, _p, _p, _p, _p, _sz, _p)
_sig("moe_expert_ffn_workspace", _sz, ctypes.POINTER(ExpertWeightsC), _i32, _i32, _i32)
_sig("moe_expert_gateup", _i32, ctypes.POINTER(ExpertWeightsC), _i32, _i32, _i32, _p, _i32, _p, _p, _p, _p, _p,
     _p, _sz, _p)
_sig("moe_expert_gateup_workspace", _sz, ctypes.POINTER(ExpertWeightsC), _i32, _i32, _i32)
_sig("moe_expert_down", _i32, ctypes.POINTER(ExpertWeightsC), _i32, _i32, _i32, _p, _p, _p, _p, _p, _p)
_sig("moe_expert_gateup_shared", _i32, ctypes.POINTER(ExpertWeightsC), ctypes.POINTER(ExpertWeightsC), _i32, _i32, _p,
     _i32, _p, _p, _p, _p, _p)
_sig("moe_router_logits", _i32, ctypes.POINTER(RouteDesc), _p, _p, _p, _p, _p, _sz, _p)
_sig("moe_topk_gateup_shared", _i32, ctypes.POINTER(RouteDesc), _p, _p, _p, _i32, ctypes.POINTER(ExpertWeightsC),
     ctypes.POINTER(ExpertWeightsC), _p, _p, _p, _p, _p, _p, _p, _p, _p, _p)
_sig("moe_expert_down_combine", _i32, ctypes.POINTER(ExpertWeightsC), ctypes.POINTER(ExpertWeightsC), _i32, _i32, _p,
     _p, _p, _p, _p, _p, _p, _p)
_sig("moe_decode_step_sync_bytes", _sz)
_sig("moe_decode_step", _i32, ctypes.POINTER(RouteDesc), _p, _p, _p, _p, _p, ctypes.POINTER(ExpertWeightsC),
     ctypes.POINTER(ExpertWeightsC), _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p)
_sig("moe_combine", _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p)
_sig("moe_dense_bf16", _i32, _i32, _i32, _i32, _p, _i32, _p, _p, _p, _p)
_sig("moe_dequant_bf16", _i32, _i32, _i32, _p, _p, _p, _p)
_sig("moe_dequant", _i32, _i32, _i32, _i32, _p, _p, _p, _p)
_sig("moe_mx_quantize", _i32, _i32, _i32, _p, _i32, _p, _p, _p)

EXPORTS = ["moe_route", "moe_route_workspace", "moe_permute", "moe_permute_workspace", "moe_route_permute",
           "moe_route_permute_noalloc",
           "moe_expert_ffn", "moe_expert_gateup_shared", "moe_router_logits", "moe_topk_gateup_shared",
           "moe_expert_down_combine", "moe_decode_step", "moe_decode_step_sync_bytes",
           "moe_expert_ffn_workspace", "moe_expert_gateup", "moe_expert_gateup_workspace", "moe_expert_down",
           "moe_combine", "moe_dense_bf16", "moe_dequant", "moe_dequant_bf16", "moe_mx_quantize", "moe_last_error",
           "moe_abi_version"]


def last_error() -> str:
    return (lib.moe_last_error() or b"").decode()


def check(status: int):
    if status != MOE_OK:
        raise MoeError(status, last_error())


def abi_version() -> int:
    return lib.moe_abi_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live in device memory (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _workspace(nbytes: int, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ router

def moe_route(x, w_router, k, score="softmax", renormalize=True, routed_scaling=1.0, logit_bias=None,
              select_bias=None, w_shared_gate=None, out=None, ws=None, n_group=1, topk_group=1):
    """Returns (topk_ids int32 [T][k], topk_w float32 [T][k], shared_gate float32 [T] or None).
    n_group > 1 selects among the topk_group best expert groups only (see moe.h)."""
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router", (E, H))
    _need(logit_bias, torch.float32, "logit_bias", (E,))
    _need(select_bias, torch.float32, "select_bias", (E,))
    _need(w_shared_gate, torch.bfloat16, "w_shared_gate", (H,))
    d = RouteDesc(T, H, E, k, SCORE[score], 1 if renormalize else 0, routed_scaling, n_group, topk_group)
    dev = x.device
    if out is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        sg = torch.empty((T,), dtype=torch.float32, device=dev) if w_shared_gate is not None else None
    else:
        ids, w, sg = out
    if ws is None:
        ws = _workspace(lib.moe_route_workspace(ctypes.byref(d)), dev)
    check(lib.moe_route(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
                        _ptr(w_shared_gate), _ptr(ids), _ptr(w), _ptr(sg), _ptr(ws), ws.numel(), _stream()))
    return ids, w, sg


def moe_permute(topk_ids, E, out=None):
    """Returns (expert_offsets [E+1], sorted_pairs [T*k], pair_to_row [T*k]), int32."""
    T, k = topk_ids.shape
    _need(topk_ids, torch.int32, "topk_ids")
    dev = topk_ids.device
    if out is None:
        offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        sp = torch.empty((T * k,), dtype=torch.int32, device=dev)
        p2r = torch.empty((T * k,), dtype=torch.int32, device=dev)
    else:
        offs, sp, p2r = out
    check(lib.moe_permute(T, k, E, _ptr(topk_ids), _ptr(offs), _ptr(sp), _ptr(p2r), None, 0, _stream()))
    return offs, sp, p2r


def moe_route_permute(x, w_router, k, score="softmax", renormalize=True, routed_scaling=1.0, logit_bias=None,
                      select_bias=None, w_shared_gate=None, out=None, ws=None, n_group=1, topk_group=1):
    """moe_route then moe_permute in one call.  Returns (topk_ids, topk_w, shared_gate or None,
    expert_offsets, sorted_pairs, pair_to_row)."""
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router", (E, H))
    _need(logit_bias, torch.float32, "logit_bias", (E,))
    _need(select_bias, torch.float32, "select_bias", (E,))
    _need(w_shared_gate, torch.bfloat16, "w_shared_gate", (H,))
    d = RouteDesc(T, H, E, k, SCORE[score], 1 if renormalize else 0, routed_scaling, n_group, topk_group)
    dev = x.device
    if out is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        sg = torch.empty((T,), dtype=torch.float32, device=dev) if w_shared_gate is not None else None
        offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        sp = torch.empty((T * k,), dtype=torch.int32, device=dev)
        p2r = torch.empty((T * k,), dtype=torch.int32, device=dev)
    else:
        ids, w, sg, offs, sp, p2r = out
    if ws is None:
        ws = _workspace(lib.moe_route_workspace(ctypes.byref(d)), dev)
    check(lib.moe_route_permute(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
                                _ptr(w_shared_gate), _ptr(ids), _ptr(w), _ptr(sg), _ptr(offs), _ptr(sp), _ptr(p2r),
                                _ptr(ws), ws.numel(), _stream()))
    return ids, w, sg, offs, sp, p2r


def moe_route_permute_noalloc(x, w_router, k, score="softmax", renormalize=True, routed_scaling=1.0,
                              logit_bias=None, select_bias=None, w_shared_gate=None, out=None, n_group=1,
                              topk_group=1):
    """moe_route_permute with the library's static scratch instead of a workspace.  `out` as for
    moe_route_permute (allocated here, by torch, when None)."""
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router", (E, H))
    _need(logit_bias, torch.float32, "logit_bias", (E,))
    _need(select_bias, torch.float32, "select_bias", (E,))
    _need(w_shared_gate, torch.bfloat16, "w_shared_gate", (H,))
    d = RouteDesc(T, H, E, k, SCORE[score], 1 if renormalize else 0, routed_scaling, n_group, topk_group)
    dev = x.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T,), dtype=torch.float32, device=dev) if w_shared_gate is not None else None,
               torch.empty((E + 1,), dtype=torch.int32, device=dev), torch.empty((T * k,), dtype=torch.int32, device=dev),
               torch.empty((T * k,), dtype=torch.int32, device=dev))
    ids, w, sg, offs, sp, p2r = out
    check(lib.moe_route_permute_noalloc(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                        _ptr(select_bias), _ptr(w_shared_gate), _ptr(ids), _ptr(w), _ptr(sg),
                                        _ptr(offs), _ptr(sp), _ptr(p2r), _stream()))
    return ids, w, sg, offs, sp, p2r


# ------------------------------------------------------------------ experts

@dataclass
class ExpertWeights:
    """Device tensors of an expert stack in the storage layout of moe.h."""
    fmt: str
    d_model: int
    d_ff: int
    gate: torch.Tensor
    gate_s: torch.Tensor
    up: torch.Tensor
    up_s: torch.Tensor
    down: torch.Tensor
    down_s: torch.Tensor

    @property
    def num_experts(self):
        return self.gate.shape[0]

    def c_struct(self):
        E, K, I = self.num_experts, self.d_model, self.d_ff
        if self.fmt == "mxfp4":
            shapes = {"gate": (E, I, K // 2), "up": (E, I, K // 2), "down": (E, K, I // 2),
                      "gate_s": (E, I, K // 32), "up_s": (E, I, K // 32), "down_s": (E, K, I // 32)}
            sdt = torch.uint8
        else:
            shapes = {"gate": (E, I, K), "up": (E, I, K), "down": (E, K, I),
                      "gate_s": (E, I // 128, K // 128), "up_s": (E, I // 128, K // 128),
                      "down_s": (E, K // 128, I // 128)}
            sdt = torch.float32
        for n, s in shapes.items():
            _need(getattr(self, n), sdt if n.endswith("_s") else torch.uint8, n, s)
        return ExpertWeightsC(WFMT[self.fmt], E, K, I, self.gate.data_ptr(), self.up.data_ptr(),
                              self.down.data_ptr(), self.gate_s.data_ptr(), self.up_s.data_ptr(),
                              self.down_s.data_ptr())

    @staticmethod
    def from_arrays(es, device=None):
        t = lambda a: a if isinstance(a, torch.Tensor) else torch.from_numpy(a).to(device)
        return ExpertWeights(es.fmt, es.d_model, es.d_ff, t(es.gate), t(es.gate_s), t(es.up), t(es.up_s),
                             t(es.down), t(es.down_s))


def moe_expert_ffn(w: ExpertWeights, x, act="float", k=1, expert_offsets=None, sorted_pairs=None, out=None,
                   ws=None):
    """y_rows [R][d_model] float32; R = T*k (routed) or T (expert_offsets None, one expert)."""
    T = x.shape[0]
    _need(x, None, "x", (T, w.d_model))
    _need(expert_offsets, torch.int32, "expert_offsets", (w.num_experts + 1,))
    _need(sorted_pairs, torch.int32, "sorted_pairs")
    c = w.c_struct()
    R = T * k if expert_offsets is not None else T
    y = out if out is not None else torch.empty((R, w.d_model), dtype=torch.float32, device=x.device)
    _need(y, torch.float32, "y_rows", (R, w.d_model))
    kk = k if expert_offsets is not None else 1
    if ws is None:
        ws = _workspace(lib.moe_expert_ffn_workspace(ctypes.byref(c), ACT[act], T, kk), x.device)
    check(lib.moe_expert_ffn(ctypes.byref(c), ACT[act], T, kk, _ptr(x), DT[x.dtype], _ptr(expert_offsets),
                             _ptr(sorted_pairs), _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y


def moe_expert_ffn_workspace(w: ExpertWeights, act, T, k):
    return lib.moe_expert_ffn_workspace(ctypes.byref(w.c_struct()), ACT[act], T, k)


def moe_expert_gateup_workspace(w: ExpertWeights, act, T, k):
    return lib.moe_expert_gateup_workspace(ctypes.byref(w.c_struct()), ACT[act], T, k)


def moe_expert_gateup(w: ExpertWeights, x, act="float", k=1, expert_offsets=None, sorted_pairs=None,
                      want_h=True, out=None, ws=None):
    """Returns (h float32 [R][d_ff] or None, h_codes or None, h_scales or None)."""
    T = x.shape[0]
    _need(x, None, "x", (T, w.d_model))
    c = w.c_struct()
    kk = k if expert_offsets is not None else 1
    R = T * kk
    dev = x.device
    if out is not None:
        h, hq, hs = out
    else:
        h = torch.empty((R, w.d_ff), dtype=torch.float32, device=dev) if (want_h or act == "float") else None
        hq = hs = None
        if act == "mxfp4":
            hq = torch.empty((R, w.d_ff // 2), dtype=torch.uint8, device=dev)
            hs = torch.empty((R, w.d_ff // 32), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = _workspace(lib.moe_expert_gateup_workspace(ctypes.byref(c), ACT[act], T, kk), dev)
    check(lib.moe_expert_gateup(ctypes.byref(c), ACT[act], T, kk, _ptr(x), DT[x.dtype], _ptr(expert_offsets),
                                _ptr(sorted_pairs), _ptr(h), _ptr(hq), _ptr(hs), _ptr(ws), ws.numel(), _stream()))
    return h, hq, hs


def moe_expert_down(w: ExpertWeights, T, act="float", k=1, expert_offsets=None, h=None, h_codes=None,
                    h_scales=None, out=None):
    c = w.c_struct()
    kk = k if expert_offsets is not None else 1
    R = T * kk
    dev = (h if h is not None else h_codes).device
    y = out if out is not None else torch.empty((R, w.d_model), dtype=torch.float32, device=dev)
    check(lib.moe_expert_down(ctypes.byref(c), ACT[act], T, kk, _ptr(h), _ptr(h_codes), _ptr(h_scales),
                              _ptr(expert_offsets), _ptr(y), _stream()))
    return y


def moe_expert_gateup_shared(w: ExpertWeights, shared, x, k, expert_offsets, sorted_pairs, out=None):
    """Routed gate/up (FLOAT activations) and, when `shared` is given, the shared expert's
    gate/up over every token, in one launch.  Returns (h [T*k][d_ff], h_shared [T][d_ff_s] or None)."""
    T = x.shape[0]
    _need(x, None, "x", (T, w.d_model))
    dev = x.device
    if out is not None:
        h, hsh = out
    else:
        h = torch.empty((T * k, w.d_ff), dtype=torch.float32, device=dev)
        hsh = torch.empty((T, shared.d_ff), dtype=torch.float32, device=dev) if shared is not None else None
    c = w.c_struct()
    cs = shared.c_struct() if shared is not None else None
    check(lib.moe_expert_gateup_shared(ctypes.byref(c), ctypes.byref(cs) if cs is not None else None, T, k, _ptr(x),
                                       DT[x.dtype], _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(h), _ptr(hsh),
                                       _stream()))
    return h, hsh


def moe_router_logits(x, w_router, k, score="softmax", w_shared_gate=None, out=None, ws=None, n_group=1,
                      topk_group=1):
    """float32 router logits [T][E (+1 with the shared gate)]."""
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router", (E, H))
    _need(w_shared_gate, torch.bfloat16, "w_shared_gate", (H,))
    d = RouteDesc(T, H, E, k, SCORE[score], 1, 1.0, n_group, topk_group)
    rows = E + (1 if w_shared_gate is not None else 0)
    lg = out if out is not None else torch.empty((T, rows), dtype=torch.float32, device=x.device)
    _need(lg, torch.float32, "logits", (T, rows))
    if ws is None:
        ws = _workspace(lib.moe_route_workspace(ctypes.byref(d)), x.device)
    check(lib.moe_router_logits(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(w_shared_gate), _ptr(lg), _ptr(ws),
                                ws.numel(), _stream()))
    return lg


def moe_topk_gateup_shared(logits, x, k, w: ExpertWeights, shared=None, score="softmax", renormalize=True,
                           routed_scaling=1.0, logit_bias=None, select_bias=None, has_shared_gate=False, out=None,
                           n_group=1, topk_group=1):
    """Routing of `logits` (moe_route_permute's selection) and the routed + shared gate/up on it,
    in one launch.  Returns (topk_ids, topk_w, shared_gate or None, expert_offsets, sorted_pairs,
    pair_to_row, h [T*k][d_ff], h_shared [T][d_ff_s] or None)."""
    T, H = x.shape
    E = w.num_experts
    _need(x, torch.bfloat16, "x")
    _need(logits, torch.float32, "logits", (T, E + (1 if has_shared_gate else 0)))
    _need(logit_bias, torch.float32, "logit_bias", (E,))
    _need(select_bias, torch.float32, "select_bias", (E,))
    d = RouteDesc(T, H, E, k, SCORE[score], 1 if renormalize else 0, routed_scaling, n_group, topk_group)
    dev = x.device
    if out is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        tw = torch.empty((T, k), dtype=torch.float32, device=dev)
        sg = torch.empty((T,), dtype=torch.float32, device=dev) if has_shared_gate else None
        offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        sp = torch.empty((T * k,), dtype=torch.int32, device=dev)
        p2r = torch.empty((T * k,), dtype=torch.int32, device=dev)
        h = torch.empty((T * k, w.d_ff), dtype=torch.float32, device=dev)
        hsh = torch.empty((T, shared.d_ff), dtype=torch.float32, device=dev) if shared is not None else None
    else:
        ids, tw, sg, offs, sp, p2r, h, hsh = out
    c = w.c_struct()
    cs = shared.c_struct() if shared is not None else None
    check(lib.moe_topk_gateup_shared(ctypes.byref(d), _ptr(logits), _ptr(logit_bias), _ptr(select_bias),
                                     1 if has_shared_gate else 0, ctypes.byref(c),
                                     ctypes.byref(cs) if cs is not None else None, _ptr(x), _ptr(ids), _ptr(tw),
                                     _ptr(sg), _ptr(offs), _ptr(sp), _ptr(p2r), _ptr(h), _ptr(hsh), _stream()))
    return ids, tw, sg, offs, sp, p2r, h, hsh


def moe_expert_down_combine(w: ExpertWeights, shared, h, h_shared, topk_ids, topk_w, pair_to_row, shared_gate=None,
                            out=None):
    """out[t] = sum_j topk_w[t][j] * down_{e_j}(h[pair_to_row[t*k+j]]) + g_t * shared_down(h_shared[t]),
    float32 [T][d_model], in one launch."""
    T, k = topk_w.shape
    _need(topk_ids, torch.int32, "topk_ids", (T, k))
    o = out if out is not None else torch.empty((T, w.d_model), dtype=torch.float32, device=topk_w.device)
    c = w.c_struct()
    cs = shared.c_struct() if shared is not None else None
    check(lib.moe_expert_down_combine(ctypes.byref(c), ctypes.byref(cs) if cs is not None else None, T, k, _ptr(h),
                                      _ptr(h_shared), _ptr(topk_ids), _ptr(topk_w), _ptr(pair_to_row),
                                      _ptr(shared_gate), _ptr(o), _stream()))
    return o


def decode_step_sync(device):
    """A zero-filled sync buffer for moe_decode_step (one per stream that runs steps)."""
    return torch.zeros((lib.moe_decode_step_sync_bytes() // 4,), dtype=torch.int32, device=device)


def moe_decode_step(x, w_router, k, w: ExpertWeights, shared=None, score="softmax", renormalize=True,
                    routed_scaling=1.0, logit_bias=None, select_bias=None, w_shared_gate=None, sync=None, out=None,
                    n_group=1, topk_group=1):
    """A whole decode layer step (router logits, top-k with the routed and shared gate/up, down
    with the weighted combine) in one launch when the shapes allow it.  `sync`: a buffer from
    decode_step_sync(), kept across calls.  Returns (logits, topk_ids, topk_w, shared_gate or
    None, expert_offsets, sorted_pairs, pair_to_row, h, h_shared or None, out [T][d_model])."""
    T, H = x.shape
    E = w.num_experts
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router", (E, H))
    _need(w_shared_gate, torch.bfloat16, "w_shared_gate", (H,))
    _need(logit_bias, torch.float32, "logit_bias", (E,))
    _need(select_bias, torch.float32, "select_bias", (E,))
    if sync is None:
        raise MoeError(1, "moe_decode_step: a sync buffer (decode_step_sync) is required")
    _need(sync, torch.int32, "sync", (lib.moe_decode_step_sync_bytes() // 4,))
    d = RouteDesc(T, H, E, k, SCORE[score], 1 if renormalize else 0, routed_scaling, n_group, topk_group)
    dev = x.device
    has_sg = w_shared_gate is not None
    if out is None:
        lg = torch.empty((T, E + (1 if has_sg else 0)), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        tw = torch.empty((T, k), dtype=torch.float32, device=dev)
        sg = torch.empty((T,), dtype=torch.float32, device=dev) if has_sg else None
        offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        sp = torch.empty((T * k,), dtype=torch.int32, device=dev)
        p2r = torch.empty((T * k,), dtype=torch.int32, device=dev)
        h = torch.empty((T * k, w.d_ff), dtype=torch.float32, device=dev)
        hsh = torch.empty((T, shared.d_ff), dtype=torch.float32, device=dev) if shared is not None else None
        o = torch.empty((T, w.d_model), dtype=torch.float32, device=dev)
    else:
        lg, ids, tw, sg, offs, sp, p2r, h, hsh, o = out
    c = w.c_struct()
    cs = shared.c_struct() if shared is not None else None
    check(lib.moe_decode_step(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(w_shared_gate), _ptr(logit_bias),
                              _ptr(select_bias), ctypes.byref(c), ctypes.byref(cs) if cs is not None else None,
                              _ptr(lg), _ptr(ids), _ptr(tw), _ptr(sg), _ptr(offs), _ptr(sp), _ptr(p2r), _ptr(h),
                              _ptr(hsh), _ptr(o), _ptr(sync), _stream()))
    return lg, ids, tw, sg, offs, sp, p2r, h, hsh, o


# ------------------------------------------------------------------ combine, dense, formats

def moe_route_workspace(T, H, E, k, score="softmax"):
    d = RouteDesc(T, H, E, k, SCORE[score], 1, 1.0, 1, 1)
    return lib.moe_route_workspace(ctypes.byref(d))


def moe_combine(y_rows, pair_to_row, topk_w, y_shared=None, shared_gate=None, out=None):
    T, k = topk_w.shape
    d = y_rows.shape[1] if y_rows is not None else y_shared.shape[1]
    _need(y_rows, torch.float32, "y_rows")
    _need(pair_to_row, torch.int32, "pair_to_row", (T * k,))
    _need(topk_w, torch.float32, "topk_w")
    _need(y_shared, torch.float32, "y_shared", (T, d))
    _need(shared_gate, torch.float32, "shared_gate", (T,))
    o = out if out is not None else torch.empty((T, d), dtype=torch.float32, device=topk_w.device)
    check(lib.moe_combine(T, k, d, _ptr(y_rows), _ptr(pair_to_row), _ptr(topk_w), _ptr(y_shared),
                          _ptr(shared_gate), _ptr(o), _stream()))
    return o


def moe_dense_bf16(x, w, residual=None, out=None):
    T, kdim = x.shape
    n = w.shape[0]
    _need(x, None, "x")
    _need(w, torch.bfloat16, "w", (n, kdim))
    _need(residual, torch.float32, "residual", (T, n))
    y = out if out is not None else torch.empty((T, n), dtype=torch.float32, device=x.device)
    check(lib.moe_dense_bf16(T, n, kdim, _ptr(x), DT[x.dtype], _ptr(w), _ptr(residual), _ptr(y), _stream()))
    return y


def moe_dequant(fmt, codes, scales):
    _need(codes, torch.uint8, "codes")
    _need(scales, None, "scales")
    n = codes.shape[0]
    kdim = codes.shape[1] * (2 if fmt == "mxfp4" else 1)
    out = torch.empty((n, kdim), dtype=torch.float32, device=codes.device)
    check(lib.moe_dequant(WFMT[fmt], n, kdim, _ptr(codes), _ptr(scales), _ptr(out), _stream()))
    return out


def moe_dequant_bf16(codes, scales):
    """MXFP4 codes [n][kdim/2] + E8M0 scales [n][kdim/32] -> bf16 [n][kdim] (the matrix-core decode)."""
    _need(codes, torch.uint8, "codes")
    n = codes.shape[0]
    kdim = codes.shape[1] * 2
    _need(scales, torch.uint8, "scales", (n, kdim // 32))
    out = torch.empty((n, kdim), dtype=torch.bfloat16, device=codes.device)
    check(lib.moe_dequant_bf16(n, kdim, _ptr(codes), _ptr(scales), _ptr(out), _stream()))
    return out


def moe_mx_quantize(x):
    rows, cols = x.shape
    _need(x, None, "x")
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    check(lib.moe_mx_quantize(rows, cols, _ptr(x), DT[x.dtype], _ptr(codes), _ptr(scales), _stream()))
    return codes, scales
