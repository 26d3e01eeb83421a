"""One routed MoE layer step composed from the C-ABI calls.

route -> permute -> routed experts (moe_expert_ffn) -> shared expert (moe_expert_ffn,
identity form) -> combine; LatentMoE layers add moe_dense_bf16 before the routed experts
and after the combine (Kimi K3 article, architecture section).  Decode-sized batches use
the fused calls instead: route+permute, routed and shared gate/up in one launch, down and
combine in one launch.  Every step runs in the
HIP library; this module only wires buffers.  All buffers for a token count are
allocated once, so a step enqueues kernels and allocates nothing.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


@dataclass
class LayerWeights:
    """Device tensors of one layer (see moe.h for layouts)."""
    score: str
    k: int
    renormalize: bool
    routed_scaling: float
    act: str
    w_router: torch.Tensor                 # bf16 [E][H]
    experts: B.ExpertWeights
    logit_bias: torch.Tensor | None = None
    select_bias: torch.Tensor | None = None
    shared: B.ExpertWeights | None = None
    w_shared_gate: torch.Tensor | None = None  # bf16 [H]
    p_down: torch.Tensor | None = None     # bf16 [L][H]
    p_up: torch.Tensor | None = None       # bf16 [H][L]
    n_group: int = 1                       # group-limited selection (1: none)
    topk_group: int = 1

    @property
    def H(self):
        return self.w_router.shape[1]

    @property
    def E(self):
        return self.w_router.shape[0]


# LDS a down-combine workgroup may hold: per slot (k, +1 with a shared expert) the h row
# in 4 * roundup(d_ff, 256) bytes and a table of 128 floats (the library's own rule)
FUSED_LDS_LIMIT = 150 * 1024


def down_combine_lds(k: int, shared: bool, d_ff: int) -> int:
    s = k + (1 if shared else 0)
    return s * 4 * ((d_ff + 255) // 256 * 256) + s * 128 * 4


def fuses(w: LayerWeights, T: int) -> bool:
    """Whether a step of T tokens takes the fused decode calls: decode-sized batches
    (T <= 4) with FLOAT activations and no latent projections, a shared expert (if any)
    of the routed format and widths, and k + 1 rows of d_ff within the LDS limit."""
    ex, sh = w.experts, w.shared
    return (w.act == "float" and w.p_down is None and w.p_up is None and 1 <= T <= 4
            and (sh is None or (sh.fmt == ex.fmt and sh.d_model == ex.d_model and sh.d_ff == ex.d_ff))
            and down_combine_lds(w.k, sh is not None, ex.d_ff) <= FUSED_LDS_LIMIT)


class MoELayer:
    def __init__(self, w: LayerWeights, T: int, device):
        self.w, self.T, self.dev = w, T, device
        E, H, k = w.E, w.H, w.k
        L, I = w.experts.d_model, w.experts.d_ff
        f32, i32 = torch.float32, torch.int32
        e = lambda *s, dt=f32: torch.empty(s, dtype=dt, device=device)
        # Decode-sized batches: the shared expert joins the routed gate/up launch and the
        # down product writes the combined output directly (moe_expert_gateup_shared,
        # moe_expert_down_combine), so y_rows and y_shared never exist.
        self.fused = fuses(w, T)
        sh = w.shared
        self.ids, self.topk_w = e(T, k, dt=i32), e(T, k)
        self.sg = e(T) if w.w_shared_gate is not None else None
        self.offs, self.sp, self.p2r = e(E + 1, dt=i32), e(T * k, dt=i32), e(T * k, dt=i32)
        self.x_lat = e(T, L) if w.p_down is not None else None
        self.y_rows = None if self.fused else e(T * k, L)
        self.y_s = e(T, H) if (sh is not None and not self.fused) else None
        self.z = e(T, L) if w.p_up is not None else None
        self.out = e(T, H)
        self.ws_route = B._workspace(B.moe_route_workspace(T, H, E, k, w.score), device)
        self.ws_ffn = B._workspace(B.moe_expert_ffn_workspace(w.experts, w.act, T, k), device)
        self.ws_sh = (B._workspace(B.moe_expert_ffn_workspace(sh, w.act, T, 1), device)
                      if (sh is not None and not self.fused) else None)
        # h rows of the staged form (gate/up and down as separate calls) and the fused form
        self.h = e(T * k, I)
        self.hq = e(T * k, I // 2, dt=torch.uint8) if w.act == "mxfp4" else None
        self.hs = e(T * k, I // 32, dt=torch.uint8) if w.act == "mxfp4" else None
        self.ws_gu = B._workspace(B.moe_expert_gateup_workspace(w.experts, w.act, T, k), device)
        self.h_sh = e(T, I) if (self.fused and sh is not None) else None
        # otherwise the shared expert does not depend on routing: it runs on a second stream,
        # joined before the combine, so it overlaps router, permutation and routed experts
        self.side = torch.cuda.Stream(device=device) if (w.shared is not None and not self.fused) else None

    def forward(self, x, mark=None):
        """One layer step on tokens x (bf16 [T][H]); returns the float32 output buffer.

        With `mark`, the routed experts run as two calls (gate/up, then down; the fused
        form always does) and mark("gateup_begin") / mark("gateup_end") are called around
        the gate/up call, so a caller can record events on the stream around that kernel."""
        w = self.w
        if self.fused:
            B.moe_route_permute(x, w.w_router, w.k, w.score, w.renormalize, w.routed_scaling, w.logit_bias,
                                w.select_bias, w.w_shared_gate,
                                out=(self.ids, self.topk_w, self.sg, self.offs, self.sp, self.p2r), ws=self.ws_route,
                                n_group=w.n_group, topk_group=w.topk_group)
            if mark is not None:
                mark("gateup_begin")
            B.moe_expert_gateup_shared(w.experts, w.shared, x, w.k, self.offs, self.sp, out=(self.h, self.h_sh))
            if mark is not None:
                mark("gateup_end")
            B.moe_expert_down_combine(w.experts, w.shared, self.h, self.h_sh, self.ids, self.topk_w, self.p2r,
                                      self.sg, out=self.out)
            return self.out
        if w.shared is not None:
            cur = torch.cuda.current_stream()
            self.side.wait_stream(cur)
            with torch.cuda.stream(self.side):
                B.moe_expert_ffn(w.shared, x, w.act, 1, None, None, out=self.y_s, ws=self.ws_sh)
        B.moe_route_permute(x, w.w_router, w.k, w.score, w.renormalize, w.routed_scaling, w.logit_bias,
                            w.select_bias, w.w_shared_gate,
                            out=(self.ids, self.topk_w, self.sg, self.offs, self.sp, self.p2r), ws=self.ws_route,
                            n_group=w.n_group, topk_group=w.topk_group)
        xe = x
        if w.p_down is not None:
            xe = B.moe_dense_bf16(x, w.p_down, out=self.x_lat)
        if mark is None:
            B.moe_expert_ffn(w.experts, xe, w.act, w.k, self.offs, self.sp, out=self.y_rows, ws=self.ws_ffn)
        else:
            mark("gateup_begin")
            h = self.h if w.act == "float" else None
            B.moe_expert_gateup(w.experts, xe, w.act, w.k, self.offs, self.sp, out=(h, self.hq, self.hs),
                                ws=self.ws_gu)
            mark("gateup_end")
            B.moe_expert_down(w.experts, self.T, w.act, w.k, self.offs, self.h, self.hq, self.hs, out=self.y_rows)
        if w.shared is not None:
            cur.wait_stream(self.side)
        if w.p_up is not None:
            B.moe_combine(self.y_rows, self.p2r, self.topk_w, out=self.z)
            B.moe_dense_bf16(self.z, w.p_up, residual=self.y_s, out=self.out)
        else:
            B.moe_combine(self.y_rows, self.p2r, self.topk_w, self.y_s, self.sg, out=self.out)
        return self.out
