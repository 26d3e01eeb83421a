"""One routed MoE layer step composed from the C-ABI calls.

route -> permute -> routed experts (moe_expert_ffn) -> shared expert (moe_expert_ffn,
identity form) -> combine; LatentMoE layers add moe_dense_bf16 before the routed experts
and after the combine (Kimi K3 article, architecture section); a gated shared expert's
output is scaled by its gate before it is added after the up projection.  Decode-sized
LatentMoE steps run the routed down product and the combine into z as one down-combine
launch.  Decode-sized
batches use the fused calls instead, three kernels a step -- the router's logits; the
selection with the routed and shared gate/up in one launch (moe_topk_gateup_shared); down
and combine in one launch -- or, on request, the whole step as one launch
(moe_decode_step).
Every step runs in the HIP library; this module only wires buffers.  All buffers for a token count are allocated once, so a step enqueues kernels and
allocates nothing.
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
# in 4 * roundup(d_ff, 512) bytes and a table of 128 floats (the library's own rule)
FUSED_LDS_LIMIT = 150 * 1024


def down_combine_lds(k: int, shared: bool, d_ff: int) -> int:
    s = k + (1 if shared else 0)
    return s * 4 * ((d_ff + 511) // 512 * 512) + s * 128 * 4


def fuses(w: LayerWeights, T: int) -> bool:
    """Whether a step of T tokens takes the fused decode calls: decode-sized batches
    (T <= 4) with FLOAT activations and no latent projections, a shared expert (if any)
    of the routed format and widths, and k + 1 rows of d_ff within the LDS limit."""
    ex, sh = w.experts, w.shared
    return (w.act == "float" and w.p_down is None and w.p_up is None and 1 <= T <= 4
            and (sh is None or (sh.fmt == ex.fmt and sh.d_model == ex.d_model and sh.d_ff == ex.d_ff))
            and down_combine_lds(w.k, sh is not None, ex.d_ff) <= FUSED_LDS_LIMIT)


class MoELayer:
    def __init__(self, w: LayerWeights, T: int, device, single_launch: bool = False):
        """single_launch: fused decode steps run as one moe_decode_step launch instead of its
        three calls (moe_router_logits, moe_topk_gateup_shared, moe_expert_down_combine); the
        results are the same bits.  The three calls are the default: on MI355X they measure a
        few per cent faster per step than the single launch."""
        self.w, self.T, self.dev = w, T, device
        E, H, k = w.E, w.H, w.k
        L, I = w.experts.d_model, w.experts.d_ff
        f32, i32 = torch.float32, torch.int32
        e = lambda *s, dt=f32: torch.empty(s, dtype=dt, device=device)
        # Decode-sized batches: the shared expert joins the routed gate/up launch and the
        # down product writes the combined output directly (moe_expert_gateup_shared,
        # moe_expert_down_combine), so y_rows and y_shared never exist.
        self.fused = fuses(w, T)
        # decode-sized LatentMoE steps: the routed down product and the combine into z run as
        # one down-combine launch with no shared slot (the shared expert's output is added after
        # the up projection), so y_rows never exists
        self.latent_down_combine = (w.act == "float" and w.p_up is not None and 1 <= T <= 8
                                    and down_combine_lds(w.k, False, w.experts.d_ff) <= FUSED_LDS_LIMIT)
        self.down_combined = self.fused or self.latent_down_combine
        sh = w.shared
        self.ids, self.topk_w = e(T, k, dt=i32), e(T, k)
        self.sg = e(T) if w.w_shared_gate is not None else None
        self.offs, self.sp, self.p2r = e(E + 1, dt=i32), e(T * k, dt=i32), e(T * k, dt=i32)
        self.x_lat = e(T, L) if w.p_down is not None else None
        self.y_rows = None if self.down_combined else e(T * k, L)
        self.y_s = e(T, H) if (sh is not None and not self.fused) else None
        self.z = e(T, L) if w.p_up is not None else None
        # LatentMoE with a gated shared expert: g * y_s is formed by moe_combine with no
        # routed slots (k = 0) before it becomes the residual of the up projection
        self.latent_gate = w.p_up is not None and sh is not None and w.w_shared_gate is not None
        self.y_sg = e(T, H) if self.latent_gate else None
        self.no_rows = e(0, dt=i32)
        self.no_w = e(T, 0)
        self.out = e(T, H)
        self.ws_route = B._workspace(B.moe_route_workspace(T, H, E, k, w.score), device)
        self.logits = e(T, E + (1 if w.w_shared_gate is not None else 0)) if self.fused else None
        self.single = self.fused and single_launch
        self.sync = B.decode_step_sync(device) if self.single else None
        # h rows: the staged form runs gate/up and down as separate calls on these buffers
        # (float32 h in FLOAT mode, MX codes and scales in MXFP4 mode), as does the fused form
        mx = w.act == "mxfp4"
        self.h = e(T * k, I)
        self.hq = e(T * k, I // 2, dt=torch.uint8) if mx else None
        self.hs = e(T * k, I // 32, dt=torch.uint8) if mx else None
        self.ws_gu = B._workspace(B.moe_expert_gateup_workspace(w.experts, w.act, T, k), device)
        staged_sh = sh is not None and not self.fused
        Is = sh.d_ff if sh is not None else 0
        self.h_sh = e(T, Is) if sh is not None else None
        self.hq_sh = e(T, Is // 2, dt=torch.uint8) if (staged_sh and mx) else None
        self.hs_sh = e(T, Is // 32, dt=torch.uint8) if (staged_sh and mx) else None
        self.ws_gu_sh = B._workspace(B.moe_expert_gateup_workspace(sh, w.act, T, 1), device) if staged_sh else None
        # otherwise the shared expert does not depend on routing: it runs on a second stream,
        # joined before the combine, so it overlaps router, permutation and routed experts;
        # so does the latent down-projection, which the routed gate/up waits for
        side = w.shared is not None or w.p_down is not None
        self.side = torch.cuda.Stream(device=device) if (side and not self.fused) else None
        self.lat_ready = torch.cuda.Event() if (w.p_down is not None and not self.fused) else None

    def forward(self, x, mark=None):
        """One layer step on tokens x (bf16 [T][H]); returns the float32 output buffer.

        With `mark`, mark(name) is called on the step's stream before and after the routed
        gate/up call ("gateup_begin", "gateup_end") and the down call ("down_begin",
        "down_end"; the down product with the combine in the fused form), or around the
        single-launch step ("step_begin", "step_end"), so a caller can record events around
        those kernels."""
        w = self.w
        if self.single:
            # the whole step in one launch (the three calls below, same results)
            if mark is not None:
                mark("step_begin")
            B.moe_decode_step(x, w.w_router, w.k, w.experts, w.shared, w.score, w.renormalize, w.routed_scaling,
                              w.logit_bias, w.select_bias, w.w_shared_gate, sync=self.sync,
                              out=(self.logits, self.ids, self.topk_w, self.sg, self.offs, self.sp, self.p2r, self.h,
                                   self.h_sh, self.out), n_group=w.n_group, topk_group=w.topk_group)
            if mark is not None:
                mark("step_end")
            return self.out
        if self.fused:
            # three kernels: the router's logits, one gate/up launch that routes in its
            # prologue (the routing results land in the same buffers as moe_route_permute's),
            # and the down product with the combine
            B.moe_router_logits(x, w.w_router, w.k, w.score, w.w_shared_gate, out=self.logits, ws=self.ws_route,
                                n_group=w.n_group, topk_group=w.topk_group)
            if mark is not None:
                mark("gateup_begin")
            B.moe_topk_gateup_shared(self.logits, x, w.k, w.experts, w.shared, w.score, w.renormalize,
                                     w.routed_scaling, w.logit_bias, w.select_bias, w.w_shared_gate is not None,
                                     out=(self.ids, self.topk_w, self.sg, self.offs, self.sp, self.p2r, self.h,
                                          self.h_sh), n_group=w.n_group, topk_group=w.topk_group)
            if mark is not None:
                mark("gateup_end")
            if mark is not None:
                mark("down_begin")
            B.moe_expert_down_combine(w.experts, w.shared, self.h, self.h_sh, self.ids, self.topk_w, self.p2r,
                                      self.sg, out=self.out)
            if mark is not None:
                mark("down_end")
            return self.out
        mx = w.act == "mxfp4"
        cur = torch.cuda.current_stream()
        xe = x
        if self.side is not None:
            self.side.wait_stream(cur)
            with torch.cuda.stream(self.side):
                if w.p_down is not None:
                    xe = B.moe_dense_bf16(x, w.p_down, out=self.x_lat)
                    self.lat_ready.record(self.side)
                if w.shared is not None:
                    B.moe_expert_gateup(w.shared, x, w.act, 1, None, None,
                                        out=(None if mx else self.h_sh, self.hq_sh, self.hs_sh), ws=self.ws_gu_sh)
                    B.moe_expert_down(w.shared, self.T, w.act, 1, None, self.h_sh, self.hq_sh, self.hs_sh,
                                      out=self.y_s)
        B.moe_route_permute(x, w.w_router, w.k, w.score, w.renormalize, w.routed_scaling, w.logit_bias,
                            w.select_bias, w.w_shared_gate,
                            out=(self.ids, self.topk_w, self.sg, self.offs, self.sp, self.p2r), ws=self.ws_route,
                            n_group=w.n_group, topk_group=w.topk_group)
        if w.p_down is not None:
            cur.wait_event(self.lat_ready)
        if mark is not None:
            mark("gateup_begin")
        B.moe_expert_gateup(w.experts, xe, w.act, w.k, self.offs, self.sp,
                            out=(None if mx else self.h, self.hq, self.hs), ws=self.ws_gu)
        if mark is not None:
            mark("gateup_end")
        if mark is not None:
            mark("down_begin")
        if self.latent_down_combine:
            B.moe_expert_down_combine(w.experts, None, self.h, None, self.ids, self.topk_w, self.p2r, out=self.z)
        else:
            B.moe_expert_down(w.experts, self.T, w.act, w.k, self.offs, self.h, self.hq, self.hs, out=self.y_rows)
        if mark is not None:
            mark("down_end")
        if self.side is not None:
            cur.wait_stream(self.side)
        if w.p_up is not None:
            if not self.latent_down_combine:
                B.moe_combine(self.y_rows, self.p2r, self.topk_w, out=self.z)
            res = self.y_s
            if self.latent_gate:
                res = B.moe_combine(None, self.no_rows, self.no_w, self.y_s, self.sg, out=self.y_sg)
            B.moe_dense_bf16(self.z, w.p_up, residual=res, out=self.out)
        else:
            B.moe_combine(self.y_rows, self.p2r, self.topk_w, self.y_s, self.sg, out=self.out)
        return self.out
