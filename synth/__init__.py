"""Seeded synthetic inputs for the routed MoE layer.

This module is shared by the float64 oracle side (tests, the CPU baseline) and the GPU
side (tests, bench).  It holds none of the layer's arithmetic: it only draws random
bytes and Gaussian values rounded to bf16, from a counter-based generator, so that any
single tensor or expert can be regenerated on its own.

Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014) used in counter mode: word i of a stream with key K is
mix64(K + (i + 1) * 0x9E3779B97F4A7C15).  A stream key folds (seed, workload tag, tensor
tag, expert, instance, batch) through mix64.

Two implementations of the byte streams exist: NumPy on the host (`*_np`) and torch
integer ops on a device (`*_torch`), used only to fill the multi-GB expert tensors in
device memory.  They are bit-identical (integer arithmetic modulo 2^64 only); the
tests check that.  Gaussian draws are host-only.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .configs import CONFIGS, LayerConfig, get  # noqa: F401

M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
C1 = 0xBF58476D1CE4E5B9
C2 = 0x94D049BB133111EB

# tensor tags
T_X, T_WR, T_WSG, T_LBIAS, T_SBIAS = 1, 2, 3, 4, 5
T_GATE_C, T_GATE_S, T_UP_C, T_UP_S, T_DOWN_C, T_DOWN_S = 10, 11, 12, 13, 14, 15
T_PD, T_PU = 20, 21
SHARED = 0xFFFFFFFF  # expert index used for the shared expert's streams


def mix64(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * C1) & M64
    z = ((z ^ (z >> 27)) * C2) & M64
    return z ^ (z >> 31)


def stream_key(seed: int, *parts: int) -> int:
    k = mix64(seed + GOLDEN)
    for p in parts:
        k = mix64(k ^ (p & M64))
    return k


# ---------------------------------------------------------------- host (NumPy) streams

def words_np(key: int, n: int, start: int = 0) -> np.ndarray:
    """Words start..start+n-1 of stream `key` as uint64."""
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + i * np.uint64(GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(C1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(C2)
    return z ^ (z >> np.uint64(31))


def bytes_np(key: int, n: int) -> np.ndarray:
    """n uniform bytes: word i supplies bytes 8i..8i+7, least significant first."""
    w = words_np(key, (n + 7) // 8)
    return w.astype("<u8").view(np.uint8)[:n].copy()


def small_uniform_np(key: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi]: lo + ((w >> 32) * (hi - lo + 1)) >> 32."""
    w = words_np(key, n)
    span = np.uint64(hi - lo + 1)
    return (np.int64(lo) + ((w >> np.uint64(32)) * span >> np.uint64(32)).astype(np.int64))


def normal_np(key: int, n: int) -> np.ndarray:
    """n standard normals (Box-Muller on word pairs), float64."""
    w = words_np(key, 2 * n).reshape(n, 2)
    u1 = ((w[:, 0] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = ((w[:, 1] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> float32 (round to nearest even) -> bf16 bits (round to nearest even), uint16."""
    f = np.asarray(v, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    rounded = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_normal_np(key: int, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    return to_bf16_bits(std * normal_np(key, n)).reshape(shape)


def fp8_codes_np(key: int, n: int) -> np.ndarray:
    """E4M3 code bytes uniform over the 254 non-NaN bytes (0x7F and 0xFF skipped)."""
    idx = small_uniform_np(key, n, 0, 253)
    return (idx + (idx >= 127)).astype(np.uint8)


# ---------------------------------------------------------------- device (torch) twin

def _i64(v: int) -> int:
    v &= M64
    return v - (1 << 64) if v >= (1 << 63) else v


def _srl(z, s: int):
    """Logical right shift of int64 tensors holding uint64 bit patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def words_torch(keys, n: int, device):
    """Words 0..n-1 for each key in `keys` (list of ints) -> int64 tensor [len(keys)][n]."""
    import torch
    kt = torch.tensor([_i64(k) for k in keys], dtype=torch.int64, device=device).view(-1, 1)
    i = torch.arange(1, n + 1, dtype=torch.int64, device=device).view(1, -1)
    z = kt + i * _i64(GOLDEN)
    z = (z ^ _srl(z, 30)) * _i64(C1)
    z = (z ^ _srl(z, 27)) * _i64(C2)
    return z ^ _srl(z, 31)


def bytes_torch(keys, n: int, device):
    """bytes_np(key, n) for each key -> uint8 tensor [len(keys)][n] on `device`."""
    import torch
    nw = (n + 7) // 8
    w = words_torch(keys, nw, device)
    return w.view(torch.uint8).view(len(keys), nw * 8)[:, :n]


def small_uniform_torch(keys, n: int, lo: int, hi: int, device):
    w = words_torch(keys, n, device)
    return lo + ((_srl(w, 32) * (hi - lo + 1)) >> 32)


# ---------------------------------------------------------------- layer inputs

@dataclass
class ExpertSet:
    """One matrix set (gate, up, down) for E experts, in the storage layout.

    MXFP4: codes [E][N][K/2] uint8 (low nibble = even k), scales [E][N][K/32] uint8 (E8M0).
    FP8:   codes [E][N][K] uint8 (E4M3), scales [E][N/128][K/128] float32.
    gate/up have N = I, K = d_model; down has N = d_model, K = I.
    """
    fmt: str
    d_model: int
    d_ff: int
    gate: object
    gate_s: object
    up: object
    up_s: object
    down: object
    down_s: object


def _mat_shapes(fmt: str, N: int, K: int):
    if fmt == "mxfp4":
        return (N, K // 2), (N, K // 32)
    return (N, K), (N // 128, K // 128)


def _fill_matrix_np(cfg: LayerConfig, seed: int, tag_c: int, tag_s: int, expert: int, N: int, K: int, inst: int):
    cshape, sshape = _mat_shapes(cfg.wfmt, N, K)
    kc = stream_key(seed, cfg.wtag, tag_c, expert, inst)
    ks = stream_key(seed, cfg.wtag, tag_s, expert, inst)
    nc, ns = int(np.prod(cshape)), int(np.prod(sshape))
    if cfg.wfmt == "mxfp4":
        codes = bytes_np(kc, nc).reshape(cshape)
        scales = small_uniform_np(ks, ns, cfg.scale_lo, cfg.scale_hi).astype(np.uint8).reshape(sshape)
    else:
        codes = fp8_codes_np(kc, nc).reshape(cshape)
        u = small_uniform_np(ks, ns, cfg.fp8_exp_lo, cfg.fp8_exp_hi)
        scales = np.ldexp(np.ones(ns, np.float32), u.astype(np.int32)).astype(np.float32).reshape(sshape)
    return codes, scales


def expert_np(cfg: LayerConfig, e: int, seed: int = 0, inst: int = 0) -> ExpertSet:
    """One routed expert (e in [0, E)) or the shared expert (e == SHARED), host arrays with E = 1."""
    if e == SHARED:
        K, I = cfg.shared_K, cfg.shared_I
    else:
        K, I = cfg.d_model, cfg.I
    g, gs = _fill_matrix_np(cfg, seed, T_GATE_C, T_GATE_S, e, I, K, inst)
    u, us = _fill_matrix_np(cfg, seed, T_UP_C, T_UP_S, e, I, K, inst)
    d, ds = _fill_matrix_np(cfg, seed, T_DOWN_C, T_DOWN_S, e, K, I, inst)
    ex = lambda a: a[None]
    return ExpertSet(cfg.wfmt, K, I, ex(g), ex(gs), ex(u), ex(us), ex(d), ex(ds))


def experts_np(cfg: LayerConfig, seed: int = 0, inst: int = 0, experts=None) -> ExpertSet:
    """Routed experts (all, or the listed ids) stacked along axis 0, host arrays."""
    ids = range(cfg.E) if experts is None else experts
    parts = [expert_np(cfg, e, seed, inst) for e in ids]
    cat = lambda name: np.concatenate([getattr(p, name) for p in parts], axis=0)
    return ExpertSet(cfg.wfmt, cfg.d_model, cfg.I, cat("gate"), cat("gate_s"), cat("up"), cat("up_s"),
                     cat("down"), cat("down_s"))


def _fill_matrix_torch(cfg: LayerConfig, seed: int, tag_c: int, tag_s: int, experts, N: int, K: int,
                       inst: int, codes_out, scales_out, chunk: int):
    import torch
    cshape, sshape = _mat_shapes(cfg.wfmt, N, K)
    nc, ns = int(np.prod(cshape)), int(np.prod(sshape))
    for c0 in range(0, len(experts), chunk):
        ids = experts[c0:c0 + chunk]
        kc = [stream_key(seed, cfg.wtag, tag_c, e, inst) for e in ids]
        ks = [stream_key(seed, cfg.wtag, tag_s, e, inst) for e in ids]
        dst_c = codes_out[c0:c0 + len(ids)]
        dst_s = scales_out[c0:c0 + len(ids)]
        if cfg.wfmt == "mxfp4":
            dst_c.copy_(bytes_torch(kc, nc, codes_out.device).reshape(dst_c.shape))
            s = small_uniform_torch(ks, ns, cfg.scale_lo, cfg.scale_hi, codes_out.device)
            dst_s.copy_(s.to(torch.uint8).reshape(dst_s.shape))
        else:
            idx = small_uniform_torch(kc, nc, 0, 253, codes_out.device)
            dst_c.copy_((idx + (idx >= 127).to(torch.int64)).to(torch.uint8).reshape(dst_c.shape))
            u = small_uniform_torch(ks, ns, cfg.fp8_exp_lo, cfg.fp8_exp_hi, codes_out.device)
            dst_s.copy_(torch.ldexp(torch.ones_like(u, dtype=torch.float32), u.to(torch.int32))
                        .reshape(dst_s.shape))
        del dst_c, dst_s


def experts_torch(cfg: LayerConfig, device, seed: int = 0, inst: int = 0, shared: bool = False,
                  chunk: int = 16) -> ExpertSet:
    """All routed experts (or the shared expert) generated directly in device memory."""
    import torch
    if shared:
        ids, K, I = [SHARED], cfg.shared_K, cfg.shared_I
    else:
        ids, K, I = list(range(cfg.E)), cfg.d_model, cfg.I
    n = len(ids)
    sdt = torch.uint8 if cfg.wfmt == "mxfp4" else torch.float32
    out = {}
    for name, tc, ts, N, KK in (("gate", T_GATE_C, T_GATE_S, I, K), ("up", T_UP_C, T_UP_S, I, K),
                                ("down", T_DOWN_C, T_DOWN_S, K, I)):
        cshape, sshape = _mat_shapes(cfg.wfmt, N, KK)
        c = torch.empty((n,) + cshape, dtype=torch.uint8, device=device)
        s = torch.empty((n,) + sshape, dtype=sdt, device=device)
        _fill_matrix_torch(cfg, seed, tc, ts, ids, N, KK, inst, c, s, chunk)
        out[name], out[name + "_s"] = c, s
    return ExpertSet(cfg.wfmt, K, I, out["gate"], out["gate_s"], out["up"], out["up_s"],
                     out["down"], out["down_s"])


@dataclass
class LayerInputs:
    """Host inputs of one layer step except the expert weights (see expert_np / experts_torch)."""
    x: np.ndarray                 # [T][H] bf16 bits (uint16)
    w_router: np.ndarray          # [E][H] bf16 bits
    logit_bias: np.ndarray | None     # [E] float32, added to the logits
    select_bias: np.ndarray | None    # [E] float32, selection only (sigmoid path)
    w_shared_gate: np.ndarray | None  # [H] bf16 bits
    p_down: np.ndarray | None     # [L][H] bf16 bits (LatentMoE)
    p_up: np.ndarray | None       # [H][L] bf16 bits


def tokens_np(cfg: LayerConfig, seed: int = 0, inst: int = 0, batch: int = 0) -> np.ndarray:
    return bf16_normal_np(stream_key(seed, cfg.tag, T_X, 0, inst, batch), (cfg.T, cfg.H), 1.0)


def layer_inputs_np(cfg: LayerConfig, seed: int = 0, inst: int = 0, batch: int = 0) -> LayerInputs:
    key = lambda t, e=0: stream_key(seed, cfg.tag, t, e, inst)
    x = tokens_np(cfg, seed, inst, batch)
    wr = bf16_normal_np(key(T_WR), (cfg.E, cfg.H), cfg.router_std)
    lb = None
    if cfg.logit_bias == "zipf1.1":
        order = np.argsort(words_np(key(T_LBIAS), cfg.E), kind="stable")
        rank = np.empty(cfg.E, np.int64)
        rank[order] = np.arange(1, cfg.E + 1)
        lb = (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)
    elif cfg.logit_bias == "hot10":
        order = np.argsort(words_np(key(T_LBIAS), cfg.E), kind="stable")
        lb = np.zeros(cfg.E, np.float32)
        lb[order[:10]] = 100.0
    sb = None
    if cfg.select_bias_std > 0:
        sb = (cfg.select_bias_std * normal_np(key(T_SBIAS), cfg.E)).astype(np.float32)
    wsg = bf16_normal_np(key(T_WSG), (cfg.H,), 0.02) if cfg.shared == "gated" else None
    pd = pu = None
    if cfg.latent:
        pd = bf16_normal_np(key(T_PD), (cfg.latent, cfg.H), 0.02)
        pu = bf16_normal_np(key(T_PU), (cfg.H, cfg.latent), 0.02)
    return LayerInputs(x, wr, lb, sb, wsg, pd, pu)
