#!/usr/bin/env python3
"""Throughput of one routed MoE layer step on one MI355X, as one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one pass of the whole layer (router, top-k, permutation, routed experts,
shared expert, combine; LatentMoE projections where the workload has them) over one
batch of seeded synthetic tokens, with all weights resident in HBM.  Steps rotate over
several independently generated layer instances and token batches, so no step finds the
previous step's weights in the 256 MB last-level cache.  Each step is captured once as a
HIP graph; the timed region replays K graphs back to back between two events.

Also reported:
  roofline      the routed gate/up dequant-GEMV (the kernel that moves the most bytes):
                algorithmic bytes per launch / its average duration, measured with events
                on the launch stream in a second, instrumented pass of the same steps;
  cpu_baseline  the float64 oracle on a bounded sample of the same workload, on the
                host cores (a baseline only).
  traffic       HBM bytes per launch of that kernel from the hardware counters (FETCH_SIZE,
                WRITE_SIZE), each scaled by what the same counter reads for a 1 GiB copy, taken
                from profiles/traffic_<workload>.json when its sources still match the library's;
                otherwise null.  Collect with two counter passes over `--traffic-run`:
                  rocprofv3 --pmc FETCH_SIZE -d D1 -o run --output-format csv -- python3 bench.py --traffic-run
                  rocprofv3 --pmc WRITE_SIZE -d D2 -o run --output-format csv -- python3 bench.py --traffic-run
                  python3 bench.py --traffic-parse D1 D2
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "mxfp4_routed_expert_amd", "csrc")
PEAK_HBM_GBPS = 8000.0
PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "bf16": 2500.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg, D, fused=False):
    """Algorithmic bytes and flops of one step at D distinct routed experts touched, for the
    layer and for the routed gate/up kernel (weights of touched experts, router, shared
    expert and projections once, activations in and out once).  `fused`: the gate/up launch
    also computes the shared expert's gate/up (its weights and h rows count there too)."""
    K, I, H, T, k = cfg.d_model, cfg.I, cfg.H, cfg.T, cfg.k
    P = T * k
    if cfg.wfmt == "mxfp4":
        gu_w = 2 * I * K * 17 // 32
    else:
        gu_w = 2 * I * K + 2 * (I // 128) * (K // 128) * 4
    shared_b = cfg.expert_bytes(cfg.shared_K, cfg.shared_I) if cfg.shared else 0
    router_b = cfg.E * H * 2 + (H * 2 if cfg.shared == "gated" else 0)
    router_b += cfg.E * 4 * ((1 if cfg.logit_bias else 0) + (1 if cfg.select_bias_std else 0))
    proj_b = 2 * cfg.latent * H * 2 if cfg.latent else 0
    layer_bytes = D * cfg.expert_bytes() + shared_b + router_b + proj_b + T * H * 2 + T * H * 4
    flops = 2 * P * 3 * K * I + 2 * T * cfg.E * H
    if cfg.shared:
        flops += 2 * T * 3 * cfg.shared_K * cfg.shared_I
    if cfg.latent:
        flops += 2 * T * 2 * cfg.latent * H
    if cfg.act == "mxfp4":
        gu_in, gu_out = T * K * 17 // 32, P * I * 17 // 32
    else:
        gu_in, gu_out = T * K * (4 if cfg.latent else 2), P * I * 4
    gu_bytes, gu_flops = D * gu_w + gu_in + gu_out, 2 * P * 2 * K * I
    if fused and cfg.shared:
        gu_bytes += cfg.expert_bytes(cfg.shared_K, cfg.shared_I) * 2 // 3 + T * cfg.shared_I * 4
        gu_flops += 2 * T * 2 * cfg.shared_K * cfg.shared_I
    return dict(layer_bytes=layer_bytes, layer_flops=flops, gu_bytes=gu_bytes, gu_flops=gu_flops)


def cpu_baseline(cfg, steps):
    """The float64 oracle on `steps` layer steps (token batches 0..steps-1 of instance 0)."""
    import synth
    from oracle import layer as OL
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    limiter = threadpool_limits(cores) if threadpool_limits else None
    total = 0.0
    cache = {}
    for b in range(steps):
        inp = synth.layer_inputs_np(cfg, 0, 0, b)
        r = OL.route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling, inp.logit_bias,
                     inp.select_bias, inp.w_shared_gate if cfg.shared == "gated" else None)
        for e in set(int(v) for v in r.ids.reshape(-1)):        # generation is not timed
            if e not in cache:
                cache[e] = synth.expert_np(cfg, e)
        if cfg.shared and "s" not in cache:
            cache["s"] = synth.expert_np(cfg, synth.SHARED)
        t0 = time.perf_counter()
        OL.layer(cfg, inp, lambda e: cache[e], lambda: cache["s"])
        total += time.perf_counter() - t0
    # threads the oracle could use: the BLAS pools (NumPy's elementwise work is single-threaded)
    used = max((i.get("num_threads", 1) for i in threadpool_info()), default=1) if threadpool_info else 1
    if limiter is not None:
        limiter.restore_original_limits()
    return dict(value=steps * cfg.T / total, unit="tokens/s", cores=used, kind="oracle",
                sample=f"{steps} step(s) of {cfg.name} ({steps * cfg.T} tokens), float64 NumPy, "
                       f"{total:.1f} s; expert bytes generated outside the timed region")


def dominant_kernel(cfg):
    """Name pattern (as rocprofv3 reports it) of the routed gate/up kernel of a workload."""
    if cfg.act == "mxfp4" and cfg.T >= 64:
        return r"mxgemm_kernel<true, true>"
    if cfg.wfmt == "mxfp4" and cfg.T >= 64:
        return r"fgemm_pair_kernel<\w+, true>"
    return r"gemv_kernel<\d+, \d+, \d+, true, true>"


def source_digest():
    """sha256 over the library sources: counter figures are void once any of them changes."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def traffic_file(cfg):
    return os.path.join(HERE, "profiles", f"traffic_{cfg.name}.json")


def load_traffic(cfg):
    try:
        with open(traffic_file(cfg)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t["traffic_bytes_per_launch"] if t.get("source_sha256") == source_digest() else None


def parse_traffic(cfg, fetch_dir, write_dir):
    """Counter passes -> profiles/traffic_<workload>.json (bytes per launch of the kernel)."""
    import csv
    import glob
    import re

    def per_dispatch(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += list(csv.DictReader(open(f)))
        pat = re.compile(dominant_kernel(cfg))
        kern = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter and pat.search(r["Kernel_Name"])]
        cal = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter and "neg_kernel" in r["Kernel_Name"]]
        if not kern or not cal:
            raise SystemExit(f"no {counter} rows for the kernel or the calibration copy in {d}")
        return sum(kern) / len(kern), len(kern), max(cal)
    f_k, nf, f_c = per_dispatch(fetch_dir, "FETCH_SIZE")
    w_k, nw, w_c = per_dispatch(write_dir, "WRITE_SIZE")
    gib = float(1 << 30)
    ff, fw = gib / (f_c * 1024.0), gib / (w_c * 1024.0)
    res = {"workload": cfg.name, "kernel": dominant_kernel(cfg), "source_sha256": source_digest(),
           "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k, "dispatches": [nf, nw],
           "calibration": "torch.neg of a 1 GiB float64 tensor (1 GiB read, 1 GiB written)",
           "calib_fetch_kib": f_c, "calib_write_kib": w_c, "fetch_factor": ff, "write_factor": fw,
           "traffic_bytes_per_launch": int(f_k * 1024 * ff + w_k * 1024 * fw),
           "commands": [f"rocprofv3 --pmc FETCH_SIZE -d D1 -o run --output-format csv -- python3 bench.py --config {cfg.name} --traffic-run",
                        f"rocprofv3 --pmc WRITE_SIZE -d D2 -o run --output-format csv -- python3 bench.py --config {cfg.name} --traffic-run",
                        f"python3 bench.py --config {cfg.name} --traffic-parse D1 D2"]}
    os.makedirs(os.path.dirname(traffic_file(cfg)), exist_ok=True)
    with open(traffic_file(cfg), "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen38max_decode")
    ap.add_argument("--instances", type=int, default=4, help="independent layer instances rotated over")
    ap.add_argument("--batches", type=int, default=16, help="token batches rotated over")
    ap.add_argument("--cpu-steps", type=int, default=3, help="oracle steps for the CPU baseline (0: skip)")
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly instead of graph replays")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--traffic-run", action="store_true",
                    help="run a few steps and a 1 GiB calibration copy, untimed (for counter passes)")
    ap.add_argument("--traffic-parse", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two counter passes into profiles/traffic_<workload>.json")
    args = ap.parse_args()
    if args.traffic_parse:
        import synth
        parse_traffic(synth.get(args.config), *args.traffic_parse)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from synth import device as sdev
    import mxfp4_routed_expert_amd as M

    cfg = synth.get(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R, NB = max(1, args.instances), max(1, args.batches)
    log(f"[bench] {cfg.name}: building {R} layer instance(s)")
    layers = []
    for r in range(R):
        t, _ = sdev.layer_tensors(cfg, dev, 0, r)
        w = M.LayerWeights(score=cfg.score, k=cfg.k, renormalize=cfg.renormalize, routed_scaling=cfg.routed_scaling,
                           act=cfg.act, w_router=t["w_router"], experts=M.ExpertWeights.from_arrays(t["experts"]),
                           logit_bias=t["logit_bias"], select_bias=t["select_bias"],
                           shared=M.ExpertWeights.from_arrays(t["shared"]) if t["shared"] is not None else None,
                           w_shared_gate=t["w_shared_gate"] if cfg.shared == "gated" else None,
                           p_down=t["p_down"], p_up=t["p_up"])
        layers.append(M.MoELayer(w, cfg.T, dev))
    xs = [sdev.token_batch(cfg, dev, 0, 0, b) for b in range(NB)]
    S = max(R, NB)
    slot = lambda j: (layers[j % R], xs[j % NB])
    torch.cuda.synchronize()

    # eager warm-up of every slot (also what the graphs capture)
    for j in range(S):
        L, x = slot(j)
        L.forward(x)
    torch.cuda.synchronize()
    graphs = None
    if not args.no_graph:
        log("[bench] capturing one graph per step slot")
        graphs = []
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for j in range(S):
                g = torch.cuda.CUDAGraph()
                L, x = slot(j)
                with torch.cuda.graph(g, stream=stream):
                    L.forward(x)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()

    def step(s):
        if graphs is not None:
            graphs[s % S].replay()
        else:
            L, x = slot(s)
            L.forward(x)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    if args.traffic_run:
        for s in range(args.steps):
            step(args.warmup + s)
        a = torch.empty(1 << 27, dtype=torch.float64, device=dev).fill_(1.0)
        torch.neg(a)
        torch.cuda.synchronize()
        log("[bench] traffic run done")
        return
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for s in range(args.steps):
        step(args.warmup + s)
    ev1.record()
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.2f} us/step")

    # distinct routed experts touched per slot (read back after a step of that slot)
    D_slot = []
    for j in range(S):
        L, x = slot(j)
        L.forward(x)
        torch.cuda.synchronize()
        offs = L.offs.cpu()
        D_slot.append(int(((offs[1:] - offs[:-1]) > 0).sum()))
    D_steps = [D_slot[(args.warmup + s) % S] for s in range(args.steps)]
    D_mean = sum(D_steps) / len(D_steps)

    # instrumented pass: events around the routed gate/up kernel on its stream.  A block of
    # matrix products is queued first so every step of the pass is enqueued before the GPU
    # reaches it (no host gaps inside the measured intervals).
    a = torch.randn(8192, 8192, device=dev)
    for _ in range(4):
        a = a @ a * 1e-4
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for s in range(args.steps):
        L, x = slot(args.warmup + s)
        pair = marks[s]
        L.forward(x, mark=lambda name, pair=pair: pair[0 if name == "gateup_begin" else 1].record())
    torch.cuda.synchronize()
    gu_ms = [b.elapsed_time(c) for b, c in marks]
    gu_us = 1e3 * sum(gu_ms) / len(gu_ms)
    del a

    fused = layers[0].fused
    alg = [algorithmic(cfg, D, fused) for D in D_steps]
    gu_bytes = sum(x["gu_bytes"] for x in alg) / len(alg)
    gu_flops = sum(x["gu_flops"] for x in alg) / len(alg)
    layer_bytes = sum(x["layer_bytes"] for x in alg) / len(alg)
    layer_flops = sum(x["layer_flops"] for x in alg) / len(alg)
    step_s = ms_per_step * 1e-3
    peak_flops = PEAK_TFLOPS["fp4"] if cfg.act == "mxfp4" else (PEAK_TFLOPS["fp8"] if cfg.wfmt != "mxfp4" else
                                                                  PEAK_TFLOPS["bf16"])
    intensity = gu_flops / gu_bytes
    if intensity * PEAK_HBM_GBPS * 1e9 > peak_flops * 1e12:
        achieved = gu_flops / (gu_us * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=peak_flops, unit="TFLOP/s",
                    frac=round(achieved / peak_flops, 4))
    else:
        achieved = gu_bytes / (gu_us * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBPS, 4))
    if cfg.act == "mxfp4" and cfg.T >= 64:
        kname = "routed gate/up grouped GEMM (mxgemm_kernel, FP4 x FP4)"
    elif cfg.wfmt == "mxfp4" and cfg.T >= 64:
        kname = "routed gate/up grouped GEMM (fgemm_pair_kernel, MXFP4 weights decoded to bf16)"
    else:
        kname = "moe::gemv_kernel (routed gate/up" + (" + shared gate/up" if fused and cfg.shared else "") + \
                ", fused SwiGLU)"
    roof.update(traffic=load_traffic(cfg), kernel=kname,
                bytes_per_launch=int(gu_bytes), flops_per_launch=int(gu_flops), avg_launch_us=round(gu_us, 2),
                launches=len(gu_ms))

    cpu = None
    if args.cpu_steps > 0:
        log(f"[bench] CPU baseline: oracle on {args.cpu_steps} step(s)")
        cpu = cpu_baseline(cfg, args.cpu_steps)

    # arithmetic type of the dominant products: bf16 dot products on exactly decoded weights
    # (FLOAT mode), or FP4 x FP4 on the block-scaled MFMA (MX mode); fp32 accumulation
    dtype = "fp4" if cfg.act == "mxfp4" else "bf16"
    arith = {("mxfp4", "float"): "mxfp4 weights decoded exactly to bf16 x bf16 activations, fp32 accumulate",
             ("mxfp4", "mxfp4"): "mxfp4 weights x OCP-MX fp4 activations on the scaled MFMA, fp32 accumulate",
             ("fp8b128", "float"): "fp8 e4m3 weights decoded exactly to bf16 x bf16 activations, fp32 accumulate"
             }[(cfg.wfmt, cfg.act)]
    res = {
        "metric": "MoE layer tokens/s; decode HBM GB/s and prefill TFLOP/s as % roofline",
        "value": round(cfg.T / step_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "d_model": cfg.d_model, "I": cfg.I, "E": cfg.E,
                   "k": cfg.k, "score": cfg.score, "weights": cfg.wfmt, "activations": cfg.act,
                   "shared": cfg.shared, "latent": cfg.latent, "arith": arith, "instances": R, "token_batches": NB,
                   "graphs": graphs is not None, "distinct_experts_per_step": round(D_mean, 2)},
        "layer": {"bytes_per_step": int(layer_bytes), "flops_per_step": int(layer_flops),
                  "GB/s": round(layer_bytes / step_s / 1e9, 1),
                  "hbm_frac": round(layer_bytes / step_s / 1e9 / PEAK_HBM_GBPS, 4),
                  "TFLOP/s": round(layer_flops / step_s / 1e12, 3)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
