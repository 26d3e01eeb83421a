#!/usr/bin/env python3
"""Throughput of the routed MoE layer on one MI355X, as one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-prefill]

A step is one pass of the whole layer (router, top-k, permutation, routed experts,
shared expert, combine; LatentMoE projections where the workload has them) over one
batch of seeded synthetic tokens, with all weights resident in HBM.  Steps rotate over
four independently generated layer instances and sixteen token batches, so no step finds
the previous step's weights in the 256 MB last-level cache.  The sixteen step slots are
captured in order as one HIP graph (a model's forward pass holds its layers in one graph),
and each slot also as a graph of its own; the timed region replays K steps back to back
between two events -- whole sixteen-step graphs, then single-step graphs for the rest.
The same K steps with one graph launch per step are reported beside it
(`ms_per_step_one_graph_per_step`, with the median, p10 and p90 of the per-step times).

The headline workload (`value`, `ms_per_step`) is the one-token decode layer.  By default
the same run also times the two 512-token prefill workloads on the same expert instances
(the weights are shared: no extra memory): the compute-bound slice in which every token
goes to the same ten experts, and the Zipf-routed prefill.  They are reported under
`prefill` with their own rooflines.

Per kernel (`kernels`, and `roofline` for the decode gate/up, the kernel that moves the
most bytes): algorithmic bytes or flops per launch / the kernel's mean duration.  The
duration comes from HIP events recorded on the launch stream right before and after each
launch, in an eager pass over the same step slots after the timed region, with the GPU
kept busy so that the events bracket device time only.  rocprofv3 --kernel-trace --stats
summaries of the same command are kept under profiles/.

  traffic       HBM bytes per launch of the decode gate/up kernel from the hardware counters
                (FETCH_SIZE, WRITE_SIZE), each scaled by what the same counter reads for a 1 GiB
                copy, taken from profiles/traffic_<workload>.json when its sources still match the
                library's; otherwise null.  Collect with two counter passes over `--traffic-run`:
                  rocprofv3 --pmc FETCH_SIZE -d D1 -o run --output-format csv -- python3 bench.py --traffic-run
                  rocprofv3 --pmc WRITE_SIZE -d D2 -o run --output-format csv -- python3 bench.py --traffic-run
                  python3 bench.py --traffic-parse D1 D2
  cpu_baseline  the float64 oracle on a bounded sample of the decode workload on the host cores,
                plus one-thread times of the small layer and of one decode step (a baseline only).
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
PREFILL_DEFAULT = ("qwen38max_prefill_hot", "qwen38max_prefill")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _mx_bytes(values):
    return values * 17 // 32


def algorithmic(cfg, D, fused=False):
    """Algorithmic bytes and flops of one step at D distinct routed experts touched, for the
    layer and for the routed gate/up launch (weights of touched experts, router, shared
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
        gu_in, gu_out = _mx_bytes(T * K), _mx_bytes(P * I)
    else:
        gu_in, gu_out = T * K * (4 if cfg.latent else 2), P * I * 4
    gu_bytes, gu_flops = D * gu_w + gu_in + gu_out, 2 * P * 2 * K * I
    if fused and cfg.shared:
        gu_bytes += cfg.expert_bytes(cfg.shared_K, cfg.shared_I) * 2 // 3 + T * cfg.shared_I * 4
        gu_flops += 2 * T * 2 * cfg.shared_K * cfg.shared_I
    return dict(layer_bytes=layer_bytes, layer_flops=flops, gu_bytes=gu_bytes, gu_flops=gu_flops)


def down_algorithmic(cfg, D, fused=False, combined=None):
    """Algorithmic bytes and flops of the routed down launch: the touched experts' down
    weights, h in, the rows out.  `combined` (default: `fused`): the down product with the
    combine, which writes one output row per token; `fused`: that launch also covers the
    shared expert's down rows."""
    K, I, T, k = cfg.d_model, cfg.I, cfg.T, cfg.k
    P = T * k
    w_down = K * I * 17 // 32 if cfg.wfmt == "mxfp4" else K * I + (K // 128) * (I // 128) * 4
    flops = 2 * P * K * I
    if cfg.act == "mxfp4":
        h_in, out = _mx_bytes(P * I), P * K * 4
    else:
        h_in, out = P * I * 4, P * K * 4
    nbytes = D * w_down + h_in + out
    if fused if combined is None else combined:
        out = T * K * 4
        nbytes = D * w_down + h_in + out
        if fused and cfg.shared:
            nbytes += cfg.expert_bytes(cfg.shared_K, cfg.shared_I) // 3 + T * cfg.shared_I * 4
            flops += 2 * T * K * cfg.shared_I
    return dict(bytes=nbytes, flops=flops)


STEP_KERNEL = r"decode_step_kernel<\d+>"


def dominant_kernel(cfg, single=False):
    """Name pattern (as rocprofv3 reports it) of the routed gate/up kernel of a workload, or
    of the single-launch decode step that holds it."""
    if single:
        return STEP_KERNEL
    if cfg.act == "mxfp4" and cfg.T >= 64:
        return r"mxgemm_kernel<true, true, (?:true|false)>"
    if cfg.wfmt == "mxfp4" and cfg.T >= 64:
        return r"fgemm_pair_kernel<\w+, true>"
    if cfg.T <= 8:
        return r"gemv_flat_kernel<\d+, \d+, \d+, true(?:, (?:true|false))?>"
    return r"gemv_kernel<\d+, \d+, \d+, true, true>"


def down_kernel(cfg, fused, combined=None):
    """Name pattern of the routed down kernel of a workload."""
    if fused if combined is None else combined:
        return r"down_combine_mfma_kernel" if cfg.wfmt == "mxfp4" else r"down_combine_kernel"
    if cfg.act == "mxfp4" and cfg.T >= 64:
        return r"mxgemm_kernel<false, true, (?:true|false)>"
    if cfg.wfmt == "mxfp4" and cfg.T >= 64:
        return r"fgemm_down_kernel"
    return r"gemv_\w*kernel<\d+, \d+, \d+, false"


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
    single = False

    def per_dispatch(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += list(csv.DictReader(open(f)))
        pat = re.compile(dominant_kernel(cfg, single))
        kern = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter and pat.search(r["Kernel_Name"])]
        cal = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter and "neg_kernel" in r["Kernel_Name"]]
        if not kern or not cal:
            raise SystemExit(f"no {counter} rows for the kernel or the calibration copy in {d}")
        return sum(kern) / len(kern), len(kern), max(cal)
    f_k, nf, f_c = per_dispatch(fetch_dir, "FETCH_SIZE")
    w_k, nw, w_c = per_dispatch(write_dir, "WRITE_SIZE")
    gib = float(1 << 30)
    ff, fw = gib / (f_c * 1024.0), gib / (w_c * 1024.0)
    res = {"workload": cfg.name, "kernel": dominant_kernel(cfg, single), "source_sha256": source_digest(),
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


def roofline(nbytes, flops, us, peak_tflops):
    """bound (the roof the kernel's intensity puts it under), achieved, peak, unit, frac."""
    if flops / nbytes * PEAK_HBM_GBPS * 1e9 > peak_tflops * 1e12:
        a = flops / (us * 1e-6) / 1e12
        return dict(bound="mfma", achieved=round(a, 1), peak=peak_tflops, unit="TFLOP/s", frac=round(a / peak_tflops, 4))
    a = nbytes / (us * 1e-6) / 1e9
    return dict(bound="hbm", achieved=round(a, 1), peak=PEAK_HBM_GBPS, unit="GB/s", frac=round(a / PEAK_HBM_GBPS, 4))


def peak_for(cfg):
    """Matrix peak of the arithmetic the routed products run in."""
    if cfg.act == "mxfp4":
        return PEAK_TFLOPS["fp4"]
    return PEAK_TFLOPS["bf16"]


# ------------------------------------------------------------------ CPU baseline

def _oracle_step(cfg, b, cache):
    import synth
    from oracle import layer as OL
    inp = synth.layer_inputs_np(cfg, 0, 0, b)
    r = OL.route(inp.x, inp.w_router, cfg.k, cfg.score, cfg.renormalize, cfg.routed_scaling, inp.logit_bias,
                 inp.select_bias, inp.w_shared_gate if cfg.shared == "gated" else None)
    for e in set(int(v) for v in r.ids.reshape(-1)):        # generation is not timed
        if (cfg.name, e) not in cache:
            cache[(cfg.name, e)] = synth.expert_np(cfg, e)
    if cfg.shared and (cfg.name, "s") not in cache:
        cache[(cfg.name, "s")] = synth.expert_np(cfg, synth.SHARED)
    t0 = time.perf_counter()
    OL.layer(cfg, inp, lambda e: cache[(cfg.name, e)], lambda: cache[(cfg.name, "s")])
    return time.perf_counter() - t0


def cpu_baseline(cfg, steps):
    """The float64 oracle on `steps` steps of `cfg` (token batches 0..steps-1 of instance 0)
    with the host's BLAS threads, and one-thread times of one step of the small layer and
    of `cfg`."""
    import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:
        threadpool_info = threadpool_limits = None
    affinity = len(os.sched_getaffinity(0))
    cache = {}
    limiter = threadpool_limits(affinity) if threadpool_limits else None
    total = sum(_oracle_step(cfg, b, cache) for b in range(steps))
    used = max((i.get("num_threads", 1) for i in threadpool_info()), default=1) if threadpool_info else 1
    if limiter is not None:
        limiter.restore_original_limits()
    one = {}
    if threadpool_limits:
        small = synth.get("tiny")
        with threadpool_limits(1):
            one = {small.name: round(small.T / _oracle_step(small, 0, cache), 2),
                   cfg.name: round(cfg.T / _oracle_step(cfg, 0, cache), 4)}
    return dict(value=round(steps * cfg.T / total, 4), unit="tokens/s", cores=used, kind="oracle",
                sample=f"{steps} step(s) of {cfg.name} ({steps * cfg.T} tokens), float64 NumPy, {total:.1f} s; "
                       f"expert bytes generated outside the timed region",
                affinity_cores=affinity, cpu_count=os.cpu_count(), one_thread_tokens_per_s=one)


# ------------------------------------------------------------------ GPU runs

def make_layers(M, sdev, cfg, insts, dev, single_launch=False):
    """One MoELayer per instance, on the instance's shared expert stacks."""
    layers = []
    for inst, (ex, sh) in enumerate(insts):
        t, _ = sdev.layer_tensors(cfg, dev, 0, inst, experts=ex, shared=sh)
        w = M.LayerWeights(score=cfg.score, k=cfg.k, renormalize=cfg.renormalize, routed_scaling=cfg.routed_scaling,
                           act=cfg.act, w_router=t["w_router"], experts=M.ExpertWeights.from_arrays(t["experts"]),
                           logit_bias=t["logit_bias"], select_bias=t["select_bias"],
                           shared=M.ExpertWeights.from_arrays(t["shared"]) if t["shared"] is not None else None,
                           w_shared_gate=t["w_shared_gate"] if cfg.shared == "gated" else None,
                           p_down=t["p_down"], p_up=t["p_up"])
        layers.append(M.MoELayer(w, cfg.T, dev, single_launch=single_launch))
    return layers


def run_workload(torch, sdev, cfg, layers, NB, steps, warmup, use_graphs, dev, traffic_run=False):
    """Time `steps` layer steps (graph replays over the step slots); then count the distinct
    experts of every slot and time the routed gate/up and down launches with events."""
    R = len(layers)
    xs = [sdev.token_batch(cfg, dev, 0, 0, b) for b in range(NB)]
    S = max(R, NB)
    slot = lambda j: (layers[j % R], xs[j % NB])
    torch.cuda.synchronize()
    for j in range(S):                                   # eager warm-up of every slot
        L, x = slot(j)
        L.forward(x)
    torch.cuda.synchronize()
    graphs = seq = None
    if use_graphs:
        # one graph per step slot, and one graph of all S slots in order (a model's forward
        # pass holds its layers' steps in one graph, so a step does not pay a graph launch)
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
            seq = torch.cuda.CUDAGraph()
            with torch.cuda.graph(seq, stream=stream):
                for j in range(S):
                    L, x = slot(j)
                    L.forward(x)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()

    def step(s):
        if graphs is not None:
            graphs[s % S].replay()
        else:
            L, x = slot(s)
            L.forward(x)

    def run_steps(n):
        """n steps from slot 0: whole S-step graphs, then single-step graphs for the rest."""
        if seq is None:
            for s in range(n):
                step(s)
            return
        for _ in range(n // S):
            seq.replay()
        for s in range(n % S):
            graphs[s].replay()

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    if traffic_run:
        for s in range(steps):
            step(warmup + s)
        torch.cuda.synchronize()
        return None
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    run_steps(steps)
    ev1.record()
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / steps
    ms_one_graph = None
    step_pct = None
    if graphs is not None:
        # the same steps, one graph launch per step, with an event after each: per-step times
        # (median, p10, p90) beside the mean
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record()
        for s in range(steps):
            step(s)
            evs[s + 1].record()
        torch.cuda.synchronize()
        ms_one_graph = evs[0].elapsed_time(evs[-1]) / steps
        per = sorted(evs[s].elapsed_time(evs[s + 1]) for s in range(steps))
        pick = lambda q: per[min(steps - 1, int(round(q * (steps - 1))))]
        step_pct = dict(p10=round(pick(0.1), 5), median=round(pick(0.5), 5), p90=round(pick(0.9), 5))

    # distinct routed experts touched per slot (read back after a step of that slot)
    D_slot = []
    for j in range(S):
        L, x = slot(j)
        L.forward(x)
        torch.cuda.synchronize()
        offs = L.offs.cpu()
        D_slot.append(int(((offs[1:] - offs[:-1]) > 0).sum()))
    D_steps = [D_slot[s % S] for s in range(steps)]

    # per-kernel durations: events on the step's stream around the routed gate/up and down
    # calls, over the same slots; a block of matrix products queued first keeps the GPU busy,
    # so every launch of the pass is enqueued before the GPU reaches it
    n = min(steps, 2 * S)
    a = torch.randn(8192, 8192, device=dev)
    for _ in range(4 if cfg.T < 64 else 8):
        a = a @ a * 1e-4
    single = bool(getattr(layers[0], "single", False))
    keys = ("step_begin", "step_end") if single else ("gateup_begin", "gateup_end", "down_begin", "down_end")
    ev = [{k: torch.cuda.Event(enable_timing=True) for k in keys} for _ in range(n)]
    for s in range(n):
        L, x = slot(warmup + s)
        L.forward(x, mark=lambda name, e=ev[s]: e[name].record())
    torch.cuda.synchronize()
    del a
    mean_us = lambda b, e_: 1e3 * sum(e[b].elapsed_time(e[e_]) for e in ev) / n
    if single:
        gu_us, dn_us, st_us = None, None, mean_us("step_begin", "step_end")
    else:
        gu_us, dn_us, st_us = mean_us("gateup_begin", "gateup_end"), mean_us("down_begin", "down_end"), None
    D_ev = [D_slot[(warmup + s) % S] for s in range(n)]
    # launches of each step kernel, in order: eager warm-up (one per slot), warm-up replays,
    # timed replays, the per-slot expert count, the instrumented pass
    phases = [["warm", S], ["warm_replay", warmup], ["timed", steps]]
    if graphs is not None:
        phases.append(["one_graph_per_step", steps])
    phases += [["count", S], ["events", n]]
    return dict(ms_per_step=ms_per_step, ms_one_graph=ms_one_graph, step_pct=step_pct, D_steps=D_steps, D_ev=D_ev, gu_us=gu_us, dn_us=dn_us, st_us=st_us,
                single=single, launches=n, graphs=graphs is not None, slots=S, phases=phases)


def kernel_entries(cfg, fused, r, combined=None):
    """Roofline entries of the routed gate/up and down launches of one workload."""
    combined = fused if combined is None else combined
    peak = peak_for(cfg)
    D_ev = r["D_ev"]
    gu = [algorithmic(cfg, D, fused) for D in D_ev]
    dn = [down_algorithmic(cfg, D, fused, combined) for D in D_ev]
    gu_b, gu_f = sum(x["gu_bytes"] for x in gu) / len(gu), sum(x["gu_flops"] for x in gu) / len(gu)
    dn_b, dn_f = sum(x["bytes"] for x in dn) / len(dn), sum(x["flops"] for x in dn) / len(dn)
    timing = ("HIP events on the launch stream around each launch, eager pass over the step slots "
              "after the timed region, GPU kept busy; mean over launches")
    out = []
    if r.get("single"):
        # one launch holds the whole step: its bytes and flops are the layer's
        st = [algorithmic(cfg, D, fused) for D in D_ev]
        b = sum(x["layer_bytes"] for x in st) / len(st)
        f = sum(x["layer_flops"] for x in st) / len(st)
        e = dict(workload=cfg.name, role="whole decode step: router, top-k, routed + shared gate/up, down, combine",
                 kernel=STEP_KERNEL)
        e.update(roofline(b, f, r["st_us"], peak))
        e.update(bytes_per_launch=int(b), flops_per_launch=int(f), avg_launch_us=round(r["st_us"], 2),
                 launches=r["launches"], timing=timing, phases=r["phases"])
        return [e]
    for role, pat, b, f, us in (("routed gate/up" + (" + shared gate/up" if fused and cfg.shared else ""),
                                 dominant_kernel(cfg), gu_b, gu_f, r["gu_us"]),
                                ("routed down" + (" + shared down + combine" if fused else
                                                  (" + combine" if combined else "")),
                                 down_kernel(cfg, fused, combined), dn_b, dn_f, r["dn_us"])):
        e = dict(workload=cfg.name, role=role, kernel=pat)
        e.update(roofline(b, f, us, peak))
        e.update(bytes_per_launch=int(b), flops_per_launch=int(f), avg_launch_us=round(us, 2), launches=r["launches"],
                 timing=timing, phases=r["phases"])
        out.append(e)
    return out


def profile_file(cfg):
    return os.path.join(HERE, "profiles", f"kernels_{cfg.name}.json")


def attach_profile(cfg, kernels):
    """Add the rocprofv3 mean duration of each kernel over the timed replays of the same
    command (profiles/kernels_<workload>.json, written by --profile-parse) when that file's
    sources match the library's; the fraction recomputed from it goes beside the events'."""
    try:
        with open(profile_file(cfg)) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return
    if prof.get("source_sha256") != source_digest():
        return
    by = {(k["workload"], k["kernel"]): k for k in prof["kernels"]}
    for e in kernels:
        k = by.get((e["workload"], e["kernel"]))
        if k is None:
            continue
        us = k["timed_mean_us"]
        a = e["flops_per_launch"] / (us * 1e-6) / 1e12 if e["bound"] == "mfma" else e["bytes_per_launch"] / (us * 1e-6) / 1e9
        e["rocprof"] = dict(avg_launch_us=round(us, 2), achieved=round(a, 1), frac=round(a / e["peak"], 4),
                            launches=k["timed_launches"], file=os.path.relpath(profile_file(cfg), HERE))


def parse_profile(trace_dir, json_line_file, headline):
    """rocprofv3 kernel trace of a bench run + that run's JSON line -> profiles/kernels_<workload>.json:
    per kernel of the line, the mean duration of its launches in the timed replays (each workload's
    launches of a kernel are taken in run order, sliced by the phases the line records)."""
    import csv
    import glob
    import re
    with open(json_line_file) as f:
        res = json.loads([l for l in f.read().splitlines() if l.startswith("{")][-1])
    rows = []
    for fn in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(fn)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    used = {}
    out = []
    for e in res["kernels"]:
        pat = re.compile(e["kernel"])
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows if pat.search(r["Kernel_Name"])]
        start = used.get(e["kernel"], 0)
        n_all = sum(c for _, c in e["phases"])
        mine = durs[start:start + n_all]
        used[e["kernel"]] = start + n_all
        off = 0
        timed = []
        for name, c in e["phases"]:
            if name == "timed":
                timed = mine[off:off + c]
            off += c
        if not timed:
            raise SystemExit(f"no timed launches of {e['kernel']} for {e['workload']} in {trace_dir}")
        out.append(dict(workload=e["workload"], kernel=e["kernel"], role=e["role"], timed_launches=len(timed),
                        timed_mean_us=sum(timed) / len(timed), timed_min_us=min(timed), timed_max_us=max(timed),
                        all_launches=len(mine)))
    cfg_name = res["config"]["workload"]
    prof = {"workload": cfg_name, "source_sha256": source_digest(), "kernels": out,
            "commands": [f"rocprofv3 --kernel-trace --stats -d P -o run --output-format csv -- python3 bench.py "
                         f"--config {cfg_name} --cpu-steps 0 --json-out P/line.json",
                         f"python3 bench.py --config {cfg_name} --profile-parse P P/line.json"]}
    path = os.path.join(HERE, "profiles", f"kernels_{cfg_name}.json")
    with open(path, "w") as f:
        json.dump(prof, f, indent=1)
    print(json.dumps(prof))


def workload_summary(cfg, fused, r):
    alg = [algorithmic(cfg, D, fused) for D in r["D_steps"]]
    step_s = r["ms_per_step"] * 1e-3
    lb = sum(x["layer_bytes"] for x in alg) / len(alg)
    lf = sum(x["layer_flops"] for x in alg) / len(alg)
    return dict(bytes_per_step=int(lb), flops_per_step=int(lf), **{"GB/s": round(lb / step_s / 1e9, 1)},
                hbm_frac=round(lb / step_s / 1e9 / PEAK_HBM_GBPS, 4), **{"TFLOP/s": round(lf / step_s / 1e12, 2)},
                distinct_experts_per_step=round(sum(r["D_steps"]) / len(r["D_steps"]), 2))


def arith_of(cfg):
    return {("mxfp4", "float"): "mxfp4 weights decoded exactly to bf16 x bf16 activations, fp32 accumulate",
            ("mxfp4", "mxfp4"): "mxfp4 weights x OCP-MX fp4 activations on the scaled MFMA, fp32 accumulate",
            ("fp8b128", "float"): "fp8 e4m3 weights decoded exactly to bf16 x bf16 activations, fp32 accumulate"
            }[(cfg.wfmt, cfg.act)]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen38max_decode", help="headline workload")
    ap.add_argument("--prefill", nargs="*", default=None,
                    help="further workloads timed in the same run (default: the two 512-token prefills "
                         "when the headline is the decode layer)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--instances", type=int, default=4, help="independent layer instances rotated over")
    ap.add_argument("--batches", type=int, default=16, help="token batches rotated over")
    ap.add_argument("--cpu-steps", type=int, default=3, help="oracle steps for the CPU baseline (0: skip)")
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly instead of graph replays")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--traffic-run", action="store_true",
                    help="run a few steps and a 1 GiB calibration copy, untimed (for counter passes)")
    ap.add_argument("--traffic-parse", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two counter passes into profiles/traffic_<workload>.json")
    ap.add_argument("--profile-parse", nargs=2, metavar=("TRACE_DIR", "JSON_LINE"),
                    help="turn a rocprofv3 --kernel-trace run of this command into profiles/kernels_<workload>.json")
    args = ap.parse_args()
    if args.traffic_parse:
        import synth
        parse_traffic(synth.get(args.config), *args.traffic_parse)
        return
    if args.profile_parse:
        parse_profile(*args.profile_parse, args.config)
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
    if args.no_prefill or args.traffic_run:
        extra = []
    elif args.prefill is not None:
        extra = [synth.get(n) for n in args.prefill]
    else:
        extra = [synth.get(n) for n in PREFILL_DEFAULT] if cfg.name == "qwen38max_decode" else []
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R, NB = max(1, args.instances), max(1, args.batches)

    # expert stacks per (weight stream, instance): workloads with the same stream share them
    stacks = {}

    def instances(c):
        key = (c.wtag, c.wfmt, c.d_model, c.I, c.E, c.shared_K, c.shared_I)
        if key not in stacks:
            log(f"[bench] generating {R} expert instance(s) for {c.name}")
            stacks[key] = [(synth.experts_torch(c, dev, 0, r),
                            synth.experts_torch(c, dev, 0, r, shared=True) if c.shared else None) for r in range(R)]
        return stacks[key]

    log(f"[bench] {cfg.name}: {R} instance(s), {NB} token batches")
    layers = make_layers(M, sdev, cfg, instances(cfg), dev)
    fused = layers[0].fused
    r = run_workload(torch, sdev, cfg, layers, NB, args.steps, args.warmup, not args.no_graph, dev,
                     traffic_run=args.traffic_run)
    if args.traffic_run:
        a = torch.empty(1 << 27, dtype=torch.float64, device=dev).fill_(1.0)
        torch.neg(a)
        torch.cuda.synchronize()
        log("[bench] traffic run done")
        return
    log(f"[bench] {cfg.name}: {args.steps} steps, {r['ms_per_step'] * 1e3:.2f} us/step")
    kernels = kernel_entries(cfg, fused, r, layers[0].down_combined)
    alt = None
    if fused and not args.traffic_run:
        # the decode step's other form (one launch, or its three calls) on the same steps
        single = not layers[0].single
        del layers
        la = make_layers(M, sdev, cfg, instances(cfg), dev, single_launch=single)
        ra = run_workload(torch, sdev, cfg, la, NB, args.steps, args.warmup, not args.no_graph, dev)
        alt = dict(form="single launch (moe_decode_step)" if single else "three calls",
                   ms_per_step=round(ra["ms_per_step"], 5),
                   ms_per_step_one_graph_per_step=round(ra["ms_one_graph"], 5) if ra["ms_one_graph"] else None,
                   kernels=kernel_entries(cfg, fused, ra, True))
        log(f"[bench] {cfg.name}, {alt['form']}: {ra['ms_per_step'] * 1e3:.2f} us/step")
        del la
    else:
        del layers

    prefill = {}
    for pc in extra:
        pl = make_layers(M, sdev, pc, instances(pc), dev)
        pf = pl[0].fused
        pr = run_workload(torch, sdev, pc, pl, NB, args.prefill_steps, 2, not args.no_graph, dev)
        log(f"[bench] {pc.name}: {args.prefill_steps} steps, {pr['ms_per_step'] * 1e3:.1f} us/step")
        pk = kernel_entries(pc, pf, pr, pl[0].down_combined)
        kernels += pk
        prefill[pc.name] = dict(T=pc.T, steps=args.prefill_steps, warmup=2, ms_per_step=round(pr["ms_per_step"], 5),
                                tokens_per_s=round(pc.T / (pr["ms_per_step"] * 1e-3), 1),
                                dtype="fp4" if pc.act == "mxfp4" else "bf16", arith=arith_of(pc),
                                routing=pc.notes, layer=workload_summary(pc, pf, pr), roofline=pk[0])  # (same dict)
        del pl
        torch.cuda.empty_cache()

    cpu = None
    if args.cpu_steps > 0:
        log(f"[bench] CPU baseline: oracle on {args.cpu_steps} step(s) of {cfg.name}")
        cpu = cpu_baseline(cfg, args.cpu_steps)

    attach_profile(cfg, kernels)
    roof = dict(kernels[0])
    roof["traffic"] = load_traffic(cfg)
    step_s = r["ms_per_step"] * 1e-3
    res = {
        "metric": "MoE layer tokens/s; decode HBM GB/s and prefill TFLOP/s as % roofline",
        "value": round(cfg.T / step_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "ms_per_step_one_graph_per_step": round(r["ms_one_graph"], 5) if r["ms_one_graph"] else None,
        "ms_per_step_one_graph_per_step_pct": r["step_pct"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic type of the dominant products: bf16 dot products on exactly decoded
        # weights (FLOAT mode) or FP4 x FP4 on the block-scaled MFMA (MX mode); fp32 accumulation
        "dtype": "fp4" if cfg.act == "mxfp4" else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "d_model": cfg.d_model, "I": cfg.I, "E": cfg.E,
                   "k": cfg.k, "score": cfg.score, "weights": cfg.wfmt, "activations": cfg.act,
                   "shared": cfg.shared, "latent": cfg.latent, "arith": arith_of(cfg), "instances": R,
                   "token_batches": NB, "graphs": r["graphs"],
                   "steps_per_graph": r["slots"] if r["graphs"] else None},
        "layer": workload_summary(cfg, fused, r),
        "decode_form": "single launch (moe_decode_step)" if r.get("single") else "three calls",
        "other_decode_form": alt,
        "roofline": roof,
        "kernels": kernels,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
