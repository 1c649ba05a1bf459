"""Benchmark of the shared-expert SwiGLU MLP on one MI355X.

Default workload: Kimi-K3 shared expert, replicated decode, M = 16 tokens,
H = 7168, I = 6144, bf16 weights with fp32 accumulation and bf16 output, 8 distinct
weight copies cycled per call (2.1 GB, beyond the 256 MB Infinity Cache).  One step
is one layer forward: the gate_up + SiLU-and-mul kernel followed by the down kernel,
on inputs already resident in HBM.

Prints one JSON line (rank 0).  ``value`` is the achieved algorithmic HBM bandwidth
(weights + x + out bytes per layer / time per layer).  ``roofline`` reports the
dominant kernel (gate_up + SiLU-and-mul): HIP events on its stream around graph
replays of back-to-back launches of that stage alone give its average launch
duration.  ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
workload.  ``--sweep`` adds one line per (layout, M) of the M sweep.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from moe_shared_expert_amd import binding, roofline  # noqa: E402

METRIC = "µs/layer & achieved HBM GB/s (% of 8 TB/s) for shared-expert MLP at M=1–8192"
H, I = synth.HIDDEN, synth.INTERMEDIATE

WORKLOADS = {
    # name: (M, I_r, partial_fp32, copies, config id, description)
    "decode_rep_m16": (16, I, False, 8, 2,
                       "Kimi-K3 shared expert, replicated decode, M=16, H=7168, I=6144, bf16 out, "
                       "8 weight copies cycled"),
    "tp8_shard_m128": (128, 768, True, 16, 3,
                       "TP8 per-rank shard, M=128, H=7168, I_r=768, fp32 partial out, 16 copies cycled"),
    "prefill_rep_m8192": (8192, I, False, 2, 5,
                          "replicated prefill, M=8192, H=7168, I=6144, bf16 out, 2 copies cycled"),
    "tp16_stack92_m128": (128, 384, True, 92, 4,
                          "TP16 per-rank shard, 92 distinct layers, M=128, H=7168, I_r=384, fp32 partial out; "
                          "chained through a per-token RMS rescale to bf16 (timed separately)"),
}


# Merged MLA latent projection (vLLM PR 345): name -> (M, tp, layers, description).  One
# step is one rank's layer: its projection into its slot of the gathered output, then
# the restore of the gathered output to the logical q_a / kv_a order.  Every (rank,
# layer) shard is a distinct buffer (24 layers x 2112 x 7168 bf16 = 727 MB in total),
# cycled, so the Infinity Cache cannot hold the weights.
LATENT_WORKLOADS = {
    "mla_latent_rep_m16": (16, 1, 24, "merged MLA latent q_a/kv_a projection, replicated (TP1), M=16, "
                                      "K=7168, N=2112 (1536 + 576), bf16, 24 layers cycled"),
    "mla_latent_tp16_m16": (16, 16, 24, "merged MLA latent q_a/kv_a projection, one TP16 rank, M=16, "
                                        "K=7168, shard [132, 7168] projected into its slot of the gathered "
                                        "[16, 2112] output, then restored to logical order; the shards of "
                                        "all 16 ranks x 24 layers cycled"),
}

# Roofline bound of the dominant kernel per workload: weight streaming is HBM-bound;
# at M = 8192 the gate_up GEMM does 2*M flops per weight byte and is MFMA-bound.
BOUND = {"decode_rep_m16": "hbm", "tp8_shard_m128": "hbm", "prefill_rep_m8192": "mfma",
         "tp16_stack92_m128": "hbm", "mla_latent_rep_m16": "hbm", "mla_latent_tp16_m16": "hbm"}


def _ev():
    return torch.cuda.Event(enable_timing=True)


def make_inputs(M, I_r, copies, cfg, dev):
    x = synth.activations(M, H, config=cfg).to(dev)
    ws = []
    for c in range(copies):
        wgu, wd = synth.layer_weights(H, I_r, config=cfg, copy=c, fan_in_down=I)
        ws.append((wgu.to(dev), wd.to(dev)))
    return x, ws


def run_workload(name, steps, warmup, dev, launch="graph"):
    """Time `steps` layer forwards (value) and, separately, `steps` launches of the
    dominant gate_up stage alone, back to back (roofline)."""
    M, I_r, partial, copies, cfg, desc = WORKLOADS[name]
    x, weights = make_inputs(M, I_r, copies, cfg, dev)
    odt = torch.float32 if partial else torch.bfloat16
    out = torch.empty(M, H, dtype=odt, device=dev)
    wsb = binding.shared_mlp_workspace_bytes(M, H, I_r, binding.SMLP_BF16)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    plan = binding.shared_mlp_plan(M, H, I_r, binding.SMLP_BF16, partial)

    def step(i, stream):
        g, d = weights[i % copies]
        binding.shared_mlp_forward(x, g, d, out, partial, ws, stream)

    # graph capture needs a side stream; eager launches use it too, so that the
    # dominant-kernel graph below can be captured in both modes
    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        for i in range(max(warmup, copies)):
            step(i, stream)
    torch.cuda.synchronize()
    graph = None
    if launch == "graph":
        # one replay = one pass over every weight copy
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for i in range(copies):
                    step(i, stream)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    reps = max(1, steps // copies) if graph is not None else 0
    n_steps = reps * copies if graph is not None else steps
    t0, t1 = _ev(), _ev()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        t0.record(stream)
        if graph is not None:
            for _ in range(reps):
                graph.replay()
        else:
            for i in range(steps):
                step(i, stream)
        t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n_steps

    # dominant kernel: gate_up + SiLU-and-mul alone, launched back to back (a graph of one
    # launch per weight copy, replayed), so the average includes no host or event
    # overhead -- the figure a kernel trace reports, plus the inter-kernel gap.
    def gu_only(i, strm):
        g, _ = weights[i % copies]
        binding.shared_mlp_gate_up_act(x, g, ws, partial, strm)

    gu_graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gu_graph, stream=stream):
            for i in range(copies):
                gu_only(i, stream)
    torch.cuda.synchronize()
    gu_reps = max(1, steps // copies)
    with torch.cuda.stream(stream):
        gu_graph.replay()
        t0.record(stream)
        for _ in range(gu_reps):
            gu_graph.replay()
        t1.record(stream)
    torch.cuda.synchronize()
    gu_us = 1e3 * t0.elapsed_time(t1) / (gu_reps * copies)

    chain_us = None
    if name == "tp16_stack92_m128":
        # the chained stack: layer l's fp32 partial, rescaled per token to unit RMS in
        # bf16, is layer l + 1's input (one graph replay = the 92 layers)
        xs = [torch.empty(M, H, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        xs[0].copy_(x)
        chain = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(chain, stream=stream):
                for i in range(copies):
                    g, d = weights[i]
                    binding.shared_mlp_forward(xs[i & 1], g, d, out, partial, ws, stream)
                    binding.shared_mlp_rms_rescale(out, xs[(i + 1) & 1], stream)
        torch.cuda.synchronize()
        chain_reps = max(1, steps // copies)
        with torch.cuda.stream(stream):
            chain.replay()
            t0.record(stream)
            for _ in range(chain_reps):
                chain.replay()
            t1.record(stream)
        torch.cuda.synchronize()
        chain_us = 1e3 * t0.elapsed_time(t1) / (chain_reps * copies)

    out_elem = 4 if partial else 2
    alg = roofline.algorithmic_bytes(M, H, I_r, 2, out_elem)
    fl = roofline.flops(M, H, I_r)
    h_elem = {binding.SMLP_FP32: 4, binding.SMLP_BF16_HILO: 4, binding.SMLP_BF16: 2}[plan["h_dtype"]]
    gu_alg = roofline.gate_up_bytes(H, I_r) + M * H * 2 + M * I_r * h_elem
    return {
        "name": name, "desc": desc, "M": M, "I_r": I_r, "partial": partial, "copies": copies,
        "steps": n_steps, "launch": launch,
        "ms_per_step": ms, "us_per_layer": ms * 1e3, "alg_bytes": alg, "flops": fl,
        "gbs": alg / (ms * 1e-3) / 1e9, "tflops": fl / (ms * 1e-3) / 1e12, "plan": plan,
        "gate_up_us": gu_us, "gate_up_alg_bytes": gu_alg, "gate_up_gbs": gu_alg / (gu_us * 1e-6) / 1e9,
        "gate_up_flops": 4 * M * H * I_r, "gate_up_tflops": 4 * M * H * I_r / (gu_us * 1e-6) / 1e12,
        "chain_us_per_layer": chain_us,
    }


def _graph_time_us(stream, fn, n, reps):
    """Average duration of fn(i) for i in range(n), captured as one graph and replayed
    `reps` times after one untimed replay (HIP events on the launch stream)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i, stream)
    torch.cuda.synchronize()
    t0, t1 = _ev(), _ev()
    with torch.cuda.stream(stream):
        g.replay()
        t0.record(stream)
        for _ in range(reps):
            g.replay()
        t1.record(stream)
    torch.cuda.synchronize()
    return 1e3 * t0.elapsed_time(t1) / (reps * n)


def run_latent(name, steps, warmup, dev):
    """Time `steps` rank-layer steps of the merged latent projection (value) and the
    projection kernel alone (roofline)."""
    M, tp, layers, desc = LATENT_WORKLOADS[name]
    sizes = synth.LATENT_SIZES
    n = sum(sizes)
    n_r = n // tp
    x = synth.activations(M, H, config=synth.LATENT_CONFIG).to(dev)
    shards = []   # (rank, weight) for every layer and rank
    for layer in range(layers):
        w = synth.latent_weight(n, H, copy=layer)
        for r in range(tp):
            if tp == 1:
                shards.append((0, w.to(dev)))
                continue
            rows, off = [], 0
            for sz in sizes:   # rank r's piece of each range, in range order
                p = sz // tp
                rows.append(w[off + r * p: off + (r + 1) * p])
                off += sz
            shards.append((r, torch.cat(rows, 0).contiguous().to(dev)))
        del w
    copies = len(shards)
    gathered = torch.empty(M, n, dtype=torch.bfloat16, device=dev)
    logical = torch.empty_like(gathered)
    wsb = binding.shared_mlp_linear_workspace_bytes(M, H, n_r)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    plan = binding.shared_mlp_linear_plan(M, H, n_r)

    def proj(i, stream):
        r, w = shards[i % copies]
        binding.shared_mlp_linear(x, w, gathered[:, r * n_r:(r + 1) * n_r], ws, stream)

    def step(i, stream):
        proj(i, stream)
        if tp > 1:
            binding.shared_mlp_restore_logical(gathered, logical, sizes, tp, stream)

    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        for i in range(max(warmup, copies)):
            step(i, stream)
    torch.cuda.synchronize()
    reps = max(1, steps // copies)
    step_us = _graph_time_us(stream, step, copies, reps)
    proj_us = _graph_time_us(stream, proj, copies, reps)
    restore_us = None
    if tp > 1:
        restore_us = _graph_time_us(
            stream, lambda i, st: binding.shared_mlp_restore_logical(gathered, logical, sizes, tp, st), 64,
            max(1, steps // 64))
    proj_alg = roofline.latent_projection_bytes(M, H, n_r)
    alg = proj_alg + (roofline.latent_restore_bytes(M, n) if tp > 1 else 0)
    fl = 2 * M * H * n_r
    return {
        "name": name, "desc": desc, "M": M, "tp": tp, "n": n, "n_r": n_r, "copies": copies,
        "steps": reps * copies, "ms_per_step": step_us * 1e-3, "us_per_layer": step_us,
        "alg_bytes": alg, "gbs": alg / (step_us * 1e-6) / 1e9, "tflops": fl / (step_us * 1e-6) / 1e12,
        "plan": plan, "proj_us": proj_us, "proj_alg_bytes": proj_alg,
        "proj_gbs": proj_alg / (proj_us * 1e-6) / 1e9, "restore_us": restore_us,
    }


def latent_cpu_baseline(name, budget_s=12.0):
    """The fp64 oracle (rank-local projection, and the restore for tp > 1) on host cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    M, tp, layers, desc = LATENT_WORKLOADS[name]
    sizes = synth.LATENT_SIZES
    n = sum(sizes)
    x = synth.to_f64(synth.activations(M, H, config=synth.LATENT_CONFIG))
    ws = [synth.to_f64(synth.latent_weight(n, H, copy=c)) for c in range(2)]
    shards = [oracle.merged_column_shard(w, sizes, tp, 0) for w in ws]
    gathered = oracle.linear(x, ws[0])   # stands in for the gathered rank outputs
    oracle.linear(x[:1], shards[0])
    k = 0
    t0 = time.perf_counter()
    while True:
        oracle.linear(x, shards[k % 2])
        if tp > 1:
            oracle.restore_logical(gathered, sizes, tp)
        k += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / k * (k + 1) > 3 * budget_s:
            break
    per = el / k
    alg = roofline.latent_projection_bytes(M, H, n // tp) + (roofline.latent_restore_bytes(M, n) if tp > 1 else 0)
    return {"value": alg / per / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{k} rank-layer steps of the {desc} workload (2 weight copies cycled), numpy fp64 "
                      f"oracle, {per * 1e3:.2f} ms per step",
            "seconds_per_layer": per, "cpu": platform.processor() or platform.machine()}


def latent_line(args, r):
    roof = {"bound": "hbm", "kernel": "merged latent projection (weight-streaming)",
            "achieved": round(r["proj_gbs"], 1), "peak": roofline.HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(r["proj_gbs"] / roofline.HBM_PEAK_GBS, 4), "kernel_us": round(r["proj_us"], 3),
            "bytes_per_launch": r["proj_alg_bytes"], "traffic": profiled_traffic(args.workload)}
    line = {
        "metric": METRIC, "value": round(r["gbs"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": r["steps"], "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/7168) weights)",
        "config": {"workload": r["desc"], "M": r["M"], "K": H, "N": r["n"], "tp": r["tp"],
                   "N_rank": r["n_r"], "weight_buffers": r["copies"], "path": r["plan"]["path_name"],
                   "launch": "hipGraph replay"},
        "us_per_layer": round(r["us_per_layer"], 3),
        "hbm_frac": round(r["gbs"] / roofline.HBM_PEAK_GBS, 4),
        "roofline": roof,
    }
    if r["restore_us"] is not None:
        line["restore_us"] = round(r["restore_us"], 3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = latent_cpu_baseline(args.workload)
    return line


KERNEL_SOURCES = ("moe_shared_expert_amd/csrc/skinny.hip", "moe_shared_expert_amd/csrc/gemm.hip",
                  "moe_shared_expert_amd/csrc/device_common.h", "moe_shared_expert_amd/csrc/api.cpp")


def kernel_source_hash():
    """SHA-256 (16 hex digits) of the kernel sources with comments and whitespace removed,
    so that a profile summary stays valid across comment-only edits."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        src = open(os.path.join(ROOT, f)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def profiled_traffic(name):
    """HBM bytes per launch of the dominant kernel (gate_up, or the latent projection)
    from the committed rocprofv3 counter summary of this workload
    (profiles/<workload>.md), or None when that summary was taken on different kernel
    sources than the ones built now."""
    import re
    path = os.path.join(ROOT, "profiles", f"{name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel source hash[^`]*`([0-9a-f]+)`", text)
    t = re.search(r"(?:gate_up|projection) traffic bytes per launch: (\d+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


def cpu_baseline(name, budget_s=12.0):
    """The fp64 oracle on host cores, on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    M, I_r, partial, copies, cfg, desc = WORKLOADS[name]
    x = synth.to_f64(synth.activations(M, H, config=cfg))
    layers = []
    for c in range(2):
        wgu, wd = synth.layer_weights(H, I_r, config=cfg, copy=c, fan_in_down=I)
        layers.append((synth.to_f64(wgu), synth.to_f64(wd)))
    oracle.swiglu_mlp(x[:1], *layers[0])
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.swiglu_mlp(x, *layers[n % 2])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or (el > 0 and n >= 1 and el / n * (n + 1) > 3 * budget_s):
            break
    per_layer = el / n
    alg = roofline.algorithmic_bytes(M, H, I_r, 2, 4 if partial else 2)
    return {"value": alg / per_layer / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} layer forwards of the {desc} workload (2 weight copies cycled), "
                      f"numpy fp64 oracle, {per_layer * 1e3:.1f} ms per layer",
            "seconds_per_layer": per_layer, "cpu": platform.processor() or platform.machine()}


def roofline_entry(name, r):
    """The dominant kernel (gate_up + SiLU-and-mul) against its bound's peak."""
    if BOUND[name] == "mfma":
        return {"bound": "mfma", "kernel": "gate_up + SiLU-and-mul",
                "achieved": round(r["gate_up_tflops"], 1), "peak": roofline.BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(r["gate_up_tflops"] / roofline.BF16_MFMA_PEAK_TFLOPS, 4),
                "kernel_us": round(r["gate_up_us"], 3), "flops_per_launch": r["gate_up_flops"],
                "bytes_per_launch": r["gate_up_alg_bytes"], "traffic": profiled_traffic(name)}
    return {"bound": "hbm", "kernel": "gate_up + SiLU-and-mul",
            "achieved": round(r["gate_up_gbs"], 1), "peak": roofline.HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(r["gate_up_gbs"] / roofline.HBM_PEAK_GBS, 4),
            "kernel_us": round(r["gate_up_us"], 3), "bytes_per_launch": r["gate_up_alg_bytes"],
            "traffic": profiled_traffic(name)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode_rep_m16", choices=sorted(WORKLOADS) + sorted(LATENT_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="also print the M sweep lines")
    ap.add_argument("--launch", default="graph", choices=("graph", "eager"),
                    help="replay the steps from a captured hipGraph (default) or launch eagerly")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 3 device copies of 256 MiB (the reference kernel for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the multi-GPU path "
                                   "(all-gather / reduce-scatter over RCCL) is not built"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "copies": 3}))
        return
    binding.lib()
    if args.workload in LATENT_WORKLOADS:
        print(json.dumps(latent_line(args, run_latent(args.workload, args.steps, args.warmup, dev))), flush=True)
        return
    r = run_workload(args.workload, args.steps, args.warmup, dev, args.launch)
    line = {
        "metric": METRIC, "value": round(r["gbs"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": r["steps"], "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": r["desc"], "M": r["M"], "H": H, "I": r["I_r"],
                   "layout": "tp-shard" if r["partial"] else "replicated",
                   "out": "fp32 partial" if r["partial"] else "bf16",
                   "weight_copies": r["copies"], "path": r["plan"]["path_name"],
                   "launch": "hipGraph replay" if r["launch"] == "graph" else "eager"},
        "us_per_layer": round(r["us_per_layer"], 3),
        "hbm_frac": round(r["gbs"] / roofline.HBM_PEAK_GBS, 4),
        "tflops": round(r["tflops"], 2),
        "roofline": roofline_entry(args.workload, r),
    }
    if r["chain_us_per_layer"] is not None:
        line["chain_us_per_layer"] = round(r["chain_us_per_layer"], 3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)
    if args.sweep:
        sweep(dev)


def sweep(dev):
    """M sweep {1..8192} for the replicated layer and the TP8 shard (8 / 16 weight copies
    cycled, hipGraph replays), then the replicated-vs-sharded crossover that the measured
    curves give under a model of the two collectives (include/smlp_layout.h)."""
    Ms = [1, 8, 32, 128, 512, 2048, 8192]
    curves = {}
    stream = torch.cuda.Stream(dev)
    for layout, I_r, partial, copies in (("replicated", I, False, 8), ("tp8", 768, True, 16)):
        weights = []
        for c in range(copies):
            wgu, wd = synth.layer_weights(H, I_r, config=6, copy=c, fan_in_down=I)
            weights.append((wgu.to(dev), wd.to(dev)))
        pts = []
        for M in Ms:
            x = synth.activations(M, H, config=6, copy=M).to(dev)
            out = torch.empty(M, H, dtype=torch.float32 if partial else torch.bfloat16, device=dev)
            ws = torch.empty(max(binding.shared_mlp_workspace_bytes(M, H, I_r, 0), 256),
                             dtype=torch.uint8, device=dev)

            def fwd(i, st):
                g, d = weights[i % copies]
                binding.shared_mlp_forward(x, g, d, out, partial, ws, st)

            with torch.cuda.stream(stream):
                for i in range(copies):
                    fwd(i, stream)
            torch.cuda.synchronize()
            us = _graph_time_us(stream, fwd, copies, max(1, (160 if M <= 512 else 16) // copies))
            alg = roofline.algorithmic_bytes(M, H, I_r, 2, 4 if partial else 2)
            fl = roofline.flops(M, H, I_r)
            pts.append((M, us))
            bound, t_roof = roofline.roofline_us(M, H, I_r, 4 if partial else 2)
            print(json.dumps({"sweep": layout, "M": M, "I_r": I_r, "us_per_layer": round(us, 2),
                              "bound": bound, "roofline_us": round(t_roof, 2),
                              "roofline_frac": round(t_roof / us, 4),
                              "gbs": round(alg / us / 1e3, 1),
                              "hbm_frac": round(alg / us / 1e3 / roofline.HBM_PEAK_GBS, 4),
                              "tflops": round(fl / us / 1e6, 1),
                              "mfma_frac": round(fl / us / 1e6 / roofline.BF16_MFMA_PEAK_TFLOPS, 4),
                              "path": binding.shared_mlp_plan(M, H, I_r, 0, partial)["path_name"],
                              "launch": "hipGraph replay"}),
                  flush=True)
        curves[layout] = ([float(m) for m, _ in pts], [u for _, u in pts])
        del weights
    # crossover at TP8 over xGMI (7 links of ~153 GB/s per GPU); the fixed cost of one
    # collective is not measured on one GPU, so the crossover is given for several values
    alphas = [2.0, 5.0, 10.0, 20.0]
    tc = []
    for a in alphas:
        m = binding.layout_model(8, H, curves["replicated"], curves["tp8"], a, 153.0, 7, 4)
        tc.append(binding.shared_mlp_layout_crossover(m, 1 << 16))
    print(json.dumps({"crossover": {"tp": 8, "link_gbps": 153.0, "links": 7, "partial": "fp32",
                                    "alpha_us": alphas, "T_cross": tc,
                                    "model": "shard while K_tp8(T) + AG(T) + RS(T) < K_rep(ceil(T/8))"}}),
          flush=True)


if __name__ == "__main__":
    main()
