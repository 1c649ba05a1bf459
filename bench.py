"""Benchmark of the shared-expert SwiGLU MLP on one MI355X.

Headline workload: Kimi-K3 shared expert, replicated decode, M = 16 tokens, H = 7168,
I = 6144, bf16 weights with fp32 accumulation and bf16 output, 8 distinct weight
copies cycled per call (2.1 GB, beyond the 256 MB Infinity Cache).  One step is one
layer forward (gate_up + SiLU-and-mul, then down) on inputs already resident in HBM.

The default run (``--workload all``) prints ONE JSON line: the headline fields of that
workload, and nested under ``configs`` every workload of the five configurations (the
tiny fp32 case, the replicated decode, the TP8 shard, the 92-layer TP16 stack and the
M = 8192 prefill), each with its own ``roofline`` and ``cpu_baseline``; under ``sweep``
the M sweep 1 ... 8192 for the replicated layer and the TP8 shard; under ``crossover``
the replicated-vs-sharded crossover those curves give; under ``ceilings`` the measured
ceilings (launch cost, HBM and L2 streaming rates, MFMA rate and clock, grid-barrier
cost) the roofline fractions are also given against.

Timing: every step count is exactly ``--steps`` (prefill: at most 40 per trial),
captured once as a hipGraph and replayed for ``trials`` trials (at least 5, and at
least 200 timed steps in total), each between two HIP events on the launch stream with
a device synchronisation on both sides; the reported time is the median trial.
``value`` is the achieved algorithmic HBM bandwidth (weights + x + out bytes per layer
/ time per layer).  ``roofline`` reports the dominant kernel: where the plan runs the
whole layer as one launch (decode at M <= 32), that kernel, timed by the layer graph
itself (the gate_up stage alone, from a graph of that stage, is reported beside it);
otherwise the dominant stage (gate_up + SiLU-and-mul), timed the same way from a graph
of that stage alone.  ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of
the same workload.
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


def trials_for(steps):
    """At least 5 trials and at least 200 timed steps in total."""
    return max(5, -(-200 // max(1, steps)))


def graph_trials(stream, fn, n, trials):
    """Capture fn(0) ... fn(n - 1) as one hipGraph on `stream`, replay it once untimed,
    then `trials` times between two HIP events on that stream (a device synchronisation
    on both sides of each trial).  Returns the per-call microseconds of every trial."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i, stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(trials):
        t0, t1 = _ev(), _ev()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            t0.record(stream)
            g.replay()
            t1.record(stream)
        torch.cuda.synchronize()
        out.append(1e3 * t0.elapsed_time(t1) / n)
    del g
    return out


def eager_trials(stream, fn, n, trials):
    out = []
    for _ in range(trials):
        t0, t1 = _ev(), _ev()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            t0.record(stream)
            for i in range(n):
                fn(i, stream)
            t1.record(stream)
        torch.cuda.synchronize()
        out.append(1e3 * t0.elapsed_time(t1) / n)
    return out


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def make_inputs(M, I_r, copies, cfg, dev):
    x = synth.activations(M, H, config=cfg).to(dev)
    ws = []
    for c in range(copies):
        wgu, wd = synth.layer_weights(H, I_r, config=cfg, copy=c, fan_in_down=I)
        ws.append((wgu.to(dev), wd.to(dev)))
    return x, ws


PREFILL_MAX_STEPS = 40


def run_workload(name, steps, warmup, dev, launch="graph"):
    """Time exactly `steps` layer forwards per trial (value) and, separately, `steps`
    launches of the dominant gate_up stage alone, back to back (roofline)."""
    M, I_r, partial, copies, cfg, desc = WORKLOADS[name]
    if M >= 4096:
        steps = min(steps, PREFILL_MAX_STEPS)
    trials = trials_for(steps)
    x, weights = make_inputs(M, I_r, copies, cfg, dev)
    odt = torch.float32 if partial else torch.bfloat16
    out = torch.empty(M, H, dtype=odt, device=dev)
    wsb = binding.shared_mlp_workspace_bytes(M, H, I_r, binding.SMLP_BF16)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    plan = binding.shared_mlp_plan(M, H, I_r, binding.SMLP_BF16, partial)

    def step(i, stream):
        g, d = weights[i % copies]
        binding.shared_mlp_forward(x, g, d, out, partial, ws, stream)

    def gu_only(i, stream):
        g, _ = weights[i % copies]
        binding.shared_mlp_gate_up_act(x, g, ws, partial, stream)

    # graph capture needs a side stream; eager launches use it too
    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        for i in range(max(warmup, copies)):
            step(i, stream)
    torch.cuda.synchronize()
    timer = graph_trials if launch == "graph" else eager_trials
    layer = timer(stream, step, steps, trials)
    gu = graph_trials(stream, gu_only, steps, trials)

    chain_us = None
    if name == "tp16_stack92_m128":
        # the chained stack: layer l's fp32 partial, rescaled per token to unit RMS in
        # bf16, is layer l + 1's input; whole passes over the 92 layers
        xs = [torch.empty(M, H, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        xs[0].copy_(x)

        def chained(i, stream):
            g, d = weights[i % copies]
            binding.shared_mlp_forward(xs[i & 1], g, d, out, partial, ws, stream)
            binding.shared_mlp_rms_rescale(out, xs[(i + 1) & 1], stream)

        n_chain = copies * max(1, round(steps / copies))
        chain_us = median(graph_trials(stream, chained, n_chain, trials))

    out_elem = 4 if partial else 2
    alg = roofline.algorithmic_bytes(M, H, I_r, 2, out_elem)
    fl = roofline.flops(M, H, I_r)
    h_elem = {binding.SMLP_FP32: 4, binding.SMLP_BF16_HILO: 4, binding.SMLP_BF16: 2,
              binding.SMLP_FP16: 2}[plan["h_dtype"]]
    gu_alg = roofline.gate_up_bytes(H, I_r) + M * H * 2 + M * I_r * h_elem
    us = median(layer)
    gu_us = median(gu)
    del weights, x, out, ws
    torch.cuda.empty_cache()
    return {
        "name": name, "desc": desc, "M": M, "I_r": I_r, "partial": partial, "copies": copies,
        "steps": steps, "trials": trials, "launch": launch, "trial_us": [round(t, 3) for t in layer],
        "ms_per_step": us * 1e-3, "us_per_layer": us, "alg_bytes": alg, "flops": fl,
        "gbs": alg / (us * 1e-6) / 1e9, "tflops": fl / (us * 1e-6) / 1e12, "plan": plan,
        "gate_up_us": gu_us, "gate_up_alg_bytes": gu_alg, "gate_up_gbs": gu_alg / (gu_us * 1e-6) / 1e9,
        "gate_up_flops": 4 * M * H * I_r, "gate_up_tflops": 4 * M * H * I_r / (gu_us * 1e-6) / 1e12,
        "chain_us_per_layer": chain_us,
        # one launch per layer (the fused decode layer): the layer graph times that kernel
        "one_launch": plan["kernels"] == 1,
    }


def run_tiny(steps, dev):
    """The tiny fp32 case (M = 12, H = 16, I = 12): launch-bound, timed per call."""
    x, gate, up, down, _, _ = synth.tiny_fp32_case()
    wgu = synth.merged_gate_up(gate, up).to(dev)
    x, down = x.to(dev), down.to(dev)
    out = torch.empty(12, 16, dtype=torch.float32, device=dev)
    ws = torch.empty(max(binding.shared_mlp_workspace_bytes(12, 16, 12, binding.SMLP_FP32), 256),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(dev)

    def step(i, st):
        binding.shared_mlp_forward(x, wgu, down, out, False, ws, st)

    with torch.cuda.stream(stream):
        for i in range(8):
            step(i, stream)
    torch.cuda.synchronize()
    trials = trials_for(steps)
    us = median(graph_trials(stream, step, steps, trials))
    return {"workload": "tiny SwiGLU MLP, fp32, M=12, H=16, I=12 (the pages' equivalence-test shapes)",
            "M": 12, "H": 16, "I": 12, "dtype": "f32", "steps": steps, "trials": trials,
            "us_per_call": round(us, 3), "kernels": binding.shared_mlp_plan(12, 16, 12, binding.SMLP_FP32)["kernels"],
            "bound": "launch", "note": "3.8 KB and 13.8 Kflop per call: the time is the two dependent launches"}


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
    trials = trials_for(steps)
    step_us = median(graph_trials(stream, step, steps, trials))
    proj_us = median(graph_trials(stream, proj, steps, trials))
    restore_us = None
    if tp > 1:
        restore_us = median(graph_trials(
            stream, lambda i, st: binding.shared_mlp_restore_logical(gathered, logical, sizes, tp, st), steps,
            trials))
    proj_alg = roofline.latent_projection_bytes(M, H, n_r)
    alg = proj_alg + (roofline.latent_restore_bytes(M, n) if tp > 1 else 0)
    fl = 2 * M * H * n_r
    return {
        "name": name, "desc": desc, "M": M, "tp": tp, "n": n, "n_r": n_r, "copies": copies,
        "steps": steps, "trials": trials, "ms_per_step": step_us * 1e-3, "us_per_layer": step_us,
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
        "steps": r["steps"], "trials": r["trials"], "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
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
    """HBM bytes per launch of the dominant kernel (the one-launch decode layer, gate_up, or
    the latent projection)
    from the committed rocprofv3 counter summary of this workload
    (profiles/<workload>.md), or None when that summary was taken on different kernel
    sources than the ones built now."""
    import re
    path = os.path.join(ROOT, "profiles", f"{name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel source hash[^`]*`([0-9a-f]+)`", text)
    t = re.search(r"(?:gate_up|projection|layer) traffic bytes per launch: (\d+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


def _blas_cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count()]))
    except Exception:
        return int(os.cpu_count())


PREFILL_SAMPLE_TOKENS = 1024


def cpu_baseline(name, budget_s=10.0):
    """The fp64 oracle on host cores, on a bounded sample of the same workload: whole
    layers (2 weight copies cycled) for the decode-sized workloads; for the M = 8192
    prefill, the first PREFILL_SAMPLE_TOKENS tokens of the layer (the oracle's cost is
    linear in M), scaled to the whole layer."""
    import numpy as np
    import oracle
    M, I_r, partial, copies, cfg, desc = WORKLOADS[name]
    Ms = min(M, PREFILL_SAMPLE_TOKENS)
    x = synth.to_f64(synth.activations(M, H, config=cfg))[:Ms]
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
        if el >= budget_s or (el > 0 and el / n * (n + 1) > 3 * budget_s):
            break
    per_layer = el / n * (M / Ms)
    alg = roofline.algorithmic_bytes(M, H, I_r, 2, 4 if partial else 2)
    sample = (f"{n} layer forwards of the {desc} workload (2 weight copies cycled), numpy fp64 oracle, "
              f"{per_layer * 1e3:.1f} ms per layer")
    if Ms < M:
        sample = (f"{n} forwards of the first {Ms} of the {M} tokens of the {desc} workload (2 weight copies "
                  f"cycled), numpy fp64 oracle, scaled by {M // Ms} to {per_layer * 1e3:.0f} ms per layer")
    return {"value": alg / per_layer / 1e9, "unit": "GB/s", "cores": _blas_cores(), "kind": "oracle",
            "sample": sample, "seconds_per_layer": per_layer,
            "tflops": roofline.flops(M, H, I_r) / per_layer / 1e12,
            "cpu": platform.processor() or platform.machine()}


def tiny_cpu_baseline(budget_s=3.0):
    import oracle
    x, gate, up, down, _, _ = synth.tiny_fp32_case()
    xs, wgu, wd = synth.to_f64(x), synth.to_f64(synth.merged_gate_up(gate, up)), synth.to_f64(down)
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.swiglu_mlp(xs, wgu, wd)
        n += 1
    per = (time.perf_counter() - t0) / n
    return {"value": round(per * 1e6, 3), "unit": "us per call", "cores": _blas_cores(), "kind": "oracle",
            "sample": f"{n} calls of the tiny fp32 case, numpy fp64 oracle"}


def roofline_entry(name, r, ceil=None):
    """The dominant stage (gate_up + SiLU-and-mul) against its bound's peak (and, when
    measured in the same run, against the measured ceiling)."""
    if BOUND[name] == "mfma":
        e = {"bound": "mfma", "kernel": "gate_up + SiLU-and-mul",
             "achieved": round(r["gate_up_tflops"], 1), "peak": roofline.BF16_MFMA_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(r["gate_up_tflops"] / roofline.BF16_MFMA_PEAK_TFLOPS, 4),
             "kernel_us": round(r["gate_up_us"], 3), "flops_per_launch": r["gate_up_flops"],
             "bytes_per_launch": r["gate_up_alg_bytes"], "traffic": profiled_traffic(name)}
        if ceil and ceil.get("mfma_tflops"):
            e["frac_of_measured_ceiling"] = round(r["gate_up_tflops"] / ceil["mfma_tflops"], 4)
        return e
    if r.get("one_launch"):
        # the whole layer is one kernel: it is the dominant (and only) kernel
        e = {"bound": "hbm", "kernel": "decode_layer_kernel (gate_up + SiLU-and-mul + down, one launch)",
             "achieved": round(r["gbs"], 1), "peak": roofline.HBM_PEAK_GBS,
             "unit": "GB/s", "frac": round(r["gbs"] / roofline.HBM_PEAK_GBS, 4),
             "kernel_us": round(r["us_per_layer"], 3), "bytes_per_launch": r["alg_bytes"],
             "traffic": profiled_traffic(name),
             "gate_up_stage_alone": {"kernel_us": round(r["gate_up_us"], 3),
                                     "achieved": round(r["gate_up_gbs"], 1),
                                     "frac": round(r["gate_up_gbs"] / roofline.HBM_PEAK_GBS, 4)}}
        if ceil and ceil.get("hbm_read_gbs"):
            e["frac_of_measured_ceiling"] = round(r["gbs"] / ceil["hbm_read_gbs"], 4)
        return e
    e = {"bound": "hbm", "kernel": "gate_up + SiLU-and-mul",
         "achieved": round(r["gate_up_gbs"], 1), "peak": roofline.HBM_PEAK_GBS,
         "unit": "GB/s", "frac": round(r["gate_up_gbs"] / roofline.HBM_PEAK_GBS, 4),
         "kernel_us": round(r["gate_up_us"], 3), "bytes_per_launch": r["gate_up_alg_bytes"],
         "traffic": profiled_traffic(name)}
    if ceil and ceil.get("hbm_read_gbs"):
        e["frac_of_measured_ceiling"] = round(r["gate_up_gbs"] / ceil["hbm_read_gbs"], 4)
    return e


def profiled_mfma_busy(name):
    """MFMA busy fraction of the dominant kernel from the committed counter summary
    (profiles/<workload>.md), with the summary's path, or None."""
    import re
    path = os.path.join(ROOT, "profiles", f"{name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel source hash[^`]*`([0-9a-f]+)`", text)
    b = re.search(r"MFMA busy of the gate_up GEMM: ([0-9.]+)%", text)
    if not b:
        return None
    return {"value": float(b.group(1)) / 100, "source": f"profiles/{name}.md",
            "current_kernels": bool(m and m.group(1) == kernel_source_hash())}


def config_entry(name, r, cpu, ceil):
    e = {"workload": r["desc"], "M": r["M"], "H": H, "I": r["I_r"],
         "layout": "tp-shard" if r["partial"] else "replicated",
         "out": "fp32 partial" if r["partial"] else "bf16", "weight_copies": r["copies"],
         "path": r["plan"]["path_name"], "kernels": r["plan"]["kernels"], "steps": r["steps"],
         "trials": r["trials"], "trial_us": r["trial_us"],
         "us_per_layer": round(r["us_per_layer"], 3), "value": round(r["gbs"], 1), "unit": "GB/s",
         "hbm_frac": round(r["gbs"] / roofline.HBM_PEAK_GBS, 4), "tflops": round(r["tflops"], 2),
         "mfma_frac": round(r["tflops"] / roofline.BF16_MFMA_PEAK_TFLOPS, 4)}
    bound, t_roof = roofline.roofline_us(r["M"], H, r["I_r"], 4 if r["partial"] else 2)
    e["layer_bound"] = bound
    e["roofline_us"] = round(t_roof, 3)
    e["roofline_frac"] = round(t_roof / r["us_per_layer"], 4)
    if r["chain_us_per_layer"] is not None:
        e["chain_us_per_layer"] = round(r["chain_us_per_layer"], 3)
    e["roofline"] = roofline_entry(name, r, ceil)
    if BOUND[name] == "mfma":
        e["mfma_busy"] = profiled_mfma_busy(name)
    if cpu is not None:
        e["cpu_baseline"] = cpu
    return e


def measure_ceilings(dev):
    """The measured ceilings (include/smlp_ceilings.h), timed from graphs of launches."""
    stream = torch.cuda.Stream(dev)
    res = {}
    res["launch_us"] = round(median(graph_trials(stream, lambda i, st: binding.ceiling_empty(256, st), 128, 5)), 3)
    src = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.zeros(4096, dtype=torch.float32, device=dev)
    blocks = 256
    # a plain read of 2 GiB of distinct buffers (8 launches of 256 MiB, > the 256 MB
    # Infinity Cache), and of one decode layer's worth (264 MB, the 176 + 88 MB split)
    per = 1 << 20
    t = median(graph_trials(stream, lambda i, st: binding.ceiling_read(
        src[(i % 8) * blocks * per:((i % 8) + 1) * blocks * per], blocks, per, False, sink, st), 8, 5))
    res["hbm_read_gbs"] = round(blocks * per / (t * 1e-6) / 1e9, 1)
    res["hbm_read_256MiB_launch_us"] = round(t, 3)
    fixed = {}
    for kb in (32, 128, 512):
        b = kb << 10
        n = (2 << 30) // (blocks * b)
        tt = median(graph_trials(stream, lambda i, st: binding.ceiling_read(
            src[(i % n) * blocks * b:((i % n) + 1) * blocks * b], blocks, b, False, sink, st), min(n, 32), 5))
        fixed[kb] = tt
    res["hbm_read_launch_us_by_mb"] = {str(blocks * kb // 1024): round(fixed[kb], 3) for kb in fixed}
    # per-launch fixed cost: the intercept of time against bytes between the two larger sizes
    slope = (fixed[512] - fixed[128]) / (blocks * (512 - 128) * 1024)
    res["read_launch_fixed_us"] = round(fixed[128] - slope * blocks * 128 * 1024, 3)
    res["read_stream_gbs_in_launch"] = round(1e-3 / slope, 1)
    # every workgroup reading one shared 1 MiB region (L2-resident after the first touch)
    tl = median(graph_trials(stream, lambda i, st: binding.ceiling_read(src, blocks, 1 << 20, True, sink, st), 16, 5))
    res["l2_shared_read_gbs_per_cu"] = round((1 << 20) / (tl * 1e-6) / 1e9, 1)
    # two streaming phases of 64 KiB per workgroup in one launch: overlapped (no barrier),
    # behind a one-counter grid barrier, behind a two-level one; and the same two phases
    # as two dependent launches
    bar = torch.zeros(binding.CEILING_BAR_WORDS, dtype=torch.int32, device=dev)
    b = 64 << 10
    tp = [median(graph_trials(stream, lambda i, st: binding.ceiling_two_phase(
        src[(i % 8) * 2 * blocks * b:], blocks, b, mode, bar, sink, st), 16, 5)) for mode in (0, 1, 2)]

    def two_launches(i, st):
        base = (i % 8) * 2 * blocks * b
        binding.ceiling_read(src[base:base + blocks * b], blocks, b, False, sink, st)
        binding.ceiling_read(src[base + blocks * b:base + 2 * blocks * b], blocks, b, False, sink, st)
    t2 = median(graph_trials(stream, two_launches, 16, 5))
    torch.cuda.synchronize()
    res["two_phases_overlapped_us"] = round(tp[0], 3)
    res["two_phases_flat_barrier_us"] = round(tp[1], 3)
    res["two_phases_two_level_barrier_us"] = round(tp[2], 3)
    res["two_phases_two_launches_us"] = round(t2, 3)
    res["grid_barrier_us"] = round(tp[1] - tp[0], 3)
    res["grid_barrier_two_level_us"] = round(tp[2] - tp[0], 3)
    res["launch_boundary_us"] = round(t2 - tp[0], 3)
    res["grid_barrier_timed_out"] = bool(int(bar[128].item()))
    del src
    # MFMA-only loop: 512 workgroups x 8 waves, 512 rounds of 4 independent 32x32x16 MFMAs
    nb, iters = 512, 512
    cyc = torch.zeros(nb, dtype=torch.int64, device=dev)
    tic = torch.zeros(nb, dtype=torch.int64, device=dev)
    tm = median(graph_trials(stream, lambda i, st: binding.ceiling_mfma(nb, iters, sink, cyc, tic, st), 8, 5))
    fl = nb * 8 * iters * 4 * 32768
    res["mfma_tflops"] = round(fl / (tm * 1e-6) / 1e12, 1)
    c, w = cyc.double().mean().item(), tic.double().mean().item()
    res["mfma_clock_ghz"] = round(c / (w / 100e6) / 1e9, 3) if w > 0 else None
    res["mfma_frac_of_spec"] = round(res["mfma_tflops"] / roofline.BF16_MFMA_PEAK_TFLOPS, 4)
    # LDS-read-only loop: 256 workgroups x 8 waves, 8 KB per wave per round
    lsink = torch.zeros(256 * 512, dtype=torch.float32, device=dev)
    lcyc = torch.zeros(256, dtype=torch.int64, device=dev)
    liters = 4096
    binding.ceiling_lds(256, liters, lsink, lcyc, stream)
    torch.cuda.synchronize()
    per_wg = (8 * 8192 * liters) / lcyc.double()
    res["lds_read_bytes_per_clk_per_cu"] = round(per_wg.median().item(), 1)
    res["lds_read_bytes_per_clk_per_cu_max"] = round(per_wg.max().item(), 1)
    res["hbm_frac_of_spec"] = round(res["hbm_read_gbs"] / roofline.HBM_PEAK_GBS, 4)
    torch.cuda.empty_cache()
    return res


CONFIG_KEYS = {  # nested key of each workload in the default run's line
    "decode_rep_m16": "cfg2_decode_rep_m16", "tp8_shard_m128": "cfg3_tp8_shard_m128",
    "tp16_stack92_m128": "cfg4_tp16_stack92_m128", "prefill_rep_m8192": "cfg5_prefill_rep_m8192",
}


def headline(args, r, ceil, cpu):
    line = {
        "metric": METRIC, "value": round(r["gbs"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": r["steps"], "trials": r["trials"], "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": r["desc"], "M": r["M"], "H": H, "I": r["I_r"],
                   "layout": "tp-shard" if r["partial"] else "replicated",
                   "out": "fp32 partial" if r["partial"] else "bf16",
                   "weight_copies": r["copies"], "path": r["plan"]["path_name"],
                   "launch": "hipGraph replay" if r["launch"] == "graph" else "eager"},
        "us_per_layer": round(r["us_per_layer"], 3), "trial_us": r["trial_us"],
        "hbm_frac": round(r["gbs"] / roofline.HBM_PEAK_GBS, 4),
        "tflops": round(r["tflops"], 2),
        "roofline": roofline_entry(r["name"], r, ceil),
    }
    if r["chain_us_per_layer"] is not None:
        line["chain_us_per_layer"] = round(r["chain_us_per_layer"], 3)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOADS) + sorted(LATENT_WORKLOADS),
                    help="all (default): every configuration nested in one line; or one workload alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="leave the M sweep and crossover out of --workload all")
    ap.add_argument("--sweep", action="store_true", help="with a single workload: also print the M sweep lines")
    ap.add_argument("--ceilings", action="store_true", help="only measure the ceilings and print them")
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
    if args.steps < 1:
        print(json.dumps({"error": "--steps must be >= 1"}))
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
    if args.ceilings:
        print(json.dumps({"ceilings": measure_ceilings(dev)}), flush=True)
        return
    if args.workload in LATENT_WORKLOADS:
        print(json.dumps(latent_line(args, run_latent(args.workload, args.steps, args.warmup, dev))), flush=True)
        return
    if args.workload != "all":
        r = run_workload(args.workload, args.steps, args.warmup, dev, args.launch)
        cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload)
        print(json.dumps(headline(args, r, None, cpu)), flush=True)
        if args.sweep:
            res = sweep(dev, args.steps)
            for p in res["points"]:
                print(json.dumps(p), flush=True)
            print(json.dumps({"crossover": res["crossover"]}), flush=True)
        return

    # --workload all: the headline (replicated decode) and every configuration nested
    t_start = time.perf_counter()
    progress = lambda msg: print(f"[bench] {msg} ({time.perf_counter() - t_start:.0f} s)", file=sys.stderr, flush=True)
    ceil = measure_ceilings(dev)
    progress("ceilings measured")
    results = {}
    for name in ("decode_rep_m16", "tp8_shard_m128", "tp16_stack92_m128", "prefill_rep_m8192"):
        results[name] = run_workload(name, args.steps, args.warmup, dev, args.launch)
        progress(f"{name} timed")
    tiny = run_tiny(args.steps, dev)
    sw = None if args.no_sweep else sweep(dev, args.steps)
    progress("GPU work done")
    cpus = {}
    if not args.no_cpu_baseline:
        for name in results:
            cpus[name] = cpu_baseline(name)
        tiny["cpu_baseline"] = tiny_cpu_baseline()
        progress("CPU baselines done")
    r2 = results["decode_rep_m16"]
    line = headline(args, r2, ceil, cpus.get("decode_rep_m16"))
    line["configs"] = {"cfg1_tiny_fp32_m12": tiny}
    for name, r in results.items():
        line["configs"][CONFIG_KEYS[name]] = config_entry(name, r, cpus.get(name), ceil)
    if sw is not None:
        line["sweep"] = sw["points"]
        line["crossover"] = sw["crossover"]
    line["ceilings"] = ceil
    print(json.dumps(line), flush=True)


def sweep(dev, steps):
    """M sweep {1..8192} for the replicated layer and the TP8 shard (8 / 16 weight copies
    cycled, hipGraph replays; M <= 512: `steps` calls per trial, larger M at most 40),
    then the replicated-vs-sharded crossover that the measured curves give under a model
    of the two collectives (include/smlp_layout.h)."""
    # 256 and 1024 bracket the replicated/sharded crossover more closely than 128 / 512 / 2048
    Ms = [1, 8, 32, 128, 256, 512, 1024, 2048, 8192]
    curves = {}
    points = []
    stream = torch.cuda.Stream(dev)
    for layout, I_r, partial, copies, cfg in (("replicated", I, False, 8, 2), ("tp8", 768, True, 16, 3)):
        weights = []
        for c in range(copies):
            wgu, wd = synth.layer_weights(H, I_r, config=cfg, copy=c, fan_in_down=I)
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
            n = steps if M <= 512 else min(steps, 40)
            us = median(graph_trials(stream, fwd, n, 3))
            alg = roofline.algorithmic_bytes(M, H, I_r, 2, 4 if partial else 2)
            fl = roofline.flops(M, H, I_r)
            pts.append((M, us))
            bound, t_roof = roofline.roofline_us(M, H, I_r, 4 if partial else 2)
            points.append({"sweep": layout, "M": M, "I_r": I_r, "us_per_layer": round(us, 2),
                           "bound": bound, "roofline_us": round(t_roof, 2),
                           "roofline_frac": round(t_roof / us, 4),
                           "gbs": round(alg / us / 1e3, 1),
                           "hbm_frac": round(alg / us / 1e3 / roofline.HBM_PEAK_GBS, 4),
                           "tflops": round(fl / us / 1e6, 1),
                           "mfma_frac": round(fl / us / 1e6 / roofline.BF16_MFMA_PEAK_TFLOPS, 4),
                           "path": binding.shared_mlp_plan(M, H, I_r, 0, partial)["path_name"],
                           "steps": n, "trials": 3})
            del x, out, ws
        curves[layout] = ([float(m) for m, _ in pts], [u for _, u in pts])
        del weights
        torch.cuda.empty_cache()
    # crossover at TP8 over xGMI (7 links of ~153 GB/s per GPU); the fixed cost of one
    # collective is not measured on one GPU, so the crossover is given for several values
    alphas = [2.0, 5.0, 10.0, 20.0]
    tc = []
    for a in alphas:
        m = binding.layout_model(8, H, curves["replicated"], curves["tp8"], a, 153.0, 7, 4)
        tc.append(binding.shared_mlp_layout_crossover(m, 1 << 16))
    return {"points": points,
            "crossover": {"tp": 8, "link_gbps": 153.0, "links": 7, "partial": "fp32", "alpha_us": alphas,
                          "T_cross": tc, "curves_us": {k: v[1] for k, v in curves.items()},
                          "model": "shard while K_tp8(T) + AG(T) + RS(T) < K_rep(ceil(T/8))"}}


if __name__ == "__main__":
    main()
