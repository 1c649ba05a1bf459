"""The per-step layout choice on kernel-time curves measured through the library.

vLLM PR 50656, "[Kimi-K3] Add option to shard the shared expert instead of
replicating", section "Trade-off and why it is opt-in": one process-wide switch cannot
suit both prefill and decode, because a sharded rank reads 1/tp of the weights but adds
an all-gather and a reduce-scatter per layer; section "Evaluation": the crossover was
estimated, not measured.  Here the replicated layer and the TP8 shard are timed on the
GPU through shared_mlp_forward, the library's choice (shared_mlp_choose_layout,
shared_mlp_layout_crossover) is evaluated on those measured curves, and it must agree
with the oracle's plain model (oracle/layout.py) on the same curves.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import DEV, H, I, workspace_for

pytestmark = pytest.mark.gpu

OL = oracle.layout
TP = 8
MS = [1, 16, 128, 512, 2048]


def _curve(binding, I_r, partial, cfg):
    weights = []
    for c in range(2):
        g, d = synth.layer_weights(H, I_r, config=cfg, copy=c, fan_in_down=I)
        weights.append((g.to(DEV), d.to(DEV)))
    stream = torch.cuda.Stream(DEV)
    ts = []
    for M in MS:
        x = synth.activations(M, H, config=cfg, copy=M).to(DEV)
        out = torch.empty(M, H, dtype=torch.float32 if partial else torch.bfloat16, device=DEV)
        ws = workspace_for(M, H, I_r, binding.SMLP_BF16)
        n = 16 if M <= 512 else 4

        def fwd(i, st):
            g, d = weights[i % 2]
            binding.shared_mlp_forward(x, g, d, out, partial, ws, st)

        with torch.cuda.stream(stream):
            for i in range(4):
                fwd(i, stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for i in range(n):
                    fwd(i, stream)
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                t0.record(stream)
                graph.replay()
                t1.record(stream)
            torch.cuda.synchronize()
            best = min(best, 1e3 * t0.elapsed_time(t1) / n)
        ts.append(best)
    return [float(m) for m in MS], ts


@pytest.fixture(scope="module")
def curves():
    from moe_shared_expert_amd import binding
    binding.lib()
    rep = _curve(binding, I, False, 2)
    shard = _curve(binding, I // TP, True, 3)
    return binding, rep, shard


def test_measured_curves_are_sane(curves):
    _, rep, shard = curves
    assert all(t > 0 and np.isfinite(t) for t in rep[1] + shard[1])
    # a TP8 rank reads 1/8 of the weights: at equal tokens its kernels are faster
    for tr, ts in zip(rep[1], shard[1]):
        assert ts < tr, (rep, shard)


@pytest.mark.parametrize("alpha", [0.0, 2.0, 5.0, 10.0, 20.0])
def test_choice_on_measured_curves_matches_oracle(curves, alpha):
    binding, rep, shard = curves
    m = binding.layout_model(TP, H, rep, shard, alpha, 153.0, 7, 4)
    for T in [1, 7, 8, 9, 64, 128, 129, 256, 500, 700, 1000, 2048, 4096, 16384]:
        er, es = OL.step_times(T, TP, H, rep, shard, alpha, 153.0e3, 7, 4)
        r, s = binding.shared_mlp_layout_times(m, T)
        assert abs(r - er) <= 1e-9 * max(1.0, er) and abs(s - es) <= 1e-9 * max(1.0, es), (T, r, er, s, es)
        if abs(er - es) > 1e-6 * max(er, es):
            assert binding.shared_mlp_choose_layout(m, T) == (es < er), (T, er, es)
    want = OL.crossover(1 << 14, TP, H, rep, shard, alpha, 153.0e3, 7, 4)
    assert binding.shared_mlp_layout_crossover(m, 1 << 14) == want
