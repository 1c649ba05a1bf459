"""GPU tests of the one-launch decode layer: at M <= 16 the gate_up and down stages of
shared_mlp_forward run as one grid, the down workgroups waiting (bounded) for the
gate_up workgroups of the same launch (shared_mlp_tune_layer_fusion).

The fused launch must give the same bits as the two-launch form (same kernels' arithmetic,
same summation order), stay correct for launches in flight on two streams at once and
for graph replays, and turn a wait that gives up into NaN output (forced from the host
with a zero poll limit, so that every kernel still ends normally) without leaving the
stream's counters unusable for the next call.
"""
import pytest
import torch

import oracle
import synth
from parity_util import BF16_TOL, DEV, H, I, assert_rms_close, f64, workspace_for

pytestmark = pytest.mark.gpu

binding = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from moe_shared_expert_amd import binding as b
    b.lib()
    binding = b


@pytest.fixture(autouse=True)
def _automatic_fusion():
    yield
    binding.shared_mlp_tune_layer_fusion(0, 0)


@pytest.fixture(scope="module")
def layers():
    out = []
    for c in range(3):
        wgu, wd = synth.layer_weights(H, I, config=2, copy=c)
        out.append((wgu.to(DEV), wd.to(DEV)))
    return out


def forward(x, wgu, wd, partial=False, stream=None, out=None, ws=None):
    M = x.shape[0]
    if out is None:
        out = torch.full((M, H), float("nan"), dtype=torch.float32 if partial else torch.bfloat16, device=DEV)
    if ws is None:
        ws = workspace_for(M, H, I, binding.SMLP_BF16)
    binding.shared_mlp_forward(x, wgu, wd, out, partial_fp32=partial, workspace=ws, stream=stream)
    return out


@pytest.mark.parametrize("partial", [False, True])
@pytest.mark.parametrize("M", [1, 5, 16])
def test_fused_layer_matches_two_launches_bit_for_bit(M, partial, layers):
    x = synth.activations(M, H, config=2).to(DEV)
    wgu, wd = layers[M % 3]
    assert binding.shared_mlp_plan(M, H, I, binding.SMLP_BF16, partial)["kernels"] == 1
    fused = forward(x, wgu, wd, partial)
    torch.cuda.synchronize()
    binding.shared_mlp_tune_layer_fusion(2, 0)
    assert binding.shared_mlp_plan(M, H, I, binding.SMLP_BF16, partial)["kernels"] == 2
    two = forward(x, wgu, wd, partial)
    torch.cuda.synchronize()
    assert torch.isfinite(fused.float()).all()
    assert torch.equal(fused, two), f"M={M} partial={partial}: fused and two-launch outputs differ"
    if M == 5:
        ref = oracle.swiglu_mlp(f64(x.cpu()), f64(wgu.cpu()), f64(wd.cpu()))
        assert_rms_close(fused, ref, BF16_TOL, f"fused decode layer M={M} partial={partial}")


def test_plan_without_the_fused_configuration_keeps_two_launches():
    # down rows per workgroup differ at H = 4096 (16 instead of 28): two launches
    assert binding.shared_mlp_plan(16, 4096, I, binding.SMLP_BF16, False)["kernels"] == 2
    # two token tiles (M = 17..32) are not fused either
    assert binding.shared_mlp_plan(32, H, I, binding.SMLP_BF16, False)["kernels"] == 2


def test_fused_layers_on_two_streams_and_graph_replays(layers):
    M = 16
    x = synth.activations(M, H, config=2).to(DEV)
    binding.shared_mlp_tune_layer_fusion(2, 0)
    refs = [forward(x, wgu, wd) for wgu, wd in layers]
    torch.cuda.synchronize()
    binding.shared_mlp_tune_layer_fusion(1, 0)

    # launches in flight on two streams at once, each stream with its own buffers
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    bufs = [(torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=DEV),
             workspace_for(M, H, I, binding.SMLP_BF16)) for _ in range(2)]
    for rnd in range(3):
        outs = []
        for k, st in enumerate((s1, s2)):
            c = (rnd + k) % 3
            outs.append((c, forward(x, *layers[c], stream=st, out=bufs[k][0], ws=bufs[k][1])))
        torch.cuda.synchronize()
        for c, o in outs:
            assert torch.equal(o, refs[c]), f"round {rnd}: copy {c} differs on a second stream"

    # a captured graph of three layers, replayed with eager launches in between
    out_g = [torch.empty(M, H, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    ws_g = workspace_for(M, H, I, binding.SMLP_BF16)
    with torch.cuda.stream(s1):
        for c in range(3):
            forward(x, *layers[c], stream=s1, out=out_g[c], ws=ws_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s1):
        with torch.cuda.graph(g, stream=s1):
            for c in range(3):
                forward(x, *layers[c], stream=s1, out=out_g[c], ws=ws_g)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in out_g:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for c in range(3):
            assert torch.equal(out_g[c], refs[c]), f"graph replay {rep}: layer {c} differs"
        eager = forward(x, *layers[rep % 3])
        torch.cuda.synchronize()
        assert torch.equal(eager, refs[rep % 3]), f"eager launch after replay {rep} differs"


def test_wait_that_gives_up_writes_nan_and_the_stream_recovers(layers):
    M = 16
    x = synth.activations(M, H, config=2).to(DEV)
    wgu, wd = layers[0]
    binding.shared_mlp_tune_layer_fusion(2, 0)
    ref = forward(x, wgu, wd)
    torch.cuda.synchronize()
    # every down workgroup gives up at once (no poll): the output is NaN, nothing hangs
    binding.shared_mlp_tune_layer_fusion(1, -1)
    bad = forward(x, wgu, wd)
    torch.cuda.synchronize()
    assert torch.isnan(bad.float()).all()
    # the same stream's counters are intact for the next launches
    binding.shared_mlp_tune_layer_fusion(1, 0)
    for _ in range(2):
        good = forward(x, wgu, wd)
        torch.cuda.synchronize()
        assert torch.equal(good, ref)
