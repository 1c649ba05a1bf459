"""GPU tests of the one-launch forms.

- The decode layer: at M <= 32 the gate_up and down stages of shared_mlp_forward run as
  one grid, the down workgroups waiting (bounded) for the gate_up workgroups of the same
  launch.  It must give the same bits as the two-launch form (same arithmetic, same
  summation order), stay correct for launches in flight on two streams at once and for
  graph replays, and turn a wait that gives up into NaN output (forced from the host
  with a zero poll limit, so that every kernel still ends normally) without leaving the
  stream's counters unusable for the next call.
- K-split streaming stages (short TP shards at decode sizes, the plain projection):
  the last-arriving slice of each column sums the partials and applies the epilogue in
  the same launch; the same bits as the separate finalize launch.

- Small fp32 layers (M * I <= 4096, M * H * I <= 2^20): both stages in one single-workgroup
  launch with h in LDS; the same bits as the two fp32 launches.

shared_mlp_tune_layer_fusion switches these off (mode 2) for the comparisons.
"""
import pytest
import torch

import oracle
import synth
from parity_util import BF16_TOL, DEV, FP32_TOL, H, I, assert_rms_close, f64, workspace_for

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
        ws = workspace_for(M, H, wd.shape[1], binding.SMLP_BF16)
    binding.shared_mlp_forward(x, wgu, wd, out, partial_fp32=partial, workspace=ws, stream=stream)
    return out


@pytest.mark.parametrize("partial", [False, True])
@pytest.mark.parametrize("M", [1, 5, 16, 17, 32])
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
    # two planes of h (short down contraction) are not fused either
    assert binding.shared_mlp_plan(32, H, 128, binding.SMLP_BF16, False)["kernels"] >= 2


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


# ------------------------------------------- K-split streaming stages reduced in-launch
def both_forms(fn):
    """fn() with the in-launch forms on, then off (separate finalize launches)."""
    binding.shared_mlp_tune_layer_fusion(1, 0)
    one = fn()
    torch.cuda.synchronize()
    binding.shared_mlp_tune_layer_fusion(2, 0)
    sep = fn()
    torch.cuda.synchronize()
    binding.shared_mlp_tune_layer_fusion(0, 0)
    return one, sep


@pytest.mark.parametrize("M,I_r", [(16, 384), (16, 512), (32, 768), (5, 384)])
def test_ksplit_gate_up_reduced_in_launch_matches_finalize(M, I_r):
    # short TP shards at decode sizes: the gate_up stage splits K four ways
    wgu, wd = synth.layer_weights(H, I_r, config=3, copy=M, fan_in_down=I)
    g, d = wgu.to(DEV), wd.to(DEV)
    x = synth.activations(M, H, config=3, copy=M).to(DEV)
    p = binding.shared_mlp_plan(M, H, I_r, binding.SMLP_BF16, True)
    assert p["path_name"] == "small_m" and p["gate_up_ksplit"] > 1 and p["kernels"] == 2
    for rep in range(2):   # the counters are left at zero for the next launch
        one, sep = both_forms(lambda: forward(x, g, d, partial=True))
        assert torch.isfinite(one).all()
        assert torch.equal(one, sep), f"M={M} I_r={I_r} rep {rep}: in-launch reduction differs"
    ref = oracle.swiglu_mlp(f64(x.cpu()), f64(wgu), f64(wd))
    assert_rms_close(one, ref, BF16_TOL, f"K-split gate_up reduced in-launch M={M} I_r={I_r}")


def test_ksplit_two_plane_down_reduced_in_launch_matches_finalize():
    M, I_r = 16, 768
    wgu, wd = synth.layer_weights(H, I_r, config=3, copy=7, fan_in_down=I)
    g, d = wgu.to(DEV), wd.to(DEV)
    x = synth.activations(M, H, config=3, copy=7).to(DEV)
    try:
        binding.shared_mlp_tune_h_planes(2)
        binding.shared_mlp_tune_skinny(1, 0, 0, 0, 0, 3)   # down stage split three ways
        assert binding.shared_mlp_plan(M, H, I_r, binding.SMLP_BF16, True)["down_ksplit"] == 3
        one, sep = both_forms(lambda: forward(x, g, d, partial=True))
    finally:
        binding.shared_mlp_tune_skinny(1, 0, 0, 0, 0, 0)
        binding.shared_mlp_tune_h_planes(0)
    assert torch.isfinite(one).all() and torch.equal(one, sep)


@pytest.mark.parametrize("N", [132, 264, 2112])
def test_ksplit_projection_reduced_in_launch_matches_finalize(N):
    M, K = 16, H
    w = synth.latent_weight(N, K, copy=N).to(DEV)
    x = synth.activations(M, K, config=3, copy=N).to(DEV)
    p = binding.shared_mlp_linear_plan(M, K, N)
    assert p["down_ksplit"] > 1 and p["kernels"] == 1

    def proj():
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        binding.shared_mlp_linear(x, w, y)
        return y
    for rep in range(2):
        one, sep = both_forms(proj)
        assert torch.isfinite(one.float()).all() and torch.equal(one, sep), f"N={N} rep {rep}"


# --------------------------------------- small fp32 layers in one single-workgroup launch
@pytest.mark.parametrize("M,Hh,Ii", [(12, 16, 12), (40, 64, 100), (7, 136, 24), (1, 8, 8)])
def test_fp32_one_launch_matches_two_launches_bit_for_bit(M, Hh, Ii):
    g = torch.Generator().manual_seed(M * 1000 + Hh + Ii)
    x = torch.randn(M, Hh, generator=g)
    wgu = torch.randn(2 * Ii, Hh, generator=g)
    wd = torch.randn(Hh, Ii, generator=g)
    xd, gd, dd = x.to(DEV), wgu.to(DEV), wd.to(DEV)

    def fwd():
        out = torch.full((M, Hh), float("nan"), dtype=torch.float32, device=DEV)
        binding.shared_mlp_forward(xd, gd, dd, out, workspace=workspace_for(M, Hh, Ii, binding.SMLP_FP32))
        return out
    assert binding.shared_mlp_plan(M, Hh, Ii, binding.SMLP_FP32)["kernels"] == 1
    one, two = both_forms(fwd)
    assert torch.equal(one, two), f"M={M} H={Hh} I={Ii}: one-launch and two-launch fp32 layers differ"
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    assert_rms_close(one, ref, FP32_TOL, f"fp32 one launch M={M} H={Hh} I={Ii}")


def test_fp32_one_launch_rank_views():
    # ranks in place (up rows I further on, w_down row stride I) on the single-workgroup form
    x, gate, up, down, tp, _ = synth.tiny_fp32_case()
    wgu = synth.merged_gate_up(gate, up)
    xd, gd, dd = x.to(DEV), wgu.to(DEV), down.to(DEV)
    for r in range(tp):
        def fwd():
            out = torch.full(tuple(x.shape[:1]) + (down.shape[0],), float("nan"), dtype=torch.float32, device=DEV)
            binding.shared_mlp_forward_rank(xd, gd, dd, out, tp, r)
            return out
        one, two = both_forms(fwd)
        assert torch.equal(one, two), f"rank {r}"
        ref = oracle.rank_partial(f64(x), f64(wgu), f64(down), tp, r)
        assert_rms_close(one, ref, FP32_TOL, f"fp32 one launch rank {r}")
