"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: max|err| <= 2e-2 * RMS(ref) for bf16 inputs with fp32 accumulation
(RMS over all elements of the oracle output of that call), and <= 1e-5 * RMS(ref)
for fp32 inputs.  Inputs are the seeded synthetic tensors of ``synth``.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (BF16_TOL, DEV, FP32_TOL, H, I, assert_rms_close, f64, rms,
                         workspace_for)

pytestmark = pytest.mark.gpu

binding = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from moe_shared_expert_amd import binding as b
    b.lib()  # fails loudly if libsmlp.so is missing
    binding = b


def run_forward(x, wgu, wd, partial=False):
    M, Hh = x.shape
    Ii = wgu.shape[0] // 2
    dt = binding.SMLP_FP32 if x.dtype == torch.float32 else binding.SMLP_BF16
    odt = torch.float32 if (partial or x.dtype == torch.float32) else torch.bfloat16
    # NaN-filled, so that an output element the kernels never write fails the comparison
    out = torch.full((M, Hh), float("nan"), dtype=odt, device=DEV)
    ws = workspace_for(M, Hh, Ii, dt)
    binding.shared_mlp_forward(x, wgu, wd, out, partial_fp32=partial, workspace=ws)
    torch.cuda.synchronize()
    return out


def slice_on_gpu(wgu, wd, tp, r):
    two_i, Hh = wgu.shape
    s = two_i // 2 // tp
    wgu_r = torch.empty(2 * s, Hh, dtype=wgu.dtype, device=DEV)
    wd_r = torch.empty(Hh, s, dtype=wd.dtype, device=DEV)
    binding.shared_mlp_slice_rank(wgu, wd, wgu_r, wd_r, tp, r)
    torch.cuda.synchronize()
    return wgu_r, wd_r


# ---------------------------------------------------------------- tiny fp32 case
def test_tiny_fp32_replicated_and_slices():
    x, gate, up, down, tp, t = synth.tiny_fp32_case()
    wgu = synth.merged_gate_up(gate, up)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(down))
    xd, wgud, wdd = x.to(DEV), wgu.to(DEV), down.to(DEV)
    rep = run_forward(xd, wgud, wdd)
    assert_rms_close(rep, ref, FP32_TOL, "tiny fp32 replicated")
    total = np.zeros_like(ref)
    for r in range(tp):
        wgu_r, wd_r = slice_on_gpu(wgud, wdd, tp, r)
        ref_r = oracle.rank_partial(f64(x), f64(wgu), f64(down), tp, r)
        part = run_forward(xd, wgu_r, wd_r, partial=True)
        assert_rms_close(part, ref_r, FP32_TOL, f"tiny fp32 partial r{r}")
        total += f64(part)
    # sum of partials over the 4 slices reproduces the replicated output, per token shard
    r_all = rms(ref)
    for r in range(tp):
        mine = oracle.rank_token_rows(total, tp, r)
        err = np.abs(mine - ref[r * t:(r + 1) * t]).max()
        assert err <= FP32_TOL * r_all, (r, err)
    # the pages' own check, reported in their terms (fp32, atol = rtol = 1e-5)
    torch.testing.assert_close(torch.from_numpy(total).float(), rep.cpu(), atol=1e-5, rtol=1e-5)


# ------------------------------------------------------- replicated decode, M = 16
@pytest.fixture(scope="module")
def x16():
    return synth.activations(16, H, config=2)


@pytest.mark.parametrize("copy", range(8))
def test_decode_replicated_m16(copy, x16):
    wgu, wd = synth.layer_weights(H, I, config=2, copy=copy)
    out = run_forward(x16.to(DEV), wgu.to(DEV), wd.to(DEV))
    assert out.dtype == torch.bfloat16
    ref = oracle.swiglu_mlp(f64(x16), f64(wgu), f64(wd))
    assert_rms_close(out, ref, BF16_TOL, f"rep M=16 copy{copy}")


@pytest.mark.parametrize("planes", [1, 2])
@pytest.mark.parametrize("M", [1, 16, 32])
def test_decode_h_planes(M, planes):
    # the small path with h forced to one bf16 plane or two (hi + lo); the default takes
    # one plane here (I >= 256, M <= 32)
    x = synth.activations(M, H, config=2, copy=M)
    wgu, wd = synth.layer_weights(H, I, config=2, copy=3)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    try:
        binding.shared_mlp_tune_h_planes(planes)
        p = binding.shared_mlp_plan(M, H, I)
        assert p["path_name"] == "small_m"
        assert p["h_dtype"] == (binding.SMLP_BF16 if planes == 1 else binding.SMLP_BF16_HILO)
        out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV))
    finally:
        binding.shared_mlp_tune_h_planes(0)
    assert_rms_close(out, ref, BF16_TOL, f"decode M={M} h planes={planes}")


@pytest.mark.parametrize("Ii", [40, 128])
def test_one_plane_short_contraction_forced(Ii):
    # one plane of h forced where the default keeps two (I < 256): still within the bar
    x = synth.activations(16, 1024, config=14, copy=Ii)
    wgu, wd = synth.layer_weights(1024, Ii, config=14)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    try:
        binding.shared_mlp_tune_h_planes(1)
        out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV), partial=True)
    finally:
        binding.shared_mlp_tune_h_planes(0)
    assert_rms_close(out, ref, BF16_TOL, f"one plane forced I={Ii}")


# -------------------------------------------------------------- TP8 shard, M = 128
@pytest.mark.parametrize("copy", range(2))
def test_tp8_shard_partial(copy):
    x = synth.activations(128, H, config=3)
    wgu, wd = synth.layer_weights(H, 768, config=3, copy=copy, fan_in_down=I)
    out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV), partial=True)
    assert out.dtype == torch.float32
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    assert_rms_close(out, ref, BF16_TOL, f"tp8 partial copy{copy}")


@pytest.fixture(scope="module")
def full_layer():
    wgu, wd = synth.layer_weights(H, I, config=5, copy=0)
    return wgu, wd, f64(wgu), f64(wd)


def test_tp8_slices_sum_to_replicated(full_layer):
    wgu, wd, wgu64, wd64 = full_layer
    x = synth.activations(128, H, config=3, copy=1)
    x64 = f64(x)
    xd, wgud, wdd = x.to(DEV), wgu.to(DEV), wd.to(DEV)
    ref = oracle.swiglu_mlp(x64, wgu64, wd64)
    tp = 8
    total = np.zeros_like(ref)
    for r in range(tp):
        wgu_r, wd_r = slice_on_gpu(wgud, wdd, tp, r)
        g_r, d_r = oracle.rank_shard(wgu64, wd64, tp, r)
        assert np.array_equal(f64(wgu_r), g_r) and np.array_equal(f64(wd_r), d_r), "slice not exact"
        part = run_forward(xd, wgu_r, wd_r, partial=True)
        assert_rms_close(part, oracle.swiglu_mlp(x64, g_r, d_r), BF16_TOL, f"tp8 slice r{r}")
        total += f64(part)
    assert_rms_close(torch.from_numpy(total), ref, BF16_TOL, "tp8 sum of 8 slices vs replicated")
    # disjoint token shards: rank r keeps rows r*16..(r+1)*16 of the summed result
    for r in range(tp):
        mine = oracle.rank_token_rows(total, tp, r)
        assert np.abs(mine - ref[r * 16:(r + 1) * 16]).max() <= BF16_TOL * rms(ref)


# ------------------------------------------------- 92-layer TP16 stack, M = 128
N_LAYERS = 92


@pytest.fixture(scope="module")
def stack92():
    return [synth.layer_weights(H, 384, config=4, copy=l, fan_in_down=I) for l in range(N_LAYERS)]


@pytest.mark.parametrize("chunk", range(4))
def test_stack92_every_layer_on_seeded_input(stack92, chunk):
    # each layer's kernel output against the oracle, on a seeded unit-RMS input
    for l in range(chunk * 23, (chunk + 1) * 23):
        wgu, wd = stack92[l]
        x = synth.activations(128, H, config=4, copy=l)
        out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV), partial=True)
        ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
        assert_rms_close(out, ref, BF16_TOL, f"stack92 layer{l}")


@pytest.fixture(scope="module")
def oracle_chain(stack92):
    """The 92-layer chain run by the oracle alone from the seeded x_0: layer l's fp64
    output, rescaled per token to unit RMS (oracle.rms_rescale_rows) and stored as bf16
    (round to nearest even, the storage conversion of the inputs), is layer l + 1's
    input.  Returns every layer's bf16 input and fp64 output."""
    x = synth.activations(128, H, config=4)
    xs, outs = [], []
    for wgu, wd in stack92:
        out = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
        xs.append(x)
        outs.append(out)
        x = torch.from_numpy(oracle.rms_rescale_rows(out)).to(torch.float32).to(torch.bfloat16)
    return xs, outs


@pytest.mark.parametrize("chunk", range(4))
def test_stack92_chain_layers_on_oracle_inputs(stack92, oracle_chain, chunk):
    # Every layer of the chain on the input distribution the chain produces: the GPU layer
    # l runs on the oracle chain's x_l (no input comes from the GPU) and must match the
    # oracle's layer-l output; the GPU rescale of the GPU output must match the oracle's
    # rescale of that same output to one bf16 rounding.
    xs, outs = oracle_chain
    ws = workspace_for(128, H, 384, binding.SMLP_BF16)
    for l in range(chunk * 23, (chunk + 1) * 23):
        wgu, wd = stack92[l]
        out = torch.full((128, H), float("nan"), dtype=torch.float32, device=DEV)
        binding.shared_mlp_forward(xs[l].to(DEV), wgu.to(DEV), wd.to(DEV), out, partial_fp32=True, workspace=ws)
        nxt = torch.empty(128, H, dtype=torch.bfloat16, device=DEV)
        binding.shared_mlp_rms_rescale(out, nxt)
        torch.cuda.synchronize()
        assert_rms_close(out, outs[l], BF16_TOL, f"stack92 chain layer{l} on the oracle's input")
        ref = oracle.rms_rescale_rows(f64(out))
        err = np.abs(f64(nxt) - ref) / np.maximum(np.abs(ref), 1e-30)
        assert err.max() <= 2.0 ** -8 * 1.01, (l, err.max())


# The free-running GPU chain departs from the oracle chain by rounding alone: a CPU
# emulation of the kernels' arithmetic (bf16 operands, fp32 sums, h rounded to bf16 once)
# gives max|diff| / RMS of 1.1e-2, 2.3e-2, 3.6e-2, 6.1e-2, 9.8e-2 at layers 0-4 (growing
# about 1.6x per layer, O(1) by layer 10).  Layer 0 is held to the parity bar; layers 1-4 to
# the envelope 2e-2 * 2^l, which a wrong or stale layer input (an O(1) error) breaks at once.
CHAIN_LAYERS = 5


def test_stack92_free_running_chain_tracks_oracle(stack92, oracle_chain):
    _, outs = oracle_chain
    x = synth.activations(128, H, config=4).to(DEV)
    ws = workspace_for(128, H, 384, binding.SMLP_BF16)
    for l in range(CHAIN_LAYERS):
        wgu, wd = stack92[l]
        out = torch.full((128, H), float("nan"), dtype=torch.float32, device=DEV)
        binding.shared_mlp_forward(x, wgu.to(DEV), wd.to(DEV), out, partial_fp32=True, workspace=ws)
        nxt = torch.empty(128, H, dtype=torch.bfloat16, device=DEV)
        binding.shared_mlp_rms_rescale(out, nxt)
        torch.cuda.synchronize()
        assert_rms_close(out, outs[l], BF16_TOL * 2 ** l, f"stack92 free-running chain layer{l}")
        x = nxt


def test_stack92_chain_properties(stack92):
    # The chained run (output rescaled to unit RMS feeds the next layer).  The chain
    # amplifies rounding differences, so it is checked by properties at every layer:
    # each layer input has unit RMS per row up to bf16 rounding, outputs are finite.
    dev_w = [(g.to(DEV), d.to(DEV)) for g, d in stack92]
    x = synth.activations(128, H, config=4).to(DEV)
    out = torch.empty(128, H, dtype=torch.float32, device=DEV)
    ws = workspace_for(128, H, 384, binding.SMLP_BF16)
    for l, (g, d) in enumerate(dev_w):
        binding.shared_mlp_forward(x, g, d, out, partial_fp32=True, workspace=ws)
        nxt = torch.empty(128, H, dtype=torch.bfloat16, device=DEV)
        binding.shared_mlp_rms_rescale(out, nxt)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), l
        row_rms = nxt.float().pow(2).mean(dim=1).sqrt()
        assert (row_rms - 1).abs().max().item() < 4e-3, (l, row_rms)
        x = nxt


@pytest.mark.parametrize("Hh", [H, 12, 2044, 4100, 8192, 9000])
def test_rms_rescale_against_oracle(Hh):
    # row lengths covering each register-resident variant, ragged tails and the two-pass
    # fallback for rows longer than 8192
    a = synth.normal((128, Hh), 0.3, seed=4242, dtype=torch.float32)
    a[5] *= 100.0
    a[7] *= 1e-3
    out = torch.empty(128, Hh, dtype=torch.bfloat16, device=DEV)
    binding.shared_mlp_rms_rescale(a.to(DEV), out)
    torch.cuda.synchronize()
    ref = oracle.rms_rescale_rows(f64(a))
    # one bf16 rounding (relative half-ulp 2^-8) plus fp32 arithmetic
    err = np.abs(f64(out) - ref) / np.maximum(np.abs(ref), 1e-30)
    assert err.max() <= 2.0 ** -8 * 1.01


# ------------------------------------------------------------ prefill, M = 8192
def test_prefill_m8192_every_row(full_layer):
    # the whole [8192, 7168] output (NaN-filled before the call) against the fp64 oracle
    wgu, wd, wgu64, wd64 = full_layer
    x = synth.activations(8192, H, config=5)
    p = binding.shared_mlp_plan(8192, H, I)
    assert p["path_name"] == "large_m"
    out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV))
    ref = oracle.swiglu_mlp(f64(x), wgu64, wd64)
    assert_rms_close(out, ref, BF16_TOL, "prefill M=8192 all rows")


@pytest.mark.parametrize("partial", [False, True])
def test_down_column_split_ragged(partial):
    # 256 x 256 down tiles that fill the chip twice plus a small last round: the whole
    # rounds' columns keep that tile, the ragged remaining columns run as a second launch.
    M, Hh, Ii = 8100, 4360, 4096
    p = binding.shared_mlp_plan(M, Hh, Ii, binding.SMLP_BF16, partial)
    # gate_up, the two down launches, and for a bf16 output (fp16 h) the fp16 copy of w_down
    assert p["path_name"] == "large_m" and p["kernels"] == (3 if partial else 4), p
    x = synth.activations(M, Hh, config=13)
    wgu, wd = synth.layer_weights(Hh, Ii, config=13)
    out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV), partial=partial)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    assert_rms_close(out, ref, BF16_TOL, f"column split partial={partial}")


def test_gate_up_column_split_ragged():
    # gate_up 256 x 256 tiles that fill the chip once plus a half-full round: the features
    # of the whole round keep that tile, the ragged remaining features run as a second
    # launch that writes its columns of h in place.
    M, Hh, Ii = 2000, 7168, 6104
    p = binding.shared_mlp_plan(M, Hh, Ii)
    # two gate_up launches, the fp16 copy of w_down (fp16 h), the down GEMM
    assert p["path_name"] == "large_m" and p["kernels"] == 4, p
    assert p["gate_up_blocks"] == 8 * 32 + 16 * ((Ii - 32 * 128 + 63) // 64), p
    x = synth.activations(M, Hh, config=14)
    wgu, wd = synth.layer_weights(Hh, Ii, config=14)
    out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV))
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    assert_rms_close(out, ref, BF16_TOL, "gate_up column split")


# ---------------------------------------------- M sweep, replicated and TP8 shard
@pytest.mark.parametrize("M", [1, 8, 32, 40, 96, 128, 512, 768, 1280, 2048])
def test_sweep_replicated(M, full_layer):
    wgu, wd, wgu64, wd64 = full_layer
    x = synth.activations(M, H, config=5, copy=M)
    out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV))
    ref = oracle.swiglu_mlp(f64(x), wgu64, wd64)
    assert_rms_close(out, ref, BF16_TOL, f"sweep rep M={M}")


@pytest.mark.parametrize("tp,M", [(8, 1), (8, 8), (8, 32), (8, 128), (8, 320), (8, 512), (8, 640), (8, 1000),
                                  (8, 1536), (8, 2048), (16, 384), (16, 1024), (16, 1536), (4, 768), (2, 320)])
def test_sweep_tp(tp, M, full_layer):
    # rank 5's shard (the last rank at TP4 / TP2); M = 320 ... 1536 run the narrow gate_up plans (128 x 256 tiles split
    # 3-12 ways, or 8-wave 128 x 64 tiles) and the unsplit short-K down tiles (128 x 64 or
    # 128 x 128), 320 and 1000 with a ragged token tile
    wgu, wd, wgu64, wd64 = full_layer
    r = min(5, tp - 1)
    g_r, d_r = oracle.rank_shard(wgu64, wd64, tp, r)
    x = synth.activations(M, H, config=5, copy=10000 * tp + M)
    wgu_r, wd_r = slice_on_gpu(wgu.to(DEV), wd.to(DEV), tp, r)
    out = run_forward(x.to(DEV), wgu_r, wd_r, partial=True)
    ref = oracle.swiglu_mlp(f64(x), g_r, d_r)
    assert_rms_close(out, ref, BF16_TOL, f"sweep tp{tp} M={M}")


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("M", [1, 3, 13, 16, 17, 33, 64, 65, 100, 127, 128, 129, 200, 255, 300])
@pytest.mark.parametrize("partial", [False, True])
def test_ragged_m_medium_shapes(M, partial):
    Hh, Ii = 1024, 768
    x = synth.activations(M, Hh, config=7, copy=M)
    wgu, wd = synth.layer_weights(Hh, Ii, config=7)
    out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV), partial=partial)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    assert_rms_close(out, ref, BF16_TOL, f"ragged M={M} partial={partial}")


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("M,Hh,Ii", [(65, 1024, 768), (100, 1024, 768), (128, 1024, 768), (128, 2048, 1536),
                                     (96, 2048, 1536)])
def test_medium_shapes_bf16_out_over_seeds(M, Hh, Ii, seed):
    # the family with the least parity margin (bf16 output, medium M, H and I): eight
    # seeds per shape, on the default path for that M
    x = synth.activations(M, Hh, config=15, copy=seed)
    wgu, wd = synth.layer_weights(Hh, Ii, config=15, copy=seed)
    out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV))
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    assert_rms_close(out, ref, BF16_TOL, f"medium bf16 M={M} H={Hh} I={Ii} seed={seed}")


@pytest.mark.parametrize("Hh,Ii", [(136, 40), (72, 8), (8, 24), (520, 1000)])
@pytest.mark.parametrize("M", [1, 7, 130])
def test_ragged_feature_sizes(Hh, Ii, M):
    x = synth.activations(M, Hh, config=8, copy=M)
    wgu, wd = synth.layer_weights(Hh, Ii, config=8)
    out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV), partial=True)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    assert_rms_close(out, ref, BF16_TOL, f"ragged H={Hh} I={Ii} M={M}")


@pytest.mark.parametrize("M", [16, 64, 128])
def test_both_paths_agree_with_oracle(M):
    Hh, Ii = 2048, 1536
    x = synth.activations(M, Hh, config=9, copy=M)
    wgu, wd = synth.layer_weights(Hh, Ii, config=9)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    xd, gd, dd = x.to(DEV), wgu.to(DEV), wd.to(DEV)
    small = run_forward(xd, gd, dd)
    prev = binding.shared_mlp_set_large_m_threshold(1)
    try:
        assert binding.shared_mlp_plan(M, Hh, Ii)["path_name"] == "large_m"
        large = run_forward(xd, gd, dd)
    finally:
        binding.shared_mlp_set_large_m_threshold(prev)
    assert_rms_close(small, ref, BF16_TOL, f"small path M={M}")
    assert_rms_close(large, ref, BF16_TOL, f"large path M={M}")


# Every compiled LDS-tiled configuration (bm, bn, wm, wn, stages), pinned one stage at a
# time on a shape that spans several tiles with ragged tails in M, N and K.
GATE_UP_TILES = [(256, 256, 2, 4, 2), (128, 256, 2, 4, 3), (128, 256, 2, 2, 3), (128, 256, 2, 4, 2),
                 (128, 128, 2, 2, 2), (128, 128, 2, 2, 4), (128, 128, 4, 2, 2), (128, 128, 4, 2, 3),
                 (128, 128, 4, 2, 4), (256, 128, 4, 2, 2), (256, 128, 4, 2, 3),
                 (128, 64, 4, 1, 2), (128, 64, 4, 1, 4), (128, 64, 4, 1, 6), (128, 64, 4, 2, 3),
                 (128, 64, 4, 2, 4), (64, 64, 2, 2, 4)]
DOWN_TILES = GATE_UP_TILES + [(128, 32, 4, 1, 2), (128, 32, 4, 1, 4)]


@pytest.mark.parametrize("ksplit", [1, 3])
@pytest.mark.parametrize("stage,tile,partial", [(0, t, True) for t in GATE_UP_TILES] +
                         [(1, t, p) for t in DOWN_TILES for p in (True, False)])
def test_every_compiled_tile(stage, tile, partial, ksplit):
    # the down tiles run with an fp32 partial (h as one bf16 plane) and with a bf16 output
    # (h as one fp16 plane, the weight fragments converted in registers)
    M, Hh, Ii = 300, 1032, 392
    x = synth.activations(M, Hh, config=12, copy=1)
    wgu, wd = synth.layer_weights(Hh, Ii, config=12)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    prev = binding.shared_mlp_set_large_m_threshold(1)
    try:
        binding.shared_mlp_tune_gemm(stage, *tile, ksplit=ksplit)
        p = binding.shared_mlp_plan(M, Hh, Ii, binding.SMLP_BF16, partial)
        assert p["path_name"] == "large_m"
        assert p["h_dtype"] == (binding.SMLP_BF16 if partial else binding.SMLP_FP16)
        assert (p["gate_up_ksplit"] if stage == 0 else p["down_ksplit"]) == ksplit
        out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV), partial=partial)
    finally:
        binding.shared_mlp_tune_gemm(stage)
        binding.shared_mlp_set_large_m_threshold(prev)
    assert_rms_close(out, ref, BF16_TOL, f"stage {stage} tile {tile} ksplit {ksplit} partial {partial}")


# Tiles of the down stage when h is two bf16 planes (hi + lo): the default where I < 256 on
# the tiled path, and forced by the h-format hook at a longer K.  The 128 x 128 tile on
# 2 x 2 waves runs the pinned cross-step schedule with two activation planes.
HILO_TILES = [(128, 128, 2, 2, 3), (128, 64, 4, 1, 2), (128, 64, 4, 1, 4)]


@pytest.mark.parametrize("ksplit", [1, 3])
@pytest.mark.parametrize("tile", HILO_TILES)
@pytest.mark.parametrize("Ii,forced", [(200, False), (1000, True)])
def test_every_two_plane_down_tile(tile, ksplit, Ii, forced):
    M, Hh = 300, 1032
    x = synth.activations(M, Hh, config=15, copy=Ii)
    wgu, wd = synth.layer_weights(Hh, Ii, config=15)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    prev = binding.shared_mlp_set_large_m_threshold(1)
    if forced:
        binding.shared_mlp_tune_h_format(2)
    try:
        binding.shared_mlp_tune_gemm(1, *tile, ksplit=ksplit)
        p = binding.shared_mlp_plan(M, Hh, Ii)
        assert p["path_name"] == "large_m" and p["h_dtype"] == binding.SMLP_BF16_HILO, p
        # K = 200 holds four 64-element steps: three slices round to two of 128
        assert p["down_ksplit"] == (ksplit if Ii >= 1000 else min(ksplit, 2)), p
        out = run_forward(x.to(DEV), wgu.to(DEV), wd.to(DEV))
    finally:
        binding.shared_mlp_tune_gemm(1)
        binding.shared_mlp_tune_h_format(0)
        binding.shared_mlp_set_large_m_threshold(prev)
    assert_rms_close(out, ref, BF16_TOL, f"two-plane down tile {tile} ksplit {ksplit} I={Ii}")


def test_m_zero_leaves_output_untouched():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    wgu = torch.zeros(2 * 32, 64, dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros(64, 32, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    binding.shared_mlp_forward(x, wgu, wd, out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M", [1, 12, 16, 128, 300])
def test_guard_bands_untouched(M):
    Hh, Ii = 1024, 768
    x = synth.activations(M, Hh, config=10, copy=M).to(DEV)
    wgu, wd = synth.layer_weights(Hh, Ii, config=10)
    wgu, wd = wgu.to(DEV), wd.to(DEV)
    for partial in (False, True):
        dt = torch.float32 if partial else torch.bfloat16
        guard = 4096
        buf = torch.full((M * Hh + 2 * guard,), float("nan"), dtype=dt, device=DEV)
        out = buf[guard:guard + M * Hh].view(M, Hh)
        ws = workspace_for(M, Hh, Ii, binding.SMLP_BF16)
        binding.shared_mlp_forward(x, wgu, wd, out, partial_fp32=partial, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + M * Hh:]).all()
        assert torch.isfinite(out).all()


@pytest.mark.parametrize("M", [16, 128, 1024])
def test_deterministic_bits(M):
    Hh, Ii = 2048, 1536
    x = synth.activations(M, Hh, config=11).to(DEV)
    wgu, wd = synth.layer_weights(Hh, Ii, config=11)
    wgu, wd = wgu.to(DEV), wd.to(DEV)
    a = run_forward(x, wgu, wd)
    b = run_forward(x, wgu, wd)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_row_independence_small_path():
    Hh, Ii = 2048, 1536
    x = synth.activations(16, Hh, config=12).to(DEV)
    wgu, wd = synth.layer_weights(Hh, Ii, config=12)
    wgu, wd = wgu.to(DEV), wd.to(DEV)
    full = run_forward(x, wgu, wd, partial=True)
    for t in (0, 7, 15):
        one = run_forward(x[t:t + 1].contiguous(), wgu, wd, partial=True)
        # same kernel shape for M = 1 and M = 16: identical accumulation order
        assert torch.equal(one[0], full[t])


@pytest.mark.parametrize("M", [16, 128, 512])
def test_stage_entry_points(M):
    Hh, Ii = 2048, 1536
    x = synth.activations(M, Hh, config=13, copy=M)
    wgu, wd = synth.layer_weights(Hh, Ii, config=13)
    xd, gd, dd = x.to(DEV), wgu.to(DEV), wd.to(DEV)
    ws = workspace_for(M, Hh, Ii, binding.SMLP_BF16)
    binding.shared_mlp_gate_up_act(xd, gd, ws)
    torch.cuda.synchronize()
    h = f64(binding.read_h(ws, M, Ii, Hh).clone())
    h_ref = oracle.gate_up_act(f64(x), f64(wgu))
    # h is an intermediate, stored as one bf16 plane or two (hi + lo): elementwise it is
    # the exact value rounded at most once to bf16 (relative 2^-9), plus fp32
    # accumulation error of the two contractions (bounded here by 2e-3 * RMS).
    bound = 2.0 ** -8 * np.abs(h_ref) + 2e-3 * rms(h_ref)
    assert np.all(np.abs(h - h_ref) <= bound), f"stage gate_up_act M={M}"
    out = torch.empty(M, Hh, dtype=torch.bfloat16, device=DEV)
    binding.shared_mlp_down(dd, out, ws)
    torch.cuda.synchronize()
    whole = run_forward(xd, gd, dd)
    assert torch.equal(out.view(torch.int16), whole.view(torch.int16))


@pytest.mark.parametrize("M,Hh,Ii", [(1100, 2048, 1536), (300, 1032, 392)])
def test_weight_copy_matches_register_conversion(M, Hh, Ii):
    # fp16 h: the down stage converts w_down to fp16 once into the workspace (one pass) or
    # its weight fragments in registers; both convert the same values exactly and multiply
    # in the same order, so the outputs are bit-identical, and both meet the bar
    x = synth.activations(M, Hh, config=16, copy=M)
    wgu, wd = synth.layer_weights(Hh, Ii, config=16)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    xd, gd, dd = x.to(DEV), wgu.to(DEV), wd.to(DEV)
    prev_thr = binding.shared_mlp_set_large_m_threshold(1)
    prev = binding.shared_mlp_tune_weight_convert(1)
    try:
        p = binding.shared_mlp_plan(M, Hh, Ii)
        assert p["h_dtype"] == binding.SMLP_FP16 and p["workspace_bytes"] >= Hh * Ii * 2
        copied = run_forward(xd, gd, dd)
        ws = workspace_for(M, Hh, Ii, binding.SMLP_BF16)
        binding.shared_mlp_gate_up_act(xd, gd, ws)
        staged = torch.full((M, Hh), float("nan"), dtype=torch.bfloat16, device=DEV)
        binding.shared_mlp_down(dd, staged, ws)
        binding.shared_mlp_tune_weight_convert(1 << 30)
        in_regs = run_forward(xd, gd, dd)
    finally:
        binding.shared_mlp_tune_weight_convert(prev)
        binding.shared_mlp_set_large_m_threshold(prev_thr)
    torch.cuda.synchronize()
    assert torch.equal(copied.view(torch.int16), in_regs.view(torch.int16))
    assert torch.equal(staged.view(torch.int16), copied.view(torch.int16))
    assert_rms_close(copied, ref, BF16_TOL, f"fp16 weight copy M={M}")


def test_slice_rank_fp32_bit_exact():
    r_ = np.random.Generator(np.random.PCG64(5))
    wgu = torch.from_numpy(r_.standard_normal((2 * 24, 20)).astype(np.float32))
    wd = torch.from_numpy(r_.standard_normal((20, 24)).astype(np.float32))
    for tp in (1, 2, 3, 8):
        for r in range(tp):
            g, d = slice_on_gpu(wgu.to(DEV), wd.to(DEV), tp, r)
            eg, ed = oracle.rank_shard(f64(wgu), f64(wd), tp, r)
            assert np.array_equal(f64(g), eg) and np.array_equal(f64(d), ed)


# ------------------------------------------------------------------ graph replays
@pytest.mark.parametrize("M,partial", [(16, False), (128, True), (512, False), (4096, False)])
def test_graph_replays_match_eager(M, partial):
    """A forward captured in a hipGraph, replayed several times with eager work (garbage
    written over the output and the workspace) between replays, reproduces the eager
    result bit for bit on every replay (small path, split-K path, large path)."""
    Hh, Ii = (2048, 1536) if M < 4096 else (1032, 2048)
    x = synth.activations(M, Hh, config=15, copy=M).to(DEV)
    wgu, wd = synth.layer_weights(Hh, Ii, config=15)
    wgu, wd = wgu.to(DEV), wd.to(DEV)
    eager = run_forward(x, wgu, wd, partial)
    out = torch.empty_like(eager)
    ws = workspace_for(M, Hh, Ii, binding.SMLP_BF16)
    side = torch.cuda.Stream(DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        binding.shared_mlp_forward(x, wgu, wd, out, partial_fp32=partial, workspace=ws, stream=side)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            binding.shared_mlp_forward(x, wgu, wd, out, partial_fp32=partial, workspace=ws, stream=side)
    torch.cuda.synchronize()
    ibits = torch.int32 if eager.dtype == torch.float32 else torch.int16
    for rep in range(3):
        out.fill_(float("nan"))
        ws.fill_(0x7f)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(ibits), eager.view(ibits)), f"replay {rep}"


# ------------------------------------------- rank partial read in place from full weights
@pytest.mark.parametrize("M", [1, 16, 32, 64, 128, 300])
@pytest.mark.parametrize("tp", [2, 4, 8, 16])
def test_forward_rank_in_place(M, tp):
    # the sharded layout run on views of the replicated weights (no shard copy): each
    # rank's partial against the oracle's, on every path the planner takes for these M
    Hh, Ii = 1024, 2048
    x = synth.activations(M, Hh, config=15, copy=M)
    wgu, wd = synth.layer_weights(Hh, Ii, config=15)
    xd, gd, dd = x.to(DEV), wgu.to(DEV), wd.to(DEV)
    for r in sorted({0, 1, tp - 1}):
        out = torch.full((M, Hh), float("nan"), dtype=torch.float32, device=DEV)
        binding.shared_mlp_forward_rank(xd, gd, dd, out, tp, r)
        torch.cuda.synchronize()
        ref = oracle.rank_partial(f64(x), f64(wgu), f64(wd), tp, r)
        assert_rms_close(out, ref, BF16_TOL, f"rank in place M={M} tp={tp} r={r}")


def test_forward_rank_matches_copied_shard_and_sums():
    # Kimi-K3 shapes, TP8, M = 128: in place equals the copied shard up to summation
    # order, and the 8 partials sum to the replicated output
    x = synth.activations(128, H, config=16)
    wgu, wd = synth.layer_weights(H, I, config=16)
    xd, gd, dd = x.to(DEV), wgu.to(DEV), wd.to(DEV)
    total = np.zeros((128, H))
    for r in range(8):
        a = torch.empty(128, H, dtype=torch.float32, device=DEV)
        binding.shared_mlp_forward_rank(xd, gd, dd, a, 8, r)
        g_r, d_r = slice_on_gpu(gd, dd, 8, r)
        b = run_forward(xd, g_r, d_r, partial=True)
        ref_r = oracle.rank_partial(f64(x), f64(wgu), f64(wd), 8, r)
        assert_rms_close(a, ref_r, BF16_TOL, f"rank {r} in place")
        assert_rms_close(a, f64(b), BF16_TOL, f"rank {r} in place vs copied")
        total += f64(a)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd))
    assert_rms_close(torch.from_numpy(total), ref, BF16_TOL, "sum of in-place partials")


def test_forward_rank_fp32_tiny():
    x, gate, up, down, tp, t = synth.tiny_fp32_case()
    wgu = synth.merged_gate_up(gate, up)
    xd, gd, dd = x.to(DEV), wgu.to(DEV), down.to(DEV)
    total = np.zeros((12, 16))
    for r in range(tp):
        out = torch.empty(12, 16, dtype=torch.float32, device=DEV)
        binding.shared_mlp_forward_rank(xd, gd, dd, out, tp, r)
        torch.cuda.synchronize()
        ref_r = oracle.rank_partial(f64(x), f64(wgu), f64(down), tp, r)
        assert_rms_close(out, ref_r, FP32_TOL, f"tiny fp32 rank {r} in place")
        total += f64(out)
    ref = oracle.swiglu_mlp(f64(x), f64(wgu), f64(down))
    assert np.abs(total - ref).max() <= FP32_TOL * rms(ref)


def test_largest_legal_token_count():
    # M * H = 2^31 - 1 - (2^31 - 1) % H, the largest the 32-bit buffer offsets allow (H = I = 256):
    # x is a seeded 4096-row block repeated on the device; sampled rows against the oracle,
    # including the last row
    Hh = Ii = 256
    M = (2 ** 31 - 1) // Hh
    block = synth.activations(4096, Hh, config=19)
    wgu, wd = synth.layer_weights(Hh, Ii, config=19)
    print(f"largest M = {M}", flush=True)
    x = block.to(DEV).repeat((M + 4095) // 4096, 1)[:M].contiguous()
    p = binding.shared_mlp_plan(M, Hh, Ii)
    assert p["path_name"] == "large_m"
    out = run_forward(x, wgu.to(DEV), wd.to(DEV))
    rows = [0, 1, 4095, 4096, M // 2, M - 4097, M - 2, M - 1]
    got = out[rows].cpu()
    del x, out
    torch.cuda.empty_cache()
    ref_all = oracle.swiglu_mlp(f64(block), f64(wgu), f64(wd))
    ref = ref_all[[r % 4096 for r in rows]]
    assert_rms_close(got, ref, BF16_TOL, f"largest M={M}", ref_rms=rms(ref_all))


def test_concurrent_streams_match_sequential():
    # calls with their own workspaces on two streams share no device state: run together,
    # every output equals its sequential result bit for bit
    xa = synth.activations(16, H, config=2, copy=5).to(DEV)
    ga, da = (t.to(DEV) for t in synth.layer_weights(H, I, config=2, copy=5))
    xb = synth.activations(128, H, config=3, copy=5).to(DEV)
    gb, db = (t.to(DEV) for t in synth.layer_weights(H, 768, config=3, copy=5, fan_in_down=I))
    ref_a = run_forward(xa, ga, da)
    ref_b = run_forward(xb, gb, db, partial=True)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    wsa, wsb = workspace_for(16, H, I, binding.SMLP_BF16), workspace_for(128, H, 768, binding.SMLP_BF16)
    outs_a = [torch.full((16, H), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(6)]
    outs_b = [torch.full((128, H), float("nan"), dtype=torch.float32, device=DEV) for _ in range(6)]
    torch.cuda.synchronize()
    for i in range(6):
        binding.shared_mlp_forward(xa, ga, da, outs_a[i], False, wsa, sa)
        binding.shared_mlp_forward(xb, gb, db, outs_b[i], True, wsb, sb)
    torch.cuda.synchronize()
    for i in range(6):
        assert torch.equal(outs_a[i].view(torch.int16), ref_a.view(torch.int16)), i
        assert torch.equal(outs_b[i], ref_b), i
