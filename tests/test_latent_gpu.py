"""GPU parity of the merged MLA latent projection (include/smlp_latent.h) against the
fp64 oracle.

Source: vLLM PR 345, "[II] TP-shard Kimi MLA latent projections" (Behavior, Technical
reason, Validation).  The projection y = x w^T is checked element by element against
the oracle within max|err| <= 2e-2 * RMS(ref) (bf16 operands, fp32 accumulation);
the restore of the logical order is a copy and must be bit-exact.  The whole TP16
path on one GPU -- every rank's shard projected into its slot of a gathered buffer,
then restored -- must reproduce the replicated projection.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import BF16_TOL, DEV, assert_rms_close, f64

pytestmark = pytest.mark.gpu

K = synth.HIDDEN
QA, KVA = synth.LATENT_SIZES
N = QA + KVA

binding = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from moe_shared_expert_amd import binding as b
    b.lib()  # fails loudly if libsmlp.so is missing
    binding = b


@pytest.fixture(scope="module")
def w_full():
    return synth.latent_weight(N, K)


def shard_rows(w, sizes, tp, r):
    """Rank r's rows of a merged column-sharded weight, built with torch indexing
    (test plumbing: piece r of each range, in range order)."""
    out, off = [], 0
    for s in sizes:
        p = s // tp
        out.append(w[off + r * p: off + (r + 1) * p])
        off += s
    return torch.cat(out, 0).contiguous()


def run_linear(x, w, out_fp32=False, ldy=None):
    M, N_ = x.shape[0], w.shape[0]
    odt = torch.float32 if out_fp32 else torch.bfloat16
    if ldy is None:
        y = torch.empty(M, N_, dtype=odt, device=DEV)
    else:
        y = torch.empty(M, ldy, dtype=odt, device=DEV)[:, :N_]
    binding.shared_mlp_linear(x, w, y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 33, 100, 128, 300])
@pytest.mark.parametrize("rows", [N, N // 16])
def test_projection_against_oracle(M, rows, w_full):
    x = synth.activations(M, K, config=synth.LATENT_CONFIG)
    w = w_full[:rows].contiguous()
    print(f"projection M={M} N={rows} path={binding.shared_mlp_linear_plan(M, K, rows)['path_name']}", flush=True)
    ref = oracle.linear(f64(x), f64(w))
    y = run_linear(x.to(DEV), w.to(DEV))
    assert_rms_close(y, ref, BF16_TOL, f"latent projection M={M} N={rows}")


@pytest.mark.parametrize("M,Kk,Nn", [(3, 8, 4), (16, 200, 20), (31, 1000, 132), (40, 72, 36), (129, 520, 68)])
@pytest.mark.parametrize("out_fp32", [False, True])
def test_projection_ragged_shapes(M, Kk, Nn, out_fp32):
    # K not a multiple of 64, N not a multiple of 16, M across both paths
    x = synth.normal((M, Kk), 1.0, seed=7 + M)
    w = synth.normal((Nn, Kk), Kk ** -0.5, seed=8 + Nn)
    ref = oracle.linear(f64(x), f64(w))
    y = run_linear(x.to(DEV), w.to(DEV), out_fp32=out_fp32)
    assert_rms_close(y, ref, BF16_TOL, f"projection ragged M={M} K={Kk} N={Nn} f32={out_fp32}")


@pytest.mark.parametrize("M", [16, 64])
def test_projection_forced_paths_agree(M, w_full):
    # the same projection on the streaming kernel with pinned splits and on the tiled
    # kernel (threshold 1) both meet the bar
    x = synth.activations(M, K, config=synth.LATENT_CONFIG).to(DEV)
    w = w_full.to(DEV)
    ref = oracle.linear(f64(x), f64(w))
    prev = binding.shared_mlp_set_large_m_threshold(1)
    try:
        assert binding.shared_mlp_linear_plan(M, K, N)["path_name"] == "large_m"
        assert_rms_close(run_linear(x, w), ref, BF16_TOL, f"projection tiled M={M}")
    finally:
        binding.shared_mlp_set_large_m_threshold(prev)
    if M <= 32:
        for ks in (1, 3, 8):
            binding.shared_mlp_tune_skinny(2, ksplit=ks)
            try:
                assert_rms_close(run_linear(x, w), ref, BF16_TOL, f"projection stream ks={ks}")
            finally:
                binding.shared_mlp_tune_skinny(2)


@pytest.mark.parametrize("M", [16, 128])
def test_projection_writes_only_its_slot(M, w_full):
    # y as rank 1's slot of a gathered [M, N] buffer (ldy = N): columns outside the slot
    # keep their sentinel
    tp, r = 16, 1
    w_r = shard_rows(w_full, synth.LATENT_SIZES, tp, r).to(DEV)
    x = synth.activations(M, K, config=synth.LATENT_CONFIG).to(DEV)
    n_r = N // tp
    gathered = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    binding.shared_mlp_linear(x, w_r, gathered[:, r * n_r:(r + 1) * n_r])
    torch.cuda.synchronize()
    g = gathered.cpu()
    assert torch.all(g[:, :r * n_r] == 7.0) and torch.all(g[:, (r + 1) * n_r:] == 7.0)
    ref = oracle.linear(f64(x), f64(w_r))
    assert_rms_close(g[:, r * n_r:(r + 1) * n_r], ref, BF16_TOL, f"slot projection M={M}")


@pytest.mark.parametrize("M", [1, 16, 128])
def test_tp16_sharded_path_reproduces_the_replicated_projection(M, w_full):
    # PR 345, Technical reason: the gather of the rank outputs, restored to the logical
    # order, is the replicated projection
    tp = 16
    x = synth.activations(M, K, config=synth.LATENT_CONFIG)
    xd = x.to(DEV)
    n_r = N // tp
    gathered = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    for r in range(tp):
        w_r = shard_rows(w_full, synth.LATENT_SIZES, tp, r).to(DEV)
        binding.shared_mlp_linear(xd, w_r, gathered[:, r * n_r:(r + 1) * n_r])
    logical = torch.empty_like(gathered)
    binding.shared_mlp_restore_logical(gathered, logical, synth.LATENT_SIZES, tp)
    torch.cuda.synchronize()
    # the restore is a copy: bit-exact against the oracle's reorder of the same gather
    np.testing.assert_array_equal(f64(logical), oracle.restore_logical(f64(gathered), synth.LATENT_SIZES, tp))
    ref = oracle.linear(f64(x), f64(w_full))
    assert_rms_close(logical, ref, BF16_TOL, f"tp16 sharded path M={M}")
    # and against the replicated kernel's own output: each element is the same dot
    # product, so they agree to the bf16 rounding of either
    rep = run_linear(xd, w_full.to(DEV))
    assert_rms_close(logical, f64(rep), BF16_TOL, f"tp16 vs replicated kernel M={M}")


@pytest.mark.parametrize("sizes,tp,dtype,M,shift", [
    ((1536, 576), 16, torch.bfloat16, 16, 0),   # 8-byte units
    ((1536, 576), 8, torch.bfloat16, 33, 0),    # 16-byte units (pieces of 192 and 72 elements)
    ((1536, 576), 16, torch.float32, 7, 0),
    ((1536, 576), 16, torch.bfloat16, 5, 1),    # base shifted by one element: 2-byte units
    ((6, 10, 4), 2, torch.bfloat16, 9, 0),      # odd pieces: 2-byte units
    ((12, 24), 4, torch.float32, 3, 1),         # 4-byte units
    ((64,), 4, torch.bfloat16, 2, 0),           # a single range
    ((16,) * 8, 1, torch.bfloat16, 4, 0),       # tp = 1: the identity
    ((1536, 576), 16, torch.bfloat16, 1000, 0),
])
def test_restore_is_the_oracle_reorder(sizes, tp, dtype, M, shift):
    n = sum(sizes)
    src = synth.normal((M * n + 8,), 1.0, seed=11, dtype=dtype).to(DEV)
    dst = torch.full((M * n + 8,), -3.0, dtype=dtype, device=DEV)
    g = src[shift:shift + M * n].view(M, n)
    o = dst[shift:shift + M * n].view(M, n)
    binding.shared_mlp_restore_logical(g, o, sizes, tp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(o), oracle.restore_logical(f64(g), sizes, tp))
    # nothing outside the output was written
    d = dst.cpu()
    assert torch.all(d[:shift] == -3.0) and torch.all(d[shift + M * n:] == -3.0)


def test_restore_rejects_bad_geometry_without_launching():
    g = torch.zeros(4, N, dtype=torch.bfloat16, device=DEV)
    o = torch.zeros_like(g)
    with pytest.raises(binding.SmlpError):
        binding.shared_mlp_restore_logical(g, o, (1536, 577), 16)
    with pytest.raises(binding.SmlpError):
        binding.shared_mlp_restore_logical(g[:, :N - 4].contiguous(), o[:, :N - 4].contiguous(), synth.LATENT_SIZES, 16)
    with pytest.raises(binding.SmlpError):
        binding.shared_mlp_restore_logical(g, o, synth.LATENT_SIZES, 7)


def test_m_zero_and_determinism(w_full):
    x = synth.activations(16, K, config=synth.LATENT_CONFIG).to(DEV)
    w = w_full.to(DEV)
    y0 = torch.empty(0, N, dtype=torch.bfloat16, device=DEV)
    binding.shared_mlp_linear(x[:0], w, y0)
    a = run_linear(x, w)
    b = run_linear(x, w)
    assert torch.equal(a, b)


def test_graph_replays_match_eager(w_full):
    # projection of each rank into its slot + restore, captured once and replayed, with
    # unrelated eager work between replays
    tp, M = 16, 16
    x = synth.activations(M, K, config=synth.LATENT_CONFIG).to(DEV)
    shards = [shard_rows(w_full, synth.LATENT_SIZES, tp, r).to(DEV) for r in range(tp)]
    n_r = N // tp
    gathered = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    logical = torch.empty_like(gathered)
    ws = torch.empty(max(binding.shared_mlp_linear_workspace_bytes(M, K, n_r), 256), dtype=torch.uint8,
                     device=DEV)

    def step(stream):
        for r in range(tp):
            binding.shared_mlp_linear(x, shards[r], gathered[:, r * n_r:(r + 1) * n_r], workspace=ws,
                                      stream=stream)
        binding.shared_mlp_restore_logical(gathered, logical, synth.LATENT_SIZES, tp, stream=stream)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.synchronize()
    eager = logical.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(side)
    for i in range(3):
        logical.fill_(float(i + 1))
        gathered.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(logical, eager), f"replay {i}"


@pytest.mark.parametrize("rows", [N, N // 16])
def test_split_projection_repeats_exactly(rows, w_full):
    # K split over workgroups, partials summed in slice order by the finalize kernel:
    # repeated calls give identical bits and write every element (y starts as NaN)
    M = 16
    x = synth.activations(M, K, config=synth.LATENT_CONFIG).to(DEV)
    w = w_full[:rows].contiguous().to(DEV)
    ref = oracle.linear(f64(x), f64(w))
    try:
        for ks in (2, 8, 28):
            binding.shared_mlp_tune_skinny(2, ksplit=ks)
            first = None
            for rep in range(3):
                y = torch.full((M, rows), float("nan"), dtype=torch.bfloat16, device=DEV)
                binding.shared_mlp_linear(x, w, y)
                torch.cuda.synchronize()
                if first is None:
                    first = y
                    assert_rms_close(y, ref, BF16_TOL, f"split ks={ks} N={rows}")
                else:
                    assert torch.equal(y, first), (ks, rep)
    finally:
        binding.shared_mlp_tune_skinny(2)
