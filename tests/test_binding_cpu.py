"""Host-only tests of the Python binding's guards and of the planner's coverage.

The C ABI takes raw pointers and cannot see buffer sizes, so the binding is the
only place that can refuse a tensor of the wrong element type or shape; every case
here must raise before anything is launched (the tensors live on the CPU, so a call
that got past the guards would fail with "tensors must be on the GPU" instead).
"""
import itertools
import os

import pytest
import torch

binding = pytest.importorskip("moe_shared_expert_amd.binding")

BF, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libsmlp.so is not built (python -m moe_shared_expert_amd.build)")
    return binding.lib()


def _t(shape, dt):
    return torch.zeros(shape, dtype=dt)


def _layer(M=4, H=64, I=24, dt=BF):
    return _t((M, H), dt), _t((2 * I, H), dt), _t((H, I), dt)


def _reaches_launch(fn):
    """True when fn got past every guard (it then fails on the CPU tensors)."""
    with pytest.raises(ValueError, match="on the GPU"):
        fn()
    return True


def test_forward_checks_output_dtype(L):
    x, wgu, wd = _layer()
    with pytest.raises(TypeError):   # a partial is fp32: a bf16 out would be overrun 2x
        binding.shared_mlp_forward(x, wgu, wd, _t((4, 64), BF), partial_fp32=True)
    with pytest.raises(TypeError):
        binding.shared_mlp_forward(x, wgu, wd, _t((4, 64), F32), partial_fp32=False)
    assert _reaches_launch(lambda: binding.shared_mlp_forward(x, wgu, wd, _t((4, 64), BF)))
    assert _reaches_launch(lambda: binding.shared_mlp_forward(x, wgu, wd, _t((4, 64), F32), partial_fp32=True))


def test_forward_checks_weight_dtypes(L):
    x, wgu, wd = _layer()
    with pytest.raises(TypeError):   # fp32 x with bf16 weights would read 2x past the weights
        binding.shared_mlp_forward(x.float(), wgu, wd, _t((4, 64), F32))
    with pytest.raises(TypeError):
        binding.shared_mlp_forward(x, wgu.float(), wd, _t((4, 64), BF))
    with pytest.raises(TypeError):
        binding.shared_mlp_forward(x, wgu, wd.float(), _t((4, 64), BF))
    with pytest.raises(TypeError):
        binding.shared_mlp_forward(x.half(), wgu.half(), wd.half(), _t((4, 64), BF))
    xf, wguf, wdf = _layer(dt=F32)
    assert _reaches_launch(lambda: binding.shared_mlp_forward(xf, wguf, wdf, _t((4, 64), F32)))
    with pytest.raises(TypeError):   # fp32 inputs always give an fp32 output
        binding.shared_mlp_forward(xf, wguf, wdf, _t((4, 64), BF))


def test_forward_checks_shapes(L):
    x, wgu, wd = _layer()
    with pytest.raises(ValueError, match="w_down"):
        binding.shared_mlp_forward(x, wgu, _t((64, 23), BF), _t((4, 64), BF))
    with pytest.raises(ValueError, match="out"):
        binding.shared_mlp_forward(x, wgu, wd, _t((5, 64), BF))
    with pytest.raises(ValueError, match="w_gate_up"):
        binding.shared_mlp_forward(x, _t((48, 63), BF), wd, _t((4, 64), BF))


def test_stage_entry_points_check_types(L):
    x, wgu, wd = _layer()
    ws = _t((1 << 16,), torch.uint8)
    with pytest.raises(TypeError):
        binding.shared_mlp_gate_up_act(x, wgu.float(), ws)
    assert _reaches_launch(lambda: binding.shared_mlp_gate_up_act(x, wgu, ws))
    with pytest.raises(ValueError, match="out"):   # out's columns must be w_down's rows
        binding.shared_mlp_down(wd, _t((4, 32), BF), ws)
    with pytest.raises(TypeError):
        binding.shared_mlp_down(wd, _t((4, 64), BF), ws, partial_fp32=True)
    with pytest.raises(TypeError):
        binding.shared_mlp_down(wd, _t((4, 64), F32), ws, partial_fp32=False)
    assert _reaches_launch(lambda: binding.shared_mlp_down(wd, _t((4, 64), F32), ws, partial_fp32=True))


def test_slice_rank_checks_destinations(L):
    _, wgu, wd = _layer(I=24)
    good = (_t((12, 64), BF), _t((64, 6), BF))   # tp = 4: s = 6
    with pytest.raises(ValueError):
        binding.shared_mlp_slice_rank(wgu, wd, _t((6, 64), BF), good[1], 4, 0)
    with pytest.raises(ValueError):
        binding.shared_mlp_slice_rank(wgu, wd, good[0], _t((64, 12), BF), 4, 0)
    with pytest.raises(TypeError):
        binding.shared_mlp_slice_rank(wgu, wd, good[0], _t((64, 6), F32), 4, 0)
    with pytest.raises(ValueError):
        binding.shared_mlp_slice_rank(wgu, _t((64, 12), BF), *good, 4, 0)
    assert _reaches_launch(lambda: binding.shared_mlp_slice_rank(wgu, wd, *good, 4, 1))


def test_forward_rank_checks_types(L):
    x, wgu, wd = _layer(I=64)
    with pytest.raises(TypeError):
        binding.shared_mlp_forward_rank(x, wgu, wd, _t((4, 64), BF), 4, 0)
    with pytest.raises(TypeError):
        binding.shared_mlp_forward_rank(x, wgu.float(), wd, _t((4, 64), F32), 4, 0)
    assert _reaches_launch(lambda: binding.shared_mlp_forward_rank(x, wgu, wd, _t((4, 64), F32), 4, 0))


def test_workspace_size_is_counted_in_bytes(L):
    # a float32 workspace of n elements holds 4n bytes
    assert binding._ws_bytes(_t((10,), F32)) == 40
    assert binding._ws_bytes(_t((10,), torch.uint8)) == 10
    assert binding._ws_bytes(None) == 0


MS = [1, 2, 5, 8, 12, 16, 17, 20, 24, 31, 32, 33, 48, 64, 65, 100, 128, 129, 200, 256, 257, 300, 512, 1024,
      2048, 8192]
HS = [8, 16, 64, 1024, 4096, 7168, 8704, 16384]
IS = [8, 24, 64, 256, 384, 768, 1032, 1536, 4096, 6144, 8192]


@pytest.mark.parametrize("threshold", [None, 129])
def test_every_unpinned_plan_succeeds(L, threshold):
    """With nothing pinned, the planner has a compiled kernel for every legal shape:
    both dispatch thresholds, both output types, Kimi-K3 and off-model sizes."""
    prev = binding.shared_mlp_set_large_m_threshold(threshold) if threshold else None
    failed = []
    try:
        for M, H, I, partial in itertools.product(MS, HS, IS, (0, 1)):
            if 2 * I * H >= 1 << 31 or M * H >= 1 << 31 or M * I >= 1 << 31:
                continue
            try:
                p = binding.shared_mlp_plan(M, H, I, binding.SMLP_BF16, partial)
                assert p["workspace_bytes"] >= 0 and p["kernels"] >= 1
            except binding.SmlpError as e:
                failed.append((M, H, I, partial, str(e)))
    finally:
        if prev is not None:
            binding.shared_mlp_set_large_m_threshold(prev)
    assert not failed, f"{len(failed)} plans failed, e.g. {failed[:5]}"
