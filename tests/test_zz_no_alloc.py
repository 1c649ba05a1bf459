"""The allocation-free entry point (shared_mlp_forward_noalloc) against the existing
entry point (shared_mlp_forward with a workspace), through the C ABI.

It runs the same kernels on the library's static per-GPU scratch array instead of a
caller workspace, so its output must equal shared_mlp_forward's bit for bit (same plan,
same summation order), and both must meet the parity bar against the fp64 oracle.  Two
calls in a row, the second with a smaller input, check that nothing of the first call's
scratch contents leaks into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import BF16_TOL, DEV, FP32_TOL, H, assert_rms_close, f64, workspace_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def binding():
    from moe_shared_expert_amd import binding as b
    b.lib()
    return b


def _both(binding, x, wgu, wd, partial):
    M, Hh = x.shape
    Ii = wgu.shape[0] // 2
    dt = binding.SMLP_FP32 if x.dtype == torch.float32 else binding.SMLP_BF16
    odt = torch.float32 if (partial or x.dtype == torch.float32) else torch.bfloat16
    ref_out = torch.full((M, Hh), float("nan"), dtype=odt, device=DEV)
    binding.shared_mlp_forward(x, wgu, wd, ref_out, partial, workspace_for(M, Hh, Ii, dt))
    out = torch.full((M, Hh), float("nan"), dtype=odt, device=DEV)
    # straight through the C ABI
    L = binding.lib()
    rc = L.shared_mlp_forward_noalloc(x.data_ptr(), wgu.data_ptr(), wd.data_ptr(), out.data_ptr(), M, Hh, Ii, dt,
                                      int(partial), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, (rc, L.shared_mlp_last_error())
    torch.cuda.synchronize()
    return out, ref_out


def _case(binding, M, Hh, Ii, partial, cfg, copy):
    x = synth.activations(M, Hh, config=cfg, copy=copy)
    wgu, wd = synth.layer_weights(Hh, Ii, config=cfg, copy=copy, fan_in_down=6144 if Hh == H else None)
    out, ref_out = _both(binding, x.to(DEV), wgu.to(DEV), wd.to(DEV), partial)
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                       ref_out.view(torch.int16) if out.dtype == torch.bfloat16 else ref_out.view(torch.int32))
    assert_rms_close(out, oracle.swiglu_mlp(f64(x), f64(wgu), f64(wd)), BF16_TOL, f"noalloc M={M} I={Ii}")


def test_two_calls_second_smaller(binding):
    # the TP8 shard at M = 128 (h and K-split partials in the scratch), then the
    # replicated decode layer at M = 16 (h only, a smaller region of it)
    _case(binding, 128, H, 768, True, 3, 0)
    _case(binding, 16, H, 6144, False, 2, 0)


def test_two_calls_small_shapes(binding):
    _case(binding, 300, 1032, 392, False, 12, 1)
    _case(binding, 7, 1032, 392, True, 12, 2)


def test_tiny_fp32(binding):
    x, gate, up, down, _, _ = synth.tiny_fp32_case()
    wgu = synth.merged_gate_up(gate, up)
    out, ref_out = _both(binding, x.to(DEV), wgu.to(DEV), down.to(DEV), False)
    assert torch.equal(out, ref_out)
    assert_rms_close(out, oracle.swiglu_mlp(f64(x), f64(wgu), f64(down)), FP32_TOL, "noalloc tiny fp32")


def test_rejects_plans_beyond_the_scratch(binding):
    # the M = 8192 prefill needs ~96 MiB of h: refused before any launch
    assert binding.shared_mlp_plan(8192, H, 6144)["workspace_bytes"] > 32 << 20
    x = torch.empty(8192, H, dtype=torch.bfloat16, device=DEV)
    wgu = torch.empty(2 * 6144, H, dtype=torch.bfloat16, device=DEV)
    wd = torch.empty(H, 6144, dtype=torch.bfloat16, device=DEV)
    out = torch.full((8192, H), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(binding.SmlpError) as e:
        binding.shared_mlp_forward_noalloc(x, wgu, wd, out)
    assert e.value.status == 5   # SMLP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
