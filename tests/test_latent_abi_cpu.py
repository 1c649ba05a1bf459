"""Host-only tests of the merged MLA latent projection entry points (include/smlp_latent.h).

Every call either fails validation on the host before any HIP call, or is a pure
host planning function.  The geometry rejections follow vLLM PR 345, "[II] TP-shard
Kimi MLA latent projections", sections "Compatibility" and "Validation": range sizes
not divisible by tp, and gathered widths that are truncated or oversized, are errors.
"""
import ctypes
import os

import pytest

binding = pytest.importorskip("moe_shared_expert_amd.binding")

K, QA, KVA = 7168, 1536, 576
N = QA + KVA
GB = 1 << 30
X, W, Y, WS, G, O = (0x7e0000000000 + k * 4 * GB for k in range(6))
OK, NULL, SHAPE, ALIGN, ALIAS, WSP, DTYPE, ARG = 0, 1, 2, 3, 4, 5, 6, 8


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libsmlp.so is not built (python -m moe_shared_expert_amd.build)")
    return binding.lib()


def _lin(L, x=X, w=W, y=Y, m=16, k=K, n=N // 16, ldy=None, f32=0, ws=WS, wsb=1 << 40):
    return L.shared_mlp_linear(x, w, y, m, k, n, n if ldy is None else ldy, f32, ws, wsb, None)


def test_linear_validation_codes(L):
    assert _lin(L, f32=2) == DTYPE
    assert _lin(L, m=-1) == SHAPE
    assert _lin(L, k=7170) == SHAPE            # K % 8
    assert _lin(L, k=0) == SHAPE
    assert _lin(L, n=130) == SHAPE             # N % 4
    assert _lin(L, n=132, ldy=128) == SHAPE    # ldy < N
    assert _lin(L, n=132, ldy=2114) == SHAPE   # ldy % 4
    assert _lin(L, m=1 << 19, k=8192) == SHAPE  # M*K >= 2^31
    assert _lin(L, x=0) == NULL
    assert _lin(L, w=0) == NULL
    assert _lin(L, y=0) == NULL
    assert _lin(L, x=X + 8) == ALIGN
    assert _lin(L, y=Y + 4) == ALIGN           # bf16 y: 8-byte aligned
    assert _lin(L, y=Y + 8, f32=1) == ALIGN    # fp32 y: 16-byte aligned
    assert _lin(L, y=X) == ALIAS
    assert _lin(L, y=W + 4096) == ALIAS


def test_linear_workspace_rules(L):
    # M = 16 on the streaming kernel splits K: workspace needed, checked, not aliased
    p = binding.shared_mlp_linear_plan(16, K, N)
    # the K split is reduced in the same launch (last-arriving slice per column)...
    assert p["path_name"] == "small_m" and p["down_ksplit"] > 1 and p["kernels"] == 1
    try:   # ...or, with in-launch reductions switched off, by a finalize launch
        binding.shared_mlp_tune_layer_fusion(2, 0)
        assert binding.shared_mlp_linear_plan(16, K, N)["kernels"] == 2
    finally:
        binding.shared_mlp_tune_layer_fusion(0, 0)
    need = binding.shared_mlp_linear_workspace_bytes(16, K, N)
    assert need == p["workspace_bytes"] >= p["down_ksplit"] * 16 * N * 4
    assert _lin(L, n=N, ws=0) == NULL
    assert _lin(L, n=N, ws=WS + 16) == ALIGN
    assert _lin(L, n=N, wsb=need - 1) == WSP
    assert _lin(L, n=N, ws=X) == ALIAS
    assert _lin(L, n=N, y=WS) == ALIAS
    assert L.shared_mlp_linear(None, None, None, 0, K, N, N, 0, None, 0, None) == OK   # M == 0


def test_linear_plan_dispatch(L):
    assert binding.shared_mlp_linear_plan(0, K, N)["path_name"] == "none"
    for m in (1, 16, 32):
        assert binding.shared_mlp_linear_plan(m, K, N)["path_name"] == "small_m"
        assert binding.shared_mlp_linear_plan(m, K, N // 16)["path_name"] == "small_m"
    for m in (33, 128, 8192):
        assert binding.shared_mlp_linear_plan(m, K, N)["path_name"] == "large_m"
    # the small-M kernel never serves more than 32 tokens, whatever the MLP threshold
    prev = binding.shared_mlp_set_large_m_threshold(129)
    try:
        assert binding.shared_mlp_linear_plan(64, K, N)["path_name"] == "large_m"
        binding.shared_mlp_set_large_m_threshold(1)
        assert binding.shared_mlp_linear_plan(1, K, N)["path_name"] == "large_m"
    finally:
        binding.shared_mlp_set_large_m_threshold(prev)
    # tuning: pinned K split and tile count
    try:
        binding.shared_mlp_tune_skinny(2, kind=3, nb=2, waves=4, u=4, ksplit=4)
        p = binding.shared_mlp_linear_plan(16, K, N)
        assert p["down_ksplit"] == 4 and p["down_blocks"] == 4 * (N // 32)
        binding.shared_mlp_tune_skinny(2, nb=4, waves=8, u=5)   # not compiled
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_linear_plan(16, K, N)
        binding.shared_mlp_tune_skinny(2)
        binding.shared_mlp_tune_gemm(2, bm=128, bn=32, wm=4, wn=1, ns=2, ksplit=1)
        p = binding.shared_mlp_linear_plan(128, K, 132)
        assert p["down_ksplit"] == 1 and p["down_blocks"] == (132 + 31) // 32
    finally:
        binding.shared_mlp_tune_skinny(2)
        binding.shared_mlp_tune_gemm(2)


def _sizes(*v):
    return (ctypes.c_int64 * max(len(v), 1))(*v)


def _restore(L, g=G, o=O, m=16, n=N, sizes=(QA, KVA), tp=16, eb=2):
    return L.shared_mlp_restore_logical(g, o, m, n, _sizes(*sizes), len(sizes), tp, eb, None)


def test_restore_accepts_the_kimi_geometry(L):
    # valid geometry passes validation; M = 0 returns before touching a pointer
    assert L.shared_mlp_restore_logical(None, None, 0, N, _sizes(QA, KVA), 2, 16, 2, None) == OK


@pytest.mark.parametrize("sizes,tp", [((QA, KVA), 7), ((QA, KVA), 128), ((QA, 577), 16),
                                      ((0, KVA), 16), ((QA, -16), 16)])
def test_restore_rejects_non_divisible_geometry(L, sizes, tp):
    assert _restore(L, n=sum(sizes), sizes=sizes, tp=tp) == SHAPE


@pytest.mark.parametrize("width", [N - 1, N - 132, N + 1, 132, 0])
def test_restore_rejects_truncated_or_oversized_gather(L, width):
    assert _restore(L, n=width) == SHAPE
    assert "does not match" in L.shared_mlp_last_error().decode()


def test_restore_other_codes(L):
    assert _restore(L, tp=0) == SHAPE
    assert _restore(L, eb=3) == ARG
    assert _restore(L, sizes=()) == ARG
    assert _restore(L, sizes=(16,) * 9, n=144) == ARG
    assert L.shared_mlp_restore_logical(G, O, 16, N, None, 2, 16, 2, None) == NULL
    assert _restore(L, g=0) == NULL
    assert _restore(L, o=O + 1) == ALIGN
    assert _restore(L, eb=4, g=G + 2) == ALIGN
    assert _restore(L, o=G + 64) == ALIAS
    assert _restore(L, m=-1) == SHAPE
