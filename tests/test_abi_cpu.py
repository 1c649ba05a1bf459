"""Host-only tests of libsmlp's C ABI: exports, validation, planning, gating.

No GPU is needed: every call here either fails validation (which happens on the
host before any HIP call) or is a pure host function.
"""
import ctypes
import itertools
import os
import re

import pytest

import oracle
from conftest import GOLDEN, ROOT

binding = pytest.importorskip("moe_shared_expert_amd.binding")

H, I = 7168, 6144
BF16, FP32 = binding.SMLP_BF16, binding.SMLP_FP32


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libsmlp.so is not built (python -m moe_shared_expert_amd.build)")
    return binding.lib()


def _declared(header):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(shared_mlp_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = _declared("smlp.h") + _declared("smlp_latent.h")
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(binding.EXPORTS), "binding and header disagree"
    tuning = _declared("smlp_tuning.h")
    for n in tuning:
        assert hasattr(L, n), n
    assert set(tuning) == set(binding.TUNING_EXPORTS)
    layout = _declared("smlp_layout.h")
    for n in layout:
        assert hasattr(L, n), n
    assert set(layout) == set(binding.LAYOUT_EXPORTS)
    ceil = _declared("smlp_ceilings.h")
    for n in ceil:
        assert hasattr(L, n), n
    assert set(ceil) == set(binding.CEILING_EXPORTS)
    # every header under include/ is covered above
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(
        ["smlp.h", "smlp_latent.h", "smlp_layout.h", "smlp_tuning.h", "smlp_ceilings.h"])


def test_tuning_hook(L):
    prev = binding.shared_mlp_set_large_m_threshold(129)   # M <= 128 on the streaming path
    try:
        binding.shared_mlp_tune_skinny(0, kind=3, nb=2, waves=4, u=4, ksplit=3)
        p = binding.shared_mlp_plan(16, H, I)
        assert p["gate_up_ksplit"] == 3 and p["gate_up_blocks"] == 3 * (I // 16)
        binding.shared_mlp_tune_skinny(0)
        p = binding.shared_mlp_plan(16, H, I)
        assert p["gate_up_ksplit"] == 1 and p["gate_up_blocks"] == 256
        binding.shared_mlp_tune_skinny(0, kind=2, nb=1, waves=4, u=1, ksplit=2)
        p = binding.shared_mlp_plan(64, H, I)
        assert p["gate_up_ksplit"] == 2 and p["gate_up_blocks"] == 2 * (I // 16)
        binding.shared_mlp_tune_skinny(0, kind=3, nb=1, waves=4, u=4, ksplit=1)
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_plan(64, H, I)   # the streaming kind serves M <= 32 only
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_tune_skinny(0, nb=5)
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_tune_skinny(0, kind=4)
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_tune_skinny(0, kind=1)   # retired kind
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_tune_skinny(3)
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_tune_skinny(2, kind=2)   # the projection streams only
    finally:
        binding.shared_mlp_tune_skinny(0)
        binding.shared_mlp_set_large_m_threshold(prev)


def test_default_threshold_and_gemm_tuning(L):
    # default dispatch: 32 tokens stream the weights, 33 take the tiled path
    assert binding.shared_mlp_plan(32, H, I)["path_name"] == "small_m"
    assert binding.shared_mlp_plan(33, H, I)["path_name"] == "large_m"
    # prefill: 256 x 256 tiles, one per workgroup, no K split
    p = binding.shared_mlp_plan(8192, H, I)
    assert p["gate_up_blocks"] == (8192 // 256) * (2 * I // 256) and p["gate_up_ksplit"] == 1
    # down: 256 x 256 tiles for the columns of three whole rounds over 256 CUs (768 tiles),
    # the last 1024 columns as one round of 128 x 128 tiles (512), a third launch
    assert p["down_blocks"] == 3 * 256 + (8192 // 128) * ((H - 3 * 256 * 256 // (8192 // 256)) // 128)
    # four launches: gate_up, the fp16 copy of w_down (fp16 h at this M), two down launches
    assert p["down_ksplit"] == 1 and p["kernels"] == 4
    assert p["workspace_bytes"] >= 8192 * I * 2 + H * I * 2
    # below the conversion threshold the weights are converted in registers instead
    prev = binding.shared_mlp_tune_weight_convert(1 << 30)
    try:
        q = binding.shared_mlp_plan(8192, H, I)
        assert q["kernels"] == 3 and q["workspace_bytes"] < p["workspace_bytes"]
        assert binding.shared_mlp_plan(8192, H, I, binding.SMLP_BF16, True)["kernels"] == 3   # bf16 h
    finally:
        binding.shared_mlp_tune_weight_convert(prev)
    with pytest.raises(binding.SmlpError):
        binding.shared_mlp_tune_weight_convert(0)
    # down from 7/8 of a round of 256 x 256 tiles: that tile, no K split; the columns
    # are split only while the last round is under 9/16 full
    p = binding.shared_mlp_plan(2048, H, I)           # 224 tiles, no full round
    assert p["down_blocks"] == 8 * (H // 256) and p["down_ksplit"] == 1
    for M in (4096, 6144):                             # last round 75% and 62.5% full
        p = binding.shared_mlp_plan(M, H, I)
        assert p["down_blocks"] == (M // 256) * (H // 256) and p["down_ksplit"] == 1, (M, p)
    p = binding.shared_mlp_plan(3072, H, I)           # 336 tiles, last round 31% full: split
    assert p["down_blocks"] != 12 * (H // 256) and p["kernels"] == 5, p
    p = binding.shared_mlp_plan(1536, H, I)           # 168 tiles: one round, no K split
    assert p["down_blocks"] == (1536 // 256) * (H // 256) and p["down_ksplit"] == 1, p
    # medium M: 256 x 256 tiles with the K split that fills about one round (at most 4)
    for M, gks, dks in ((512, 2, 4), (768, 1, 3), (1024, 1, 2), (1280, 1, 1), (1536, 2, 1)):
        p = binding.shared_mlp_plan(M, H, I)
        tm = (M + 255) // 256
        assert (p["gate_up_ksplit"], p["down_ksplit"]) == (gks, dks), (M, p)
        assert p["gate_up_blocks"] == tm * (2 * I // 256) * gks and p["down_blocks"] == tm * (H // 256) * dks, (M, p)
    # a TP shard's few weight tiles keep their own rules: gate_up on 128 x 256 tiles split to
    # about 224 workgroups (at most 12 slices), or under 16 such tiles on 8-wave 128 x 64
    # tiles split to about 192 (at most 6); the short-K down stage never split, 128 x 128
    # tiles once they outnumber the compute units, else 128 x 64
    for tp, M, bn, gks, dbn in ((8, 320, 256, 12, 64), (8, 512, 256, 9, 64), (8, 640, 256, 7, 128),
                                (8, 1024, 256, 4, 128), (8, 1536, 256, 3, 128), (16, 384, 64, 6, 64),
                                (16, 512, 64, 4, 64), (16, 1024, 256, 9, 128), (16, 2048, 256, 4, 128)):
        p = binding.shared_mlp_plan(M, H, I // tp, BF16, True)
        tm = (M + 127) // 128
        assert p["gate_up_ksplit"] == gks and p["gate_up_blocks"] == tm * (2 * I // tp // bn) * gks, (tp, M, p)
        assert p["down_ksplit"] == 1 and p["down_blocks"] == tm * (H // dbn) and p["kernels"] == 3, (tp, M, p)
    # a pinned down tile is never split
    binding.shared_mlp_tune_gemm(1, bm=256, bn=256, wm=2, wn=4, ns=2)
    try:
        p = binding.shared_mlp_plan(8192, H, I)
        assert p["down_blocks"] == (8192 // 256) * (H // 256) and p["kernels"] == 3
    finally:
        binding.shared_mlp_tune_gemm(1)
    try:
        binding.shared_mlp_tune_gemm(0, bm=128, bn=128, wm=2, wn=2, ns=4, ksplit=2)
        p = binding.shared_mlp_plan(512, H, I)
        assert p["gate_up_ksplit"] == 2 and p["gate_up_blocks"] == 2 * (512 // 128) * (2 * I // 128)
        binding.shared_mlp_tune_gemm(0, bm=128, bn=128, wm=2, wn=2, ns=5)   # not compiled
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_plan(512, H, I)
        for bad in (dict(bm=96, bn=128), dict(bm=128, bn=0), dict(bm=128, bn=128, wm=3, wn=1),
                    dict(ns=9), dict(ksplit=-1)):
            with pytest.raises(binding.SmlpError):
                binding.shared_mlp_tune_gemm(0, **bad)
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_tune_gemm(3)
    finally:
        binding.shared_mlp_tune_gemm(0)


def test_status_strings(L):
    for code, name in enumerate(["SMLP_OK", "SMLP_ERR_NULL", "SMLP_ERR_SHAPE", "SMLP_ERR_ALIGN",
                                 "SMLP_ERR_ALIAS", "SMLP_ERR_WORKSPACE", "SMLP_ERR_DTYPE",
                                 "SMLP_ERR_HIP", "SMLP_ERR_ARG"]):
        assert L.shared_mlp_status_string(code).decode() == name
    assert L.shared_mlp_status_string(99).decode() == "SMLP_ERR_UNKNOWN"


# Fake, never dereferenced device addresses, far apart and 256-byte aligned.
GB = 1 << 30
X, WGU, WD, OUT, WS = (0x7f0000000000 + k * 4 * GB for k in range(5))


def _ws(m, h, i, dt=BF16):
    return binding.shared_mlp_workspace_bytes(m, h, i, dt)


def _fwd(L, x=X, wgu=WGU, wd=WD, out=OUT, m=16, h=H, i=I, dt=BF16, partial=0, ws=WS, wsb=None):
    if wsb is None:
        try:
            wsb = _ws(m, h, i, dt)
        except binding.SmlpError:
            wsb = 1 << 40
    return L.shared_mlp_forward(x, wgu, wd, out, m, h, i, dt, partial, ws, wsb, None)


def test_forward_validation_codes(L):
    assert _fwd(L, dt=7) == 6                      # dtype
    assert _fwd(L, m=-1) == 2                      # shape
    assert _fwd(L, h=0) == 2
    assert _fwd(L, i=0) == 2
    assert _fwd(L, h=7170) == 2                    # bf16 needs H % 8
    assert _fwd(L, i=6148) == 2                    # bf16 needs I % 8
    assert _fwd(L, m=1 << 20, h=4096, i=64) == 2   # M*H >= 2^31
    assert _fwd(L, x=0) == 1                       # null
    assert _fwd(L, wgu=0) == 1
    assert _fwd(L, wd=0) == 1
    assert _fwd(L, out=0) == 1
    assert _fwd(L, ws=0) == 1
    assert _fwd(L, x=X + 8) == 3                   # bf16 needs 16-byte alignment
    assert _fwd(L, out=OUT + 2) == 3
    assert _fwd(L, ws=WS + 16) == 3                # workspace 256-byte aligned
    assert _fwd(L, wsb=_ws(16, H, I) - 1) == 5     # workspace too small
    assert _fwd(L, out=X) == 4                     # out aliases x
    assert _fwd(L, out=WGU + 1024) == 4            # out inside w_gate_up
    assert _fwd(L, out=WS) == 4                    # out aliases the workspace
    assert _fwd(L, ws=WD) == 4                     # workspace aliases w_down
    # fp32 inputs: any sizes, 4-byte alignment; misalignment below 4 still fails
    assert _fwd(L, dt=FP32, x=X + 2, m=3, h=5, i=3) == 3
    assert "alignment" in L.shared_mlp_last_error().decode() or "aligned" in L.shared_mlp_last_error().decode()


def test_m_zero_is_a_noop(L):
    # M == 0 returns OK before touching a pointer or the GPU
    assert L.shared_mlp_forward(None, None, None, None, 0, H, I, BF16, 0, None, 0, None) == 0
    assert L.shared_mlp_last_error().decode() == ""


def test_stage_entry_points_validate(L):
    wsb = _ws(16, H, I)
    assert L.shared_mlp_gate_up_act(0, WGU, 16, H, I, BF16, 0, WS, wsb, None) == 1
    assert L.shared_mlp_gate_up_act(X, WGU, 16, H, I, BF16, 0, X, wsb, None) == 4
    assert L.shared_mlp_down(WD, OUT, 16, H, I, BF16, 0, WS, 0, None) == 5
    assert L.shared_mlp_down(WD, WS, 16, H, I, BF16, 0, WS, wsb, None) == 4


def test_workspace_and_plan(L):
    p = binding.shared_mlp_plan(16, H, I)
    # decode: one bf16 plane of h; two planes (hi + lo) for a short down contraction,
    # or on request
    assert p["path_name"] == "small_m" and p["h_dtype"] == BF16
    assert p["workspace_bytes"] >= 16 * I * 2
    assert binding.shared_mlp_plan(16, H, 128)["h_dtype"] == binding.SMLP_BF16_HILO
    assert binding.shared_mlp_plan(8192, H, 128)["h_dtype"] == binding.SMLP_BF16_HILO
    try:
        binding.shared_mlp_tune_h_planes(2)
        q = binding.shared_mlp_plan(16, H, I)
        assert q["h_dtype"] == binding.SMLP_BF16_HILO and q["workspace_bytes"] >= 16 * I * 4
        binding.shared_mlp_tune_h_planes(1)
        assert binding.shared_mlp_plan(16, H, 128)["h_dtype"] == BF16
        prev = binding.shared_mlp_set_large_m_threshold(129)
        try:
            with pytest.raises(binding.SmlpError):   # one plane: M <= 32 on the small path
                binding.shared_mlp_plan(64, H, I)
            binding.shared_mlp_tune_h_planes(0)
            assert binding.shared_mlp_plan(64, H, I)["h_dtype"] == binding.SMLP_BF16_HILO
        finally:
            binding.shared_mlp_set_large_m_threshold(prev)
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_tune_h_planes(3)
    finally:
        binding.shared_mlp_tune_h_planes(0)
    p = binding.shared_mlp_plan(8192, H, I)   # bf16 output: h as one fp16 plane
    assert p["path_name"] == "large_m" and p["h_dtype"] == binding.SMLP_FP16
    assert p["workspace_bytes"] >= 8192 * I * 2
    # an fp32 partial keeps one bf16 plane; the tuning hook pins any format
    assert binding.shared_mlp_plan(8192, H, I, BF16, True)["h_dtype"] == BF16
    try:
        for fmt, want in ((1, BF16), (2, binding.SMLP_BF16_HILO), (3, binding.SMLP_FP16)):
            binding.shared_mlp_tune_h_format(fmt)
            assert binding.shared_mlp_plan(512, H, I)["h_dtype"] == want
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_tune_h_format(4)
    finally:
        binding.shared_mlp_tune_h_format(0)
    p = binding.shared_mlp_plan(12, 16, 12, FP32)
    assert p["path_name"] == "fp32"
    p = binding.shared_mlp_plan(0, H, I)
    assert p["path_name"] == "none" and p["kernels"] == 0
    # the TP-shard shapes need a K split to fill the chip
    p = binding.shared_mlp_plan(128, H, 384, BF16, True)
    assert p["gate_up_ksplit"] > 1
    assert p["workspace_bytes"] <= binding.shared_mlp_workspace_bytes(128, H, 384, BF16)


def test_threshold_setter(L):
    prev = binding.shared_mlp_set_large_m_threshold(64)
    try:
        assert binding.shared_mlp_plan(64, H, I)["path_name"] == "large_m"
        assert binding.shared_mlp_plan(63, H, I)["path_name"] == "small_m"
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_set_large_m_threshold(0)
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_set_large_m_threshold(1 << 20)
    finally:
        binding.shared_mlp_set_large_m_threshold(prev)


def test_shard_eligible_matches_oracle_exhaustively(L):
    for flag, sp, ok, tp, hid, inter in itertools.product(
            (0, 1), (0, 1), (0, 1), (0, 1, 2, 3, 4, 5, 8, 16), (16, 7168, 7170), (12, 6144, 6148)):
        assert binding.shared_mlp_shard_eligible(flag, sp, ok, tp, hid, inter) == \
            oracle.shard_sequence_parallel_mlp(flag, sp, ok, tp, hid, inter)


def test_shard_eligible_golden_cases(L):
    with open(os.path.join(GOLDEN, "gating_cases.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for flag, sp, ok, tp, hid, inter, expect, label in rows:
        assert binding.shared_mlp_shard_eligible(int(flag), int(sp), int(ok), int(tp), int(hid),
                                                 int(inter)) == bool(int(expect)), label


def test_slice_rank_validation(L):
    s = L.shared_mlp_slice_rank
    assert s(WGU, WD, OUT, WS, H, I, 8, 8, BF16, None) == 8      # rank out of range
    assert s(WGU, WD, OUT, WS, H, I, 5, 0, BF16, None) == 8      # 6144 % 5 != 0
    assert s(WGU, WD, OUT, WS, H, I, 0, 0, BF16, None) == 8
    assert s(0, WD, OUT, WS, H, I, 8, 0, BF16, None) == 1
    assert s(WGU, WD, WGU, WS, H, I, 8, 0, BF16, None) == 4      # dest aliases source
    assert s(WGU, WD, OUT, OUT + 64, H, I, 8, 0, BF16, None) == 4  # dests overlap
    assert s(WGU, WD, OUT, WS, H, I, 8, 0, 3, None) == 6


def test_rescale_validation(L):
    r = L.shared_mlp_rms_rescale
    assert r(X, OUT, 128, 7170, None) == 2
    assert r(X, OUT, -1, H, None) == 2
    assert r(0, OUT, 128, H, None) == 1
    assert r(X + 4, OUT, 128, H, None) == 3
    assert r(X, X + 64, 128, H, None) == 4
    assert r(None, None, 0, H, None) == 0


def test_forward_rank_validation(L):
    # every call below fails validation on the host (none may reach a launch)
    ws = _ws(16, H, I // 8)
    f = lambda **k: L.shared_mlp_forward_rank(k.get("x", X), k.get("g", WGU), k.get("d", WD), k.get("o", OUT),
                                              k.get("m", 16), H, k.get("i", I), k.get("tp", 8), k.get("r", 0),
                                              k.get("dt", BF16), k.get("ws", WS), k.get("wsb", ws), None)
    assert f(tp=0) == 8 and f(tp=7) == 8 and f(r=8) == 8 and f(r=-1) == 8     # SMLP_ERR_ARG
    assert f(i=6152, tp=8) == 2                    # the bf16 slice 769 is not a multiple of 8
    assert f(i=8 * 12, tp=8) == 2                  # bf16 slice of 12 is not a multiple of 8
    assert f(x=0) == 1 and f(o=0) == 1 and f(ws=0) == 1
    assert f(d=WD + 8) == 3
    assert f(wsb=ws - 1) == 5
    assert f(o=WD + 64) == 4 and f(ws=X) == 4
    assert f(dt=5) == 6
    assert L.shared_mlp_forward_rank(None, None, None, None, 0, H, I, 8, 0, BF16, None, 0, None) == 0


def test_last_error_is_per_thread(L):
    # each thread sees the detail of its own last failure (both calls fail validation on
    # the host: thread 0 an unknown dtype, thread 1 a misaligned x)
    import threading
    seen = {0: set(), 1: set()}

    def worker(k):
        for _ in range(200):
            if k == 0:
                rc = L.shared_mlp_forward(X, WGU, WD, OUT, 16, H, I, 7, 0, WS, 1 << 40, None)
            else:
                rc = L.shared_mlp_forward(X + 8, WGU, WD, OUT, 16, H, I, BF16, 0, WS, 1 << 40, None)
            seen[k].add((rc, L.shared_mlp_last_error().decode().split(" ")[0]))

    ts = [threading.Thread(target=worker, args=(k,)) for k in (0, 1)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert seen[0] == {(6, "dtype")}, seen[0]
    assert seen[1] == {(3, "x")}, seen[1]


def test_ceiling_kernels_validate_before_launch(L):
    # every case fails host validation, so no HIP call is made (no GPU here)
    NULL_, SHAPE, ALIGN, ARG = 1, 2, 3, 8
    p = ctypes.c_void_p(1 << 20)       # aligned, never dereferenced
    odd = ctypes.c_void_p((1 << 20) + 8)
    nul = ctypes.c_void_p(0)
    s = ctypes.c_void_p(0)
    assert L.shared_mlp_ceiling_empty(0, s) == ARG
    assert L.shared_mlp_ceiling_empty(65536, s) == ARG
    assert L.shared_mlp_ceiling_read(nul, 1 << 20, 1, 1024, 0, p, s) == NULL_
    assert L.shared_mlp_ceiling_read(odd, 1 << 20, 1, 1024, 0, p, s) == ALIGN
    assert L.shared_mlp_ceiling_read(p, 1 << 20, 1, 1000, 0, p, s) == ARG
    assert L.shared_mlp_ceiling_read(p, 1 << 20, 2048, 1024, 0, p, s) == SHAPE
    assert L.shared_mlp_ceiling_mfma(1, 1, nul, p, p, s) == NULL_
    assert L.shared_mlp_ceiling_mfma(1, 0, p, p, p, s) == ARG
    assert L.shared_mlp_ceiling_lds(1, 1, p, nul, s) == NULL_
    assert L.shared_mlp_ceiling_lds(0, 1, p, p, s) == ARG
    for barrier in (-1, 3):
        assert L.shared_mlp_ceiling_two_phase(p, 1 << 30, 256, 1024, barrier, p, p, s) == ARG
    assert L.shared_mlp_ceiling_two_phase(p, 1 << 30, 256, 1024, 2, nul, p, s) == NULL_
    assert L.shared_mlp_ceiling_two_phase(p, 1 << 30, 257, 1024, 0, p, p, s) == ARG
    assert L.shared_mlp_ceiling_two_phase(p, 1 << 20, 256, 4096, 0, p, p, s) == SHAPE


def test_layer_fusion_plan_and_hook(L):
    """The one-launch decode layer: one kernel for the fused configurations (M <= 32, one
    plane of h, the Kimi-K3 stage tiles), two when it is switched off or does not apply;
    the hook validates its mode before any state changes."""
    try:
        for M in (1, 8, 16, 17, 32):
            assert binding.shared_mlp_plan(M, H, I)["kernels"] == 1
            assert binding.shared_mlp_plan(M, H, I, BF16, True)["kernels"] == 1
        assert binding.shared_mlp_plan(16, 4096, I)["kernels"] == 2   # down tile of another width
        assert binding.shared_mlp_plan(16, H, 128)["kernels"] >= 2     # two planes of h
        binding.shared_mlp_tune_h_planes(2)
        assert binding.shared_mlp_plan(16, H, I)["kernels"] == 2
        binding.shared_mlp_tune_h_planes(0)
        assert binding.shared_mlp_plan(12, 16, 12, FP32)["kernels"] == 1      # one-workgroup fp32 layer
        assert binding.shared_mlp_plan(40, 64, 100, FP32)["kernels"] == 1
        assert binding.shared_mlp_plan(41, 64, 100, FP32)["kernels"] == 2     # h past 4096 floats
        assert binding.shared_mlp_plan(16, 4096, 64, FP32)["kernels"] == 2    # past 2^20 multiply-adds
        binding.shared_mlp_tune_layer_fusion(2, 0)
        assert binding.shared_mlp_plan(12, 16, 12, FP32)["kernels"] == 2
        assert binding.shared_mlp_plan(16, H, I)["kernels"] == 2
        binding.shared_mlp_tune_layer_fusion(1, 1000)
        assert binding.shared_mlp_plan(16, H, I)["kernels"] == 1
        for bad in (-1, 3):
            with pytest.raises(binding.SmlpError):
                binding.shared_mlp_tune_layer_fusion(bad, 0)
    finally:
        binding.shared_mlp_tune_h_planes(0)
        binding.shared_mlp_tune_layer_fusion(0, 0)


def test_pinned_streaming_shape_takes_the_finalize_launch(L):
    """A K-split streaming stage is reduced in its own launch with the planner's shapes or a
    pinned K split alone; a pinned tile count, wave count or ring depth takes the finalize
    launch (one more kernel), for the layer stages and the projection alike."""
    I16 = I // 16   # a TP16 shard: the default gate_up splits K four ways at M = 16
    try:
        base = binding.shared_mlp_plan(16, H, I16, BF16, True)
        assert base["gate_up_ksplit"] > 1 and base["kernels"] == 2
        binding.shared_mlp_tune_skinny(0, ksplit=3)
        assert binding.shared_mlp_plan(16, H, I16, BF16, True)["kernels"] == 2
        for pin in (dict(kind=3, nb=2), dict(kind=3, waves=8), dict(kind=3, nb=3, u=5)):
            binding.shared_mlp_tune_skinny(0, ksplit=3, **pin)
            p = binding.shared_mlp_plan(16, H, I16, BF16, True)
            assert p["gate_up_ksplit"] == 3 and p["kernels"] == 3, (pin, p)
        binding.shared_mlp_tune_skinny(0)
        binding.shared_mlp_tune_skinny(2, ksplit=4)
        assert binding.shared_mlp_linear_plan(16, H, 2112)["kernels"] == 1
        binding.shared_mlp_tune_skinny(2, kind=3, nb=2, waves=4, u=4, ksplit=4)
        assert binding.shared_mlp_linear_plan(16, H, 2112)["kernels"] == 2
    finally:
        binding.shared_mlp_tune_skinny(0)
        binding.shared_mlp_tune_skinny(2)
