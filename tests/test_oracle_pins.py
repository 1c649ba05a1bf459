"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes the oracle to something independent: brute-force loops on tiny
inputs, scalar closed forms evaluated with the math module, special cases that
reduce to a known result, the sharded-equals-replicated invariant of vLLM PR
50656 ("[Kimi-K3] Add option to shard the shared expert instead of
replicating", sections "Change" and "Testing"), the rejected feature-concat
design described there, and the printed gating cases and byte counts.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from moe_shared_expert_amd import roofline

from conftest import GOLDEN

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _brute(x, wgu, wd):
    """Per-token, per-feature Python loops with math.exp; no numpy arithmetic."""
    m_dim, h_dim = len(x), len(x[0])
    i_dim = len(wgu) // 2
    out = []
    for m in range(m_dim):
        h = []
        for i in range(i_dim):
            g = 0.0
            u = 0.0
            for k in range(h_dim):
                g += x[m][k] * wgu[i][k]
                u += x[m][k] * wgu[i_dim + i][k]
            # silu(g) = g * sigmoid(g); sigmoid via the form that cannot overflow
            if g >= 0:
                sg = 1.0 / (1.0 + math.exp(-g))
            else:
                e = math.exp(g)
                sg = e / (1.0 + e)
            h.append(g * sg * u)
        row = []
        for n in range(h_dim):
            acc = 0.0
            for i in range(i_dim):
                acc += h[i] * wd[n][i]
            row.append(acc)
        out.append(row)
    return np.array(out, dtype=np.float64)


@pytest.mark.parametrize("m,h,i,seed", [
    (1, 1, 1, 1), (3, 4, 3, 2), (12, 16, 12, 3), (5, 7, 9, 4), (2, 16, 1, 5), (1, 3, 12, 6),
])
def test_brute_force_tiny(m, h, i, seed):
    r = _rng(seed)
    x = r.standard_normal((m, h))
    wgu = r.standard_normal((2 * i, h))
    wd = r.standard_normal((h, i))
    ref = _brute(x.tolist(), wgu.tolist(), wd.tolist())
    got = oracle.swiglu_mlp(x, wgu, wd)
    assert got.shape == (m, h)
    scale = max(1.0, float(np.abs(ref).max()))
    assert np.abs(got - ref).max() <= 1e-12 * scale


@pytest.mark.parametrize("x,wg,wu,wd", [
    (1.0, 1.0, 2.0, 3.0), (2.0, -1.0, 0.5, -4.0), (-0.75, 3.0, 1.25, 0.5), (0.5, 0.0, 7.0, 1.0),
])
def test_scalar_closed_form(x, wg, wu, wd):
    # M = H = I = 1: out = wd * silu(wg x) * (wu x), silu(g) = g / (1 + e^-g)
    g = wg * x
    expect = wd * (g / (1.0 + math.exp(-g))) * (wu * x)
    got = oracle.swiglu_mlp(np.array([[x]]), np.array([[wg], [wu]]), np.array([[wd]]))
    assert got.shape == (1, 1)
    assert abs(got[0, 0] - expect) <= 1e-15 * max(1.0, abs(expect))


def test_sigmoid_identities():
    g = np.linspace(-30, 30, 601)
    s = oracle.silu(g)
    # silu(g) - silu(-g) = g * (sigma(g) + sigma(-g)) = g
    assert np.abs((s - oracle.silu(-g)) - g).max() <= 1e-13
    # silu(0) = 0 exactly, silu(g) -> g for large g, -> -0 for g below -709
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) <= 40.0 * 1e-16
    z = oracle.silu(np.array([-800.0]))[0]
    assert z == 0.0 and math.copysign(1.0, z) < 0
    # Taylor series at 0: silu(e) = e/2 + e^2/4 + O(e^4)
    e = 1e-6
    assert abs(oracle.silu(np.array([e]))[0] - (e / 2 + e * e / 4)) <= 1e-21


def test_gate_is_first_half():
    # Gate row -50 suppresses the output (silu(-50) ~ -1e-20); the same numbers
    # with gate and up swapped give silu(1) * (-50).
    x = np.array([[1.0]])
    wd = np.array([[1.0]])
    out = oracle.swiglu_mlp(x, np.array([[-50.0], [1.0]]), wd)[0, 0]
    assert abs(out) < 1e-18
    swapped = oracle.swiglu_mlp(x, np.array([[1.0], [-50.0]]), wd)[0, 0]
    assert abs(swapped - (-50.0 / (1.0 + math.exp(-1.0)))) < 1e-12


def test_zero_operands_give_exact_zero():
    r = _rng(7)
    x = r.standard_normal((6, 10))
    wgu = r.standard_normal((16, 10))
    wd = r.standard_normal((10, 8))
    for zx, zg, zu, zd in [(1, 0, 0, 0), (0, 1, 0, 0), (0, 0, 1, 0), (0, 0, 0, 1)]:
        xx = np.zeros_like(x) if zx else x
        w = wgu.copy()
        if zg:
            w[:8] = 0.0
        if zu:
            w[8:] = 0.0
        dd = np.zeros_like(wd) if zd else wd
        out = oracle.swiglu_mlp(xx, w, dd)
        assert np.all(out == 0.0)


def test_down_identity_and_permutation():
    r = _rng(8)
    n = 9
    x = r.standard_normal((4, n))
    wgu = r.standard_normal((2 * n, n))
    g = x @ wgu[:n].T
    u = x @ wgu[n:].T
    h_expect = g / (1.0 + np.exp(-g)) * u
    out = oracle.swiglu_mlp(x, wgu, np.eye(n))
    assert np.abs(out - h_expect).max() <= 1e-14
    # down = permutation matrix P with P[j, perm[j]] = 1: out[:, j] = h[:, perm[j]].
    # A transposed down operand would give the inverse permutation instead.
    perm = np.array([3, 0, 7, 1, 8, 2, 6, 4, 5])
    p = np.zeros((n, n))
    p[np.arange(n), perm] = 1.0
    out = oracle.swiglu_mlp(x, wgu, p)
    assert np.abs(out - h_expect[:, perm]).max() <= 1e-14
    assert np.abs(out - h_expect[:, np.argsort(perm)]).max() > 1e-3


def test_large_gate_limit_is_relu_bilinear():
    # silu(c g) / c -> max(g, 0) as c grows: out/c -> ((xWg^T)^+ * xWu^T) Wd^T
    r = _rng(9)
    x = r.standard_normal((5, 6))
    wgu = r.standard_normal((8, 6))
    wd = r.standard_normal((6, 4))
    c = 1e4
    w = wgu.copy()
    w[:4] *= c
    g = x @ wgu[:4].T
    assert np.abs(g).min() > 1e-3
    expect = (np.maximum(g, 0.0) * (x @ wgu[4:].T)) @ wd.T
    got = oracle.swiglu_mlp(x, w, wd) / c
    assert np.abs(got - expect).max() <= 1e-10 * max(1.0, np.abs(expect).max())


def test_linear_in_up_and_down_not_in_gate():
    r = _rng(10)
    x = r.standard_normal((3, 5))
    wgu = r.standard_normal((12, 5))
    wd = r.standard_normal((5, 6))
    base = oracle.swiglu_mlp(x, wgu, wd)
    w2 = wgu.copy()
    w2[6:] *= 3.0
    assert np.allclose(oracle.swiglu_mlp(x, w2, wd), 3.0 * base, rtol=1e-13, atol=1e-14)
    assert np.allclose(oracle.swiglu_mlp(x, wgu, -2.0 * wd), -2.0 * base, rtol=1e-13, atol=1e-14)
    w3 = wgu.copy()
    w3[:6] *= 3.0
    assert not np.allclose(oracle.swiglu_mlp(x, w3, wd), 3.0 * base, rtol=1e-3)


def test_intermediate_permutation_and_token_permutation():
    r = _rng(11)
    m, h, i = 7, 6, 10
    x = r.standard_normal((m, h))
    wgu = r.standard_normal((2 * i, h))
    wd = r.standard_normal((h, i))
    base = oracle.swiglu_mlp(x, wgu, wd)
    p = r.permutation(i)
    wgu_p = np.concatenate([wgu[:i][p], wgu[i:][p]])
    assert np.abs(oracle.swiglu_mlp(x, wgu_p, wd[:, p]) - base).max() <= 1e-13
    # permuting only the up rows (not jointly) must change the result
    wgu_bad = np.concatenate([wgu[:i], wgu[i:][p]])
    assert np.abs(oracle.swiglu_mlp(x, wgu_bad, wd) - base).max() > 1e-3
    q = r.permutation(m)
    assert np.abs(oracle.swiglu_mlp(x[q], wgu, wd) - base[q]).max() <= 1e-13


def test_rank_shard_layout():
    # rank r holds gate rows r*s..(r+1)*s then up rows I + r*s.., and down columns r*s..
    i_dim, h_dim, tp = 12, 5, 4
    s = i_dim // tp
    wgu = np.arange(2 * i_dim * h_dim, dtype=np.float64).reshape(2 * i_dim, h_dim)
    wd = np.arange(h_dim * i_dim, dtype=np.float64).reshape(h_dim, i_dim) + 1000
    for r in range(tp):
        wgu_r, wd_r = oracle.rank_shard(wgu, wd, tp, r)
        assert wgu_r.shape == (2 * s, h_dim) and wd_r.shape == (h_dim, s)
        for j in range(s):
            assert wgu_r[j, 0] == (r * s + j) * h_dim
            assert wgu_r[s + j, 0] == (i_dim + r * s + j) * h_dim
            assert wd_r[0, j] == 1000 + r * s + j
    with pytest.raises(ValueError):
        oracle.rank_shard(wgu, wd, 5, 0)


def test_tiny_case_slices_sum_to_replicated():
    # The pages' equivalence test shapes: tp=4, hidden 16, intermediate 12,
    # 3 tokens per rank, seed 0, draws x, gate, up, down.
    x, gate, up, down, tp, t = synth.tiny_fp32_case()
    x64, wgu64, wd64 = synth.to_f64(x), synth.to_f64(synth.merged_gate_up(gate, up)), synth.to_f64(down)
    rep = oracle.swiglu_mlp(x64, wgu64, wd64)
    summed = oracle.slice_sum(x64, wgu64, wd64, tp)
    rms = np.sqrt(np.mean(rep ** 2))
    assert np.abs(summed - rep).max() <= 1e-13 * rms
    for r in range(tp):
        mine = oracle.rank_token_rows(summed, tp, r)
        assert np.abs(mine - rep[r * t:(r + 1) * t]).max() <= 1e-13 * rms


@pytest.mark.parametrize("tp", [2, 3, 4, 6, 12])
def test_slice_sum_invariant_random(tp):
    r = _rng(100 + tp)
    i_dim = 12 * 4
    x = r.standard_normal((8, 24))
    wgu = r.standard_normal((2 * i_dim, 24))
    wd = r.standard_normal((24, i_dim))
    rep = oracle.swiglu_mlp(x, wgu, wd)
    assert np.abs(oracle.slice_sum(x, wgu, wd, tp) - rep).max() <= 1e-12 * np.sqrt(np.mean(rep ** 2))


def test_feature_concat_design_fails_only_with_disjoint_tokens():
    x, gate, up, down, tp, t = synth.tiny_fp32_case()
    x64, wgu64, wd64 = synth.to_f64(x), synth.to_f64(synth.merged_gate_up(gate, up)), synth.to_f64(down)
    rep = oracle.swiglu_mlp(x64, wgu64, wd64)
    rms = np.sqrt(np.mean(rep ** 2))
    disjoint = [x64[q * t:(q + 1) * t] for q in range(tp)]
    wrong = oracle.feature_concat_design(disjoint, wgu64, wd64)
    worst = max(np.abs(wrong - rep[r * t:(r + 1) * t]).max() for r in range(tp))
    assert worst > 0.1 * rms
    # every rank holding the same tokens hides the bug
    same = [x64[:t]] * tp
    assert np.abs(oracle.feature_concat_design(same, wgu64, wd64) - rep[:t]).max() <= 1e-13 * rms
    # the correct design (gather tokens, sum partials) passes on the disjoint shards
    summed = oracle.slice_sum(x64, wgu64, wd64, tp)
    assert max(np.abs(oracle.rank_token_rows(summed, tp, r) - rep[r * t:(r + 1) * t]).max()
               for r in range(tp)) <= 1e-13 * rms


def test_rms_rescale_rows():
    r = _rng(12)
    a = r.standard_normal((6, 33)) * np.array([[0.1], [1], [10], [3], [1e-3], [7]])
    y = oracle.rms_rescale_rows(a)
    assert np.abs(np.sqrt(np.mean(y ** 2, axis=1)) - 1.0).max() <= 1e-14
    assert np.abs(oracle.rms_rescale_rows(5.0 * a) - y).max() <= 1e-14
    assert np.abs(oracle.rms_rescale_rows(-a) + y).max() == 0.0
    # a row of n equal values c rescales to sign(c)
    assert np.all(oracle.rms_rescale_rows(np.full((1, 4), -2.5)) == -1.0)
    with pytest.raises(ValueError):
        oracle.rms_rescale_rows(np.zeros((2, 3)))


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_gating_truth_table():
    rows = _read_table("gating_cases.txt")
    assert len(rows) == 6
    for flag, sp, ok, tp, hid, inter, expect, _label in rows:
        got = oracle.shard_sequence_parallel_mlp(bool(int(flag)), bool(int(sp)), bool(int(ok)),
                                                  int(tp), int(hid), int(inter))
        assert got == bool(int(expect)), _label


def test_printed_byte_counts_pin_the_accounting():
    units = {"MB": 1e6, "GiB": 2.0 ** 30}
    for name, hid, inter, layers, printed, unit in _read_table("kimi_k3_bytes.txt"):
        hid, inter, layers = int(hid), int(inter), int(layers)
        b = {"gate_up": roofline.gate_up_bytes(hid, inter),
             "down": roofline.down_bytes(hid, inter),
             "per_layer": roofline.weight_bytes(hid, inter),
             "stack": layers * roofline.weight_bytes(hid, inter)}[name]
        assert round(b / units[unit], 1) == float(printed), name


def test_roofline_bound_and_ridge():
    """The per-layer roofline: HBM-bound while 6*M*H*I flops at 2.5 PFLOP/s take less
    than the algorithmic bytes at 8 TB/s.  Hand-worked: replicated decode M = 16 moves
    3*7168*6144*2 + 2*16*7168*2 bytes = 264,699,904 B -> 33.087 us; prefill M = 8192
    does 6*8192*7168*6144 = 2.1646e12 flops -> 865.9 us.  The replicated ridge in M
    (3*M*I / (3*I + 2*M) = 312.5 flop/B at 2.5e15 / 8e12) lies between 256 and 512."""
    b, t = roofline.roofline_us(16, 7168, 6144)
    assert b == "hbm" and abs(t - 264699904 / 8e6) < 1e-9
    b, t = roofline.roofline_us(8192, 7168, 6144)
    assert b == "mfma" and abs(t - 6 * 8192 * 7168 * 6144 / 2.5e9) < 1e-6
    assert roofline.roofline_us(256, 7168, 6144)[0] == "hbm"
    assert roofline.roofline_us(512, 7168, 6144)[0] == "mfma"
    # a TP8 rank's fp32 partial (4-byte output) stays HBM-bound through M = 512
    assert roofline.roofline_us(512, 7168, 768, 4)[0] == "hbm"
    assert roofline.roofline_us(2048, 7168, 768, 4)[0] == "mfma"


def test_statistical_output_scale():
    """x ~ N(0,1), W ~ N(0, 1/fan_in) gives RMS(out) ~ sqrt(E[silu(g)^2] * I_r / I)
    with g ~ N(0,1); E[silu^2] by quadrature.  Pins the generator's std and
    fan-in together with the oracle's scale."""
    from scipy import integrate
    e_silu2, _ = integrate.quad(
        lambda g: (g / (1.0 + math.exp(-g))) ** 2 * math.exp(-g * g / 2) / math.sqrt(2 * math.pi),
        -40, 40)
    assert 0.35 < e_silu2 < 0.36
    hid, inter = 1024, 768
    x = synth.to_f64(synth.activations(48, hid, config=99))
    wgu, wd = synth.layer_weights(hid, inter, config=99)
    out = oracle.swiglu_mlp(x, synth.to_f64(wgu), synth.to_f64(wd))
    rms = float(np.sqrt(np.mean(out ** 2)))
    assert abs(rms / math.sqrt(e_silu2) - 1.0) < 0.05
    # a slice of s intermediate units of the same layer scales by sqrt(s / I)
    tp = 8
    part = oracle.rank_partial(x, synth.to_f64(wgu), synth.to_f64(wd), tp, 3)
    rms_p = float(np.sqrt(np.mean(part ** 2)))
    assert abs(rms_p / math.sqrt(e_silu2 / tp) - 1.0) < 0.08


def test_synth_is_deterministic_and_bf16():
    a = synth.activations(4, 64, config=2)
    b = synth.activations(4, 64, config=2)
    assert a.dtype == torch.bfloat16 and torch.equal(a, b)
    assert not torch.equal(a, synth.activations(4, 64, config=2, copy=1))
