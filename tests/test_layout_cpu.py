"""The library's per-step layout choice (include/smlp_layout.h, host-only) against the
oracle (oracle/layout.py) on random models, plus its validation.

Source: vLLM PR 50656, "[Kimi-K3] Add option to shard the shared expert instead of
replicating" (Change; Trade-off and why it is opt-in; Evaluation).
"""
import math
import os

import numpy as np
import pytest

import oracle

binding = pytest.importorskip("moe_shared_expert_amd.binding")
OL = oracle.layout


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libsmlp.so is not built (python -m moe_shared_expert_amd.build)")
    binding.lib()


def _random_model(rng):
    tp = int(rng.choice([2, 4, 8, 16]))
    hidden = int(rng.choice([16, 1024, 7168]))
    def curve():
        n = int(rng.integers(1, 7))
        ms = np.cumsum(rng.integers(1, 900, size=n)).astype(float)
        ts = np.sort(rng.uniform(1, 500, size=n)) if rng.random() < 0.8 else rng.uniform(1, 500, size=n)
        return list(ms), list(ts)
    return dict(tp=tp, hidden=hidden, rep_curve=curve(), shard_curve=curve(),
                alpha_us=float(rng.uniform(0, 30)), link_gbps=float(rng.uniform(20, 400)),
                links=int(rng.integers(1, 8)), partial_elem_bytes=int(rng.choice([2, 4])))


def test_times_and_choice_match_the_oracle():
    rng = np.random.Generator(np.random.PCG64(50656))
    for _ in range(200):
        kw = _random_model(rng)
        m = binding.layout_model(**kw)
        for T in list(rng.integers(1, 20000, size=8)) + [1, kw["tp"], kw["tp"] + 1]:
            T = int(T)
            r, s = binding.shared_mlp_layout_times(m, T)
            er, es = OL.step_times(T, kw["tp"], kw["hidden"], kw["rep_curve"], kw["shard_curve"], kw["alpha_us"],
                                   kw["link_gbps"] * 1e3, kw["links"], kw["partial_elem_bytes"])
            assert math.isclose(r, er, rel_tol=1e-12, abs_tol=1e-12), (kw, T)
            assert math.isclose(s, es, rel_tol=1e-12, abs_tol=1e-12), (kw, T)
            if abs(er - es) > 1e-9 * max(er, es):
                assert binding.shared_mlp_choose_layout(m, T) == (es < er)


def test_crossover_matches_the_oracle():
    rng = np.random.Generator(np.random.PCG64(94))
    checked = 0
    for _ in range(60):
        kw = _random_model(rng)
        m = binding.layout_model(**kw)
        got = binding.shared_mlp_layout_crossover(m, 3000)
        want = OL.crossover(3000, kw["tp"], kw["hidden"], kw["rep_curve"], kw["shard_curve"], kw["alpha_us"],
                            kw["link_gbps"] * 1e3, kw["links"], kw["partial_elem_bytes"])
        if got != want:   # only a tie within rounding may differ
            T = min(x for x in (got, want) if x) 
            er, es = OL.step_times(T, kw["tp"], kw["hidden"], kw["rep_curve"], kw["shard_curve"], kw["alpha_us"],
                                   kw["link_gbps"] * 1e3, kw["links"], kw["partial_elem_bytes"])
            assert abs(er - es) <= 1e-9 * max(er, es), (kw, got, want)
        checked += 1
    assert checked == 60


def test_worked_example():
    # TP8, H = 7168, T = 128: replicated rank runs 16 tokens; sharded rank runs 128 tokens
    # plus an all-gather (229376 bytes per peer) and an fp32 reduce-scatter (458752 bytes)
    m = binding.layout_model(8, 7168, ([1, 16, 128], [46.0, 48.0, 87.0]), ([1, 128, 1024], [14.0, 24.0, 110.0]),
                             10.0, 153.0, 7, 4)
    r, s = binding.shared_mlp_layout_times(m, 128)
    assert r == 48.0
    assert math.isclose(s, 24.0 + 10.0 + 229376 / 153000.0 + 10.0 + 458752 / 153000.0, rel_tol=1e-14)
    assert binding.shared_mlp_choose_layout(m, 128) == (s < r)


def test_validation():
    ok = dict(tp=8, hidden=7168, rep_curve=([1, 16], [40.0, 48.0]), shard_curve=([1, 128], [14.0, 24.0]),
              alpha_us=10.0, link_gbps=153.0, links=7, partial_elem_bytes=4)
    assert binding.shared_mlp_layout_crossover(binding.layout_model(**ok), 100) >= 0
    bad = [dict(tp=1), dict(hidden=0), dict(partial_elem_bytes=3), dict(alpha_us=-1.0), dict(link_gbps=0.0),
           dict(links=0), dict(rep_curve=([1, 1], [1.0, 2.0])), dict(shard_curve=([2, 1], [1.0, 2.0])),
           dict(rep_curve=([1], [float("nan")])), dict(shard_curve=([1], [-1.0])), dict(rep_curve=([], []))]
    for b in bad:
        m = binding.layout_model(**{**ok, **b})
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_layout_times(m, 16)
    m = binding.layout_model(**ok)
    for T in (0, -5):
        with pytest.raises(binding.SmlpError):
            binding.shared_mlp_choose_layout(m, T)
    with pytest.raises(binding.SmlpError):
        binding.shared_mlp_layout_crossover(m, 0)
    L = binding.lib()
    assert L.shared_mlp_layout_times(None, 16, None, None) == 1
