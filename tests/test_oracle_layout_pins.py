"""Pins of the layout-choice oracle (oracle/layout.py) against facts outside it.

Source: vLLM PR 50656, "[Kimi-K3] Add option to shard the shared expert instead of
replicating" (Change; Trade-off and why it is opt-in; Evaluation).  Pins: the
interpolation on functions it must reproduce exactly, a hand-worked collective cost,
the limits of the decision (free collectives, infinitely slow collectives), and the
pages' qualitative finding that sharding pays off for small token counts only: with a
weight-bound replicated curve and a shard curve that grows with T, the choice flips
once, from sharded to replicated.
"""
import math

import pytest

import oracle

L = oracle.layout


def test_interp_reproduces_linear_functions_and_ends():
    ms = [1, 8, 32, 128]
    ts = [3 + 0.5 * m for m in ms]
    for m in (1, 2, 7.5, 8, 20, 100, 128):
        assert math.isclose(L.interp(ms, ts, m), 3 + 0.5 * m, rel_tol=1e-15)
    assert L.interp(ms, ts, 0.25) == ts[0]                      # below the first point
    assert math.isclose(L.interp(ms, ts, 1000), 3 + 0.5 * 1000)  # extrapolated last segment
    # a decreasing last segment is not extrapolated below the last value
    assert L.interp([1, 2], [5.0, 4.0], 10) == 4.0
    assert L.interp([4], [7.0], 100) == 7.0
    with pytest.raises(ValueError):
        L.interp([1, 1], [1, 2], 1)
    with pytest.raises(ValueError):
        L.interp([], [], 1)


def test_interp_by_hand():
    # between (8, 10) and (32, 34): at 14 the value is 10 + 24 * 6 / 24 = 16
    assert L.interp([1, 8, 32], [9.0, 10.0, 34.0], 14) == 16.0


def test_collective_cost_worked_example():
    # T = 128 tokens over tp = 8 ranks, H = 7168: 16 rows per chunk; bf16 chunk =
    # 16 * 7168 * 2 = 229376 bytes, fp32 chunk = 458752 bytes; 7 peers over 7 links is
    # one round; at 153 GB/s = 153000 bytes/us: 1.4992 us and 2.9984 us, plus alpha
    ag = L.collective_us(128, 8, 7168, 2, 10.0, 153000.0, 7)
    rs = L.collective_us(128, 8, 7168, 4, 10.0, 153000.0, 7)
    assert math.isclose(ag, 10.0 + 229376 / 153000.0, rel_tol=1e-15)
    assert math.isclose(rs, 10.0 + 458752 / 153000.0, rel_tol=1e-15)
    # 15 peers over 7 links: three rounds
    assert math.isclose(L.collective_us(160, 16, 7168, 2, 0.0, 1.0, 7), 3 * 10 * 7168 * 2)
    # ragged T: the largest chunk counts
    assert L.collective_us(129, 8, 1, 1, 0.0, 1.0, 7) == 17.0
    with pytest.raises(ValueError):
        L.collective_us(128, 1, 7168, 2, 0, 1, 7)


REP = ([1, 16, 128, 1024, 8192], [46.0, 48.0, 87.0, 400.0, 1913.0])      # flat, then compute-bound
SHARD = ([1, 16, 128, 1024, 8192], [14.0, 15.0, 24.0, 110.0, 418.0])


def test_decision_limits():
    # free collectives: shard exactly when the shard kernel alone is faster
    for T in (1, 64, 512, 4096, 20000):
        t_rep, t_shard = L.step_times(T, 8, 7168, REP, SHARD, 0.0, 1e30, 7)
        kr = L.interp(*REP, math.ceil(T / 8))
        ks = L.interp(*SHARD, T)
        assert math.isclose(t_rep, kr) and math.isclose(t_shard, ks, rel_tol=1e-12)
        assert L.choose_sharded(T, 8, 7168, REP, SHARD, 0.0, 1e30, 7) == (ks < kr)
    # collectives that never finish: never shard
    assert L.crossover(4096, 8, 7168, REP, SHARD, 1e12, 153000.0, 7) == 1


def test_sharding_wins_only_at_low_token_counts():
    # the choice flips once, from sharded to replicated, and a larger collective latency
    # moves the crossover down
    prev = None
    for alpha in (2.0, 5.0, 10.0, 15.0):
        Tc = L.crossover(65536, 8, 7168, REP, SHARD, alpha, 153000.0, 7)
        assert Tc > 1
        assert all(L.choose_sharded(T, 8, 7168, REP, SHARD, alpha, 153000.0, 7) for T in range(1, Tc, 7))
        assert not any(L.choose_sharded(T, 8, 7168, REP, SHARD, alpha, 153000.0, 7)
                       for T in range(Tc, min(65536, Tc + 4000), 13))
        if prev is not None:
            assert Tc <= prev
        prev = Tc
