"""Pins of the MLA latent projection oracle against facts outside the oracle.

Source: vLLM PR 345, "[II] TP-shard Kimi MLA latent projections" (sections
"Behavior", "Technical reason", "Compatibility", "Validation").  The pins are a
hand-written worked example of the rank-major to logical order, the
gather-reconstructs-the-exact-output property, the TP1 special case, the printed
per-GPU saving, and the geometry rejections the page lists.
"""
import os

import numpy as np
import pytest

import oracle

from conftest import GOLDEN


def _labels(n):
    """A weight whose row j is j * e_0, so projecting x = e_0 yields the row labels."""
    w = np.zeros((n, 3))
    w[:, 0] = np.arange(n, dtype=np.float64)
    return w


def test_worked_example_rank_major_to_logical():
    # ranges q (4 rows: q0..q3) and kv (2 rows: k0, k1), tp = 2.  Written out by hand:
    # rank 0 holds q0 q1 k0, rank 1 holds q2 q3 k1; the gather is rank 0 then rank 1.
    q = [10.0, 11.0, 12.0, 13.0]
    k = [20.0, 21.0]
    gathered = np.array([[q[0], q[1], k[0], q[2], q[3], k[1]]])
    logical = oracle.restore_logical(gathered, [4, 2], 2)
    assert logical.tolist() == [[10.0, 11.0, 12.0, 13.0, 20.0, 21.0]]
    # the shard function selects the same rows of a labelled weight
    w = _labels(6)
    assert oracle.merged_column_shard(w, [4, 2], 2, 0)[:, 0].tolist() == [0.0, 1.0, 4.0]
    assert oracle.merged_column_shard(w, [4, 2], 2, 1)[:, 0].tolist() == [2.0, 3.0, 5.0]


def test_three_ranges_by_hand():
    # sizes [3, 6, 3], tp = 3: rank r holds a_r, b_{2r}, b_{2r+1}, c_r
    w = _labels(12)
    got = [oracle.merged_column_shard(w, [3, 6, 3], 3, r)[:, 0].tolist() for r in range(3)]
    assert got == [[0, 3, 4, 9], [1, 5, 6, 10], [2, 7, 8, 11]]
    gathered = np.array([sum(got, [])], dtype=np.float64)
    assert oracle.restore_logical(gathered, [3, 6, 3], 3)[0].tolist() == list(range(12))


@pytest.mark.parametrize("sizes,tp", [([1536, 576], 16), ([1536, 576], 8), ([1536, 576], 1),
                                      ([32, 16, 48], 4), ([6], 3)])
def test_labels_come_back_in_logical_order(sizes, tp):
    n = sum(sizes)
    w = _labels(n)
    x = np.zeros((1, 3))
    x[0, 0] = 1.0
    got = oracle.sharded_projection(x, w, sizes, tp)
    assert got[0].tolist() == list(range(n))


@pytest.mark.parametrize("tp", [1, 2, 4, 8, 16])
def test_gather_reconstructs_the_exact_output(tp):
    # integer operands: every product and sum is exact in float64, so the sharded path
    # must equal the replicated projection bit for bit
    rng = np.random.Generator(np.random.PCG64(345 + tp))
    sizes = [96, 64]
    x = rng.integers(-8, 9, size=(5, 40)).astype(np.float64)
    w = rng.integers(-8, 9, size=(sum(sizes), 40)).astype(np.float64)
    np.testing.assert_array_equal(oracle.sharded_projection(x, w, sizes, tp), x @ w.T)


def test_linear_brute_force():
    rng = np.random.Generator(np.random.PCG64(7))
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    y = oracle.linear(x, w)
    for m in range(3):
        for n in range(4):
            s = 0.0
            for k in range(5):
                s += x[m][k] * w[n][k]
            assert abs(y[m, n] - s) < 1e-12


def test_tp1_is_the_identity():
    rng = np.random.Generator(np.random.PCG64(1))
    w = rng.standard_normal((10, 4))
    np.testing.assert_array_equal(oracle.merged_column_shard(w, [7, 3], 1, 0), w)
    g = rng.standard_normal((2, 10))
    np.testing.assert_array_equal(oracle.restore_logical(g, [7, 3], 1), g)


def test_printed_saving_pins_the_shard_size():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "mla_latent_bytes.txt")).read().splitlines()
            if ln.strip() and not ln.startswith("#")]
    layers, n, k, tp, printed, unit = rows[0]
    layers, n, k, tp, printed = int(layers), int(n), int(k), int(tp), float(printed)
    assert unit == "GiB"
    sizes = [1536, 576]
    assert sum(sizes) == n
    # bytes of one rank's shard, from the shard the oracle selects
    w = np.zeros((n, 1))
    shard_rows = oracle.merged_column_shard(w, sizes, tp, 0).shape[0]
    saving = layers * (n - shard_rows) * k * 2 / 2**30
    assert round(saving, 3) == printed


@pytest.mark.parametrize("sizes,tp", [([1536, 576], 7), ([1536, 576], 128), ([1536, 577], 16),
                                      ([0, 576], 16), ([], 2), ([8], 0)])
def test_non_divisible_geometry_is_rejected(sizes, tp):
    w = np.zeros((max(sum(sizes), 1), 2))
    with pytest.raises(ValueError):
        oracle.merged_column_shard(w, sizes, tp, 0)
    with pytest.raises(ValueError):
        oracle.restore_logical(np.zeros((1, max(sum(sizes), 1))), sizes, tp)


@pytest.mark.parametrize("width", [2111, 2048, 2113, 132])
def test_truncated_or_oversized_gather_is_rejected(width):
    with pytest.raises(ValueError):
        oracle.restore_logical(np.zeros((2, width)), [1536, 576], 16)


def test_weight_rows_must_match_ranges():
    with pytest.raises(ValueError):
        oracle.merged_column_shard(np.zeros((2100, 4)), [1536, 576], 16, 0)
    with pytest.raises(ValueError):
        oracle.merged_column_shard(np.zeros((2112, 4)), [1536, 576], 16, 16)
