"""Plain float64 definition of the TP-sharded merged MLA latent projection.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py. It shares no code with the HIP library.

Source (cited as [PR345 section]):
  [PR345]  local-inference-lab/vllm PR 345, "[II] TP-shard Kimi MLA latent
           projections" -- sections "Behavior", "Technical reason",
           "Compatibility", "Validation".

What the page describes: each MLA layer has one merged projection whose output
rows are the q_a range followed by the kv_a range ([PR345 Behavior]: a
2112 x 7168 bf16 weight).  Under tensor parallelism the weight is stored as
column shards of a merged-column linear layer: every logical range is split into
tp equal contiguous pieces and rank r holds piece r of each range, in range order.
A forward pass computes each rank's local output, gathers the rank outputs in rank
order ("rank-major"), and restores the logical layout -- all of range 0, then all of
range 1 -- before the latents are used ([PR345 Behavior], [PR345 Technical reason]).
Every range size must be divisible by tp, and collective geometry that does not
match the ranges is rejected ([PR345 Compatibility], [PR345 Validation]).

Storage: x [M, K] (tokens x hidden), w [N, K] ([out, in]), outputs [M, N].  Every
function takes float64 numpy arrays and computes in float64.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def _f64(a: np.ndarray, name: str) -> np.ndarray:
    if not isinstance(a, np.ndarray) or a.dtype != np.float64:
        raise TypeError(f"oracle expects float64 numpy arrays; {name} is "
                        f"{type(a).__name__} {getattr(a, 'dtype', '')}")
    return a


def check_geometry(sizes: Sequence[int], tp: int) -> None:
    """Reject range sizes that are not positive multiples of tp ([PR345 Compatibility]: the
    sharded layout needs each range to split evenly over the ranks)."""
    if tp < 1:
        raise ValueError(f"tp must be >= 1, got {tp}")
    if not sizes:
        raise ValueError("no output ranges")
    for s in sizes:
        if s <= 0 or s % tp:
            raise ValueError(f"range size {s} is not a positive multiple of tp = {tp}")


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x . w^T: the projection (a plain matmul, no bias, no activation)."""
    _f64(x, "x"), _f64(w, "w")
    return x @ w.T


def merged_column_shard(w: np.ndarray, sizes: Sequence[int], tp: int, r: int) -> np.ndarray:
    """Rank r's rows of the merged weight: piece r of each logical range (each range cut
    into tp equal contiguous pieces), concatenated in range order ([PR345 Behavior])."""
    _f64(w, "w")
    check_geometry(sizes, tp)
    if sum(sizes) != w.shape[0]:
        raise ValueError(f"ranges {list(sizes)} do not cover the {w.shape[0]} weight rows")
    if not 0 <= r < tp:
        raise ValueError(f"rank {r} outside [0, {tp})")
    pieces, off = [], 0
    for s in sizes:
        p = s // tp
        pieces.append(w[off + r * p: off + (r + 1) * p])
        off += s
    return np.concatenate(pieces, axis=0)


def gather_rank_major(parts: Sequence[np.ndarray]) -> np.ndarray:
    """The gather of the rank outputs: rank 0's columns, then rank 1's, ... (the
    merged-column collective's rank-major order, [PR345 Technical reason])."""
    for i, p in enumerate(parts):
        _f64(p, f"parts[{i}]")
    return np.concatenate(list(parts), axis=1)


def restore_logical(gathered: np.ndarray, sizes: Sequence[int], tp: int) -> np.ndarray:
    """Rank-major [M, tp * (sum(sizes)/tp)] -> logical [M, sum(sizes)]: for each range in
    order, the pieces of all ranks in rank order ([PR345 Behavior]: restore the logical
    q_a followed by kv_a layout).  Truncated or oversized gathers are rejected
    ([PR345 Validation])."""
    _f64(gathered, "gathered")
    check_geometry(sizes, tp)
    n = sum(sizes)
    if gathered.ndim != 2 or gathered.shape[1] != n:
        raise ValueError(f"gathered width {gathered.shape[-1]} does not match the ranges (sum {n})")
    per_rank = n // tp
    blocks, off = [], 0
    for s in sizes:
        p = s // tp
        for r in range(tp):
            c0 = r * per_rank + off // tp
            blocks.append(gathered[:, c0: c0 + p])
        off += s
    return np.concatenate(blocks, axis=1)


def sharded_projection(x: np.ndarray, w: np.ndarray, sizes: Sequence[int], tp: int) -> np.ndarray:
    """The whole sharded path on one host: every rank's local projection, the rank-major
    gather, the restore.  Equals linear(x, w) ([PR345 Technical reason]: gathering the
    ranks' pieces gives back the replicated result exactly)."""
    parts = [linear(x, merged_column_shard(w, sizes, tp, r)) for r in range(tp)]
    return restore_logical(gather_rank_major(parts), sizes, tp)
