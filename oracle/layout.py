"""Plain definition of the per-step layout choice: replicated vs TP-sharded shared expert.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py. It shares no code with the HIP library.

Source (cited as [PR50656 section]): vLLM PR 50656, "[Kimi-K3] Add option to shard the
shared expert instead of replicating" -- sections "Change" (an all-gather of the tokens
before the sharded MLP and a reduce-scatter of its partial outputs after it), "Trade-off
and why it is opt-in" (a sharded rank reads a 1/tp slice of the weights but adds an
all-gather and a reduce-scatter to every layer, which pays off for small token counts only,
so a single process-wide switch is wrong for either prefill or decode) and
"Evaluation" (the crossover is estimated, about 700 tokens at TP8, not measured).

The model, for one step of T tokens spread over tp ranks (sequence parallel):
  replicated: every rank runs the full MLP on its own ceil(T / tp) tokens:
      t_rep = K_rep(ceil(T / tp))
  sharded: every rank gathers all T tokens, runs its intermediate slice, and
  reduce-scatters the partial outputs:
      t_shard = K_shard(T) + t_AG + t_RS
  where K_rep and K_shard are measured kernel-time curves (piecewise linear in M), and a
  collective moves one chunk of ceil(T / tp) rows of H elements to or from each of the
  tp - 1 peers, in ceil((tp - 1) / links) rounds over point-to-point links:
      t_coll = alpha + ceil((tp - 1) / links) * ceil(T / tp) * H * elem / link_bw
  with elem = 2 bytes (bf16 tokens) for the all-gather and the partial's element size for
  the reduce-scatter.  The step shards when t_shard < t_rep.

Times are in microseconds, bandwidths in bytes per microsecond (GB/s * 1e3).
"""
from __future__ import annotations

import math
from typing import Sequence


def interp(ms: Sequence[float], ts: Sequence[float], m: float) -> float:
    """Piecewise-linear kernel-time curve through the points (ms[i], ts[i]), ms strictly
    increasing: the first value below the first point, linear extrapolation of the last
    segment above the last point (never below the last value)."""
    n = len(ms)
    if n == 0 or n != len(ts):
        raise ValueError("curve needs matching, non-empty point lists")
    for i in range(1, n):
        if not ms[i] > ms[i - 1]:
            raise ValueError("curve points must have strictly increasing M")
    if n == 1 or m <= ms[0]:
        return float(ts[0])
    for i in range(n - 1):
        if m <= ms[i + 1]:
            f = (m - ms[i]) / (ms[i + 1] - ms[i])
            return float(ts[i] + (ts[i + 1] - ts[i]) * f)
    slope = (ts[n - 1] - ts[n - 2]) / (ms[n - 1] - ms[n - 2])
    return float(max(ts[n - 1], ts[n - 1] + slope * (m - ms[n - 1])))


def collective_us(T: int, tp: int, hidden: int, elem: int, alpha_us: float, link_bytes_per_us: float,
                  links: int) -> float:
    """One all-gather or reduce-scatter of T token rows over tp ranks ([PR50656 Change])."""
    if tp < 2 or links < 1 or T < 1:
        raise ValueError("collective needs tp >= 2, links >= 1, T >= 1")
    chunk = math.ceil(T / tp) * hidden * elem
    rounds = math.ceil((tp - 1) / links)
    return alpha_us + rounds * chunk / link_bytes_per_us


def step_times(T: int, tp: int, hidden: int, rep_curve, shard_curve, alpha_us: float,
               link_bytes_per_us: float, links: int, partial_elem: int = 4):
    """(t_rep, t_shard) of one step ([PR50656 Trade-off and why it is opt-in])."""
    t_rep = interp(rep_curve[0], rep_curve[1], math.ceil(T / tp))
    t_ag = collective_us(T, tp, hidden, 2, alpha_us, link_bytes_per_us, links)
    t_rs = collective_us(T, tp, hidden, partial_elem, alpha_us, link_bytes_per_us, links)
    t_shard = interp(shard_curve[0], shard_curve[1], T) + t_ag + t_rs
    return t_rep, t_shard


def choose_sharded(T: int, tp: int, hidden: int, rep_curve, shard_curve, alpha_us: float,
                   link_bytes_per_us: float, links: int, partial_elem: int = 4) -> bool:
    t_rep, t_shard = step_times(T, tp, hidden, rep_curve, shard_curve, alpha_us, link_bytes_per_us,
                                links, partial_elem)
    return t_shard < t_rep


def crossover(T_max: int, tp: int, hidden: int, rep_curve, shard_curve, alpha_us: float,
              link_bytes_per_us: float, links: int, partial_elem: int = 4) -> int:
    """Smallest T in [1, T_max] at which the step does not shard, or 0 if it shards at
    every T up to T_max ([PR50656 Evaluation]: the crossover token count)."""
    for T in range(1, T_max + 1):
        if not choose_sharded(T, tp, hidden, rep_curve, shard_curve, alpha_us, link_bytes_per_us, links,
                              partial_elem):
            return T
    return 0
