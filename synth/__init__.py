"""Seeded synthetic inputs for the shared-expert SwiGLU MLP.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds no arithmetic of the method itself: it only draws random
numbers, scales them to the stated standard deviation and rounds them to the
storage dtype. Every tensor comes back on the CPU; callers move it where they
need it.

Recipes
-------
* Tiny fp32 case (the equivalence test of vLLM PR "[Kimi-K3] Add option to shard
  the shared expert instead of replicating", as transcribed in the prhub digest's
  key-code section): ``torch.manual_seed(0)`` and CPU ``torch.randn`` in the draw
  order x, gate, up, down, all N(0, 1), fp32.  tp = 4, hidden 16,
  intermediate 12, 3 tokens per emulated rank.
* Kimi-K3 shapes (hidden 7168, shared intermediate 6144, PR page section
  "Problem"): x ~ N(0, 1); each weight ~ N(0, 1/fan_in), where the second
  parameter is the variance, fan_in = hidden for the gate and up rows and
  fan_in = the logical full intermediate (6144) for the down weight, also when
  only a per-rank slice of it is materialised, so that slices are slices of
  one full layer.  Values are drawn as float32 from numpy's PCG64 generator,
  multiplied by the standard deviation in float32 and rounded to bfloat16
  with round-to-nearest-even (torch's conversion).
* Seeds: ``1000 * config + 10 * copy + tensor_id`` with tensor_id x=0, gate=1,
  up=2, down=3; the per-layer stack uses copy = layer index.
* Merged MLA latent projection (vLLM PR 345, "[II] TP-shard Kimi MLA latent
  projections", section "Behavior": 24 layers of 2112 x 7168 bf16): the q_a range
  followed by the kv_a range, taken as 1536 + 576 rows (the page gives only the
  total); x ~ N(0, 1), w ~ N(0, 1/7168); config 6, tensor_id 4 for the weight, so
  ``seed_of(6, layer, 4)``.
"""
from __future__ import annotations

import numpy as np
import torch

HIDDEN = 7168          # Kimi-K3 hidden size
INTERMEDIATE = 6144    # Kimi-K3 shared-expert intermediate size

TID_X, TID_GATE, TID_UP, TID_DOWN, TID_LATENT = 0, 1, 2, 3, 4

LATENT_SIZES = (1536, 576)   # q_a rows, kv_a rows of the merged latent projection
LATENT_LAYERS = 24           # MLA layers of Kimi-K3
LATENT_CONFIG = 6


def seed_of(config: int, copy: int, tensor_id: int) -> int:
    return 1000 * config + 10 * copy + tensor_id


def normal(shape, std: float, seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std^2) drawn in float32 (PCG64), scaled in float32, cast to ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    t = torch.from_numpy(a)
    return t if dtype == torch.float32 else t.to(dtype)


def tiny_fp32_case():
    """The pages' tiny equivalence case: returns (x, gate, up, down, tp, tokens_per_rank).

    x [12, 16], gate [12, 16], up [12, 16], down [16, 12], fp32, all N(0, 1),
    drawn from ``torch.manual_seed(0)`` in that order.
    """
    tp, hidden, intermediate, tokens_per_rank = 4, 16, 12, 3
    gen = torch.Generator().manual_seed(0)
    m = tp * tokens_per_rank
    x = torch.randn(m, hidden, generator=gen)
    gate = torch.randn(intermediate, hidden, generator=gen)
    up = torch.randn(intermediate, hidden, generator=gen)
    down = torch.randn(hidden, intermediate, generator=gen)
    return x, gate, up, down, tp, tokens_per_rank


def merged_gate_up(gate: torch.Tensor, up: torch.Tensor) -> torch.Tensor:
    """Storage layout of the merged projection: rows [0, I) gate, rows [I, 2I) up."""
    return torch.cat([gate, up], dim=0).contiguous()


def activations(m: int, hidden: int, config: int, copy: int = 0,
                dtype=torch.bfloat16) -> torch.Tensor:
    """x [m, hidden] ~ N(0, 1)."""
    return normal((m, hidden), 1.0, seed_of(config, copy, TID_X), dtype)


def layer_weights(hidden: int, intermediate: int, config: int, copy: int = 0,
                  dtype=torch.bfloat16, fan_in_down: int | None = None):
    """One layer's weights in storage layout.

    Returns (w_gate_up [2I, H], w_down [H, I]).  ``fan_in_down`` defaults to
    ``intermediate``; pass the logical full intermediate size when ``intermediate``
    is a per-rank slice size.
    """
    fid = intermediate if fan_in_down is None else fan_in_down
    sg = float(hidden) ** -0.5
    sd = float(fid) ** -0.5
    gate = normal((intermediate, hidden), sg, seed_of(config, copy, TID_GATE), dtype)
    up = normal((intermediate, hidden), sg, seed_of(config, copy, TID_UP), dtype)
    down = normal((hidden, intermediate), sd, seed_of(config, copy, TID_DOWN), dtype)
    return merged_gate_up(gate, up), down


def latent_weight(rows: int, hidden: int, copy: int = 0, config: int = LATENT_CONFIG,
                  dtype=torch.bfloat16) -> torch.Tensor:
    """One layer's merged latent projection weight [rows, hidden] ~ N(0, 1/hidden)."""
    return normal((rows, hidden), float(hidden) ** -0.5, seed_of(config, copy, TID_LATENT), dtype)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of fp32/bf16 storage to a float64 numpy array."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
