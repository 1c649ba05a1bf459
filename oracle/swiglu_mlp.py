"""Plain float64 definition of the shared-expert SwiGLU MLP and of its TP slicing.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py. It shares no code with the HIP library.

Sources (cited as [key section]):
  [PR50656]  vLLM PR 50656, "[Kimi-K3] Add option to shard the shared expert
             instead of replicating" -- sections "Problem", "Change", "Testing".
  [Digest]   prhub.com.cn digest of the same PR -- section 实现拆解
             (implementation breakdown, steps 2-3) and section 关键源码片段
             (key source excerpt: the sharded-vs-replicated equivalence test).

Storage conventions (read from the equivalence test in [Digest 关键源码片段]):
  x          [M, H]    tokens x hidden, row-major
  w_gate_up  [2I, H]   rows [0, I) are the gate projection, rows [I, 2I) the up
                       projection (the test concatenates gate then up)
  w_down     [H, I]    PyTorch [out, in] layout
  out        [M, H]

Every function below is the plain definition: float64 throughout, library
matmul (numpy -> BLAS dgemm) for the contractions, no blocking or fusion.
"""
from __future__ import annotations

import numpy as np


def _f64(a: np.ndarray, name: str) -> np.ndarray:
    if not isinstance(a, np.ndarray) or a.dtype != np.float64:
        raise TypeError(f"oracle expects float64 numpy arrays; {name} is "
                        f"{type(a).__name__} {getattr(a, 'dtype', '')}")
    return a


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), elementwise, float64.

    The activation of vLLM's SiluAndMul, applied to the gate half
    ([PR50656 Change]: ``act_fn(gate_up)``).  For g < -709 exp overflows to
    +inf and the quotient is -0, which is the correctly rounded limit.
    """
    _f64(g, "g")
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def gate_up_act(x: np.ndarray, w_gate_up: np.ndarray) -> np.ndarray:
    """h = SiLU(x Wg^T) * (x Wu^T): the gate_up projection followed by SiluAndMul.

    [PR50656 Change] ``gate_up, _ = self.gate_up_proj(x); x = self.act_fn(gate_up)``;
    SiluAndMul multiplies SiLU of the first half by the second half, and the
    first half is the gate ([Digest 关键源码片段]: ``cat([gate, up])``).
    Returns h [M, I].
    """
    _f64(x, "x"); _f64(w_gate_up, "w_gate_up")
    two_i, h_dim = w_gate_up.shape
    if two_i % 2 or x.shape[1] != h_dim:
        raise ValueError(f"bad shapes x{x.shape} w_gate_up{w_gate_up.shape}")
    i_dim = two_i // 2
    g = x @ w_gate_up[:i_dim].T
    u = x @ w_gate_up[i_dim:].T
    return silu(g) * u


def down_proj(h: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """out = h Wd^T with Wd stored [H, I] ([PR50656 Change] ``self.down_proj(x)``)."""
    _f64(h, "h"); _f64(w_down, "w_down")
    if h.shape[1] != w_down.shape[1]:
        raise ValueError(f"bad shapes h{h.shape} w_down{w_down.shape}")
    return h @ w_down.T


def swiglu_mlp(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """The replicated MLP forward: out = down(SiLU(x Wg^T) * (x Wu^T)).

    [PR50656 Problem/Change]; the replicated expression of the equivalence
    test in [Digest 关键源码片段].  With a per-rank shard as the weights this is
    the rank's partial over its intermediate slice (RowParallel down with the
    reduction turned off, [Digest 实现拆解] step 3).
    """
    return down_proj(gate_up_act(x, w_gate_up), w_down)


def rank_shard(w_gate_up: np.ndarray, w_down: np.ndarray, tp: int, rank: int):
    """Rank ``rank``'s shard of a full layer under TP size ``tp``.

    With s = I / tp the rank holds [gate[r*s:(r+1)*s]; up[r*s:(r+1)*s]] -- not a
    contiguous row block of the merged weight -- and the column block
    w_down[:, r*s:(r+1)*s] ([Digest 关键源码片段], the per-rank partial list).
    Returns copies (w_gate_up_r [2s, H], w_down_r [H, s]).
    """
    _f64(w_gate_up, "w_gate_up"); _f64(w_down, "w_down")
    i_dim = w_gate_up.shape[0] // 2
    if tp < 1 or i_dim % tp or not 0 <= rank < tp:
        raise ValueError(f"cannot take rank {rank} of tp={tp} from I={i_dim}")
    s = i_dim // tp
    lo, hi = rank * s, (rank + 1) * s
    wgu_r = np.concatenate([w_gate_up[lo:hi], w_gate_up[i_dim + lo:i_dim + hi]], axis=0)
    wd_r = np.ascontiguousarray(w_down[:, lo:hi])
    return wgu_r, wd_r


def rank_partial(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray,
                 tp: int, rank: int) -> np.ndarray:
    """Rank r's partial over its intermediate slice for the full gathered tokens x."""
    wgu_r, wd_r = rank_shard(w_gate_up, w_down, tp, rank)
    return swiglu_mlp(x, wgu_r, wd_r)


def slice_sum(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray, tp: int) -> np.ndarray:
    """Sum over ranks of the per-slice partials: the reduce part of the
    reduce-scatter that ends the sharded block ([PR50656 Change]).  Equals the
    replicated output exactly in real arithmetic."""
    total = None
    for r in range(tp):
        p = rank_partial(x, w_gate_up, w_down, tp, r)
        total = p if total is None else total + p
    return total


def rank_token_rows(full: np.ndarray, tp: int, rank: int) -> np.ndarray:
    """The scatter part: rank r keeps token rows [r*t, (r+1)*t) with t = M / tp."""
    m = full.shape[0]
    if m % tp:
        raise ValueError(f"M={m} not divisible by tp={tp}")
    t = m // tp
    return full[rank * t:(rank + 1) * t]


def feature_concat_design(x_by_rank, w_gate_up: np.ndarray, w_down: np.ndarray):
    """The rejected design of [PR50656 Testing]: shard both projections over their
    output dimension and all-gather the feature slices instead of the tokens.

    ``x_by_rank[q]`` is the [t, H] token block rank q holds.  Rank q computes its
    intermediate slice q only for its own tokens; gathering feature slices
    then builds, for local row j, the intermediate row
    concat_q h_q(token j of rank q) -- features of different tokens when the
    ranks hold different tokens.  Every rank ends with the same [t, H] result,
    which is returned.  (The pages do not print the broken code; this is the
    plainest reading of the description.)
    """
    tp = len(x_by_rank)
    slices = []
    for q in range(tp):
        wgu_q, _ = rank_shard(w_gate_up, w_down, tp, q)
        slices.append(gate_up_act(x_by_rank[q], wgu_q))
    h_cat = np.concatenate(slices, axis=1)
    return down_proj(h_cat, w_down)


def rms_rescale_rows(out: np.ndarray) -> np.ndarray:
    """Per-token rescale to unit RMS: y[m, :] = out[m, :] / sqrt(mean_k out[m, k]^2).

    Glue between the layers of the stacked-layer workload (not part of the
    pages' method).  No epsilon: an all-zero row is an error.
    """
    _f64(out, "out")
    rms = np.sqrt(np.mean(out * out, axis=1, keepdims=True))
    if np.any(rms == 0.0):
        raise ValueError("row with zero RMS")
    return out / rms


def shard_sequence_parallel_mlp(flag_on: bool, use_sequence_parallel: bool,
                                can_shard: bool, tp_size: int,
                                hidden_size: int, intermediate_size: int) -> bool:
    """Whether the MLP is TP-sharded under sequence parallelism.

    [Digest 实现拆解] step 2: shard only when the opt-in flag is on, sequence
    parallelism is on, the call site is eligible, tp_size > 1, and both the
    hidden and the intermediate size divide by tp_size; otherwise the layer
    stays replicated.
    """
    return bool(flag_on and use_sequence_parallel and can_shard and tp_size > 1
                and hidden_size % tp_size == 0 and intermediate_size % tp_size == 0)
