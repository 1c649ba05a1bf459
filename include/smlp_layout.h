/*
 * smlp_layout.h -- per-step choice between the replicated and the TP-sharded shared
 * expert (host-only functions of libsmlp.so; no HIP call).
 *
 * vLLM PR 50656, "[Kimi-K3] Add option to shard the shared expert instead of
 * replicating": a sharded rank reads a 1/tp slice of the weights but adds two
 * collectives to every layer (an all-gather of the tokens before the MLP and a
 * reduce-scatter of the partial outputs after it, section "Change"); that pays off for
 * small token counts only, so one process-wide switch is wrong for either prefill or
 * decode (section "Trade-off and why it is opt-in"); the
 * crossover is an estimate, about 700 tokens at TP8 on the authors' hardware (section
 * "Evaluation").  These functions make the choice per step from measured kernel-time
 * curves and a model of the two collectives:
 *
 *   replicated: t_rep   = K_rep(ceil(T / tp))
 *   sharded:    t_shard = K_shard(T) + t_coll(2) + t_coll(partial_elem_bytes)
 *   t_coll(e)   = alpha_us + ceil((tp - 1) / links) * ceil(T / tp) * hidden * e / (link_gbps * 1e3)
 *
 * for a step of T tokens spread over tp ranks.  K_rep and K_shard are piecewise linear
 * through the given points (M strictly increasing): the first value below the first
 * point, the last segment extended above the last point (never below the last value).
 * The step shards when t_shard < t_rep.  Times in microseconds.
 */
#ifndef SMLP_LAYOUT_H
#define SMLP_LAYOUT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int tp;                    /* ranks sharing the layer, >= 2                              */
  int64_t hidden;            /* H, >= 1                                                    */
  int partial_elem_bytes;    /* element size of the reduce-scattered partial: 2 or 4       */
  double alpha_us;           /* fixed cost of one collective, >= 0                         */
  double link_gbps;          /* bandwidth of one point-to-point link in GB/s, > 0          */
  int links;                 /* links a rank drives at once, >= 1                          */
  int n_rep;                 /* points of the replicated kernel curve, >= 1                */
  const double* rep_m;       /* host arrays of n_rep token counts (strictly increasing)    */
  const double* rep_us;      /*   and kernel times in microseconds (finite, >= 0)          */
  int n_shard;               /* points of the shard (I / tp slice) kernel curve, >= 1      */
  const double* shard_m;
  const double* shard_us;
} smlp_layout_model;

/* Predicted step times of both layouts for T >= 1 tokens.  Returns SMLP_OK,
 * SMLP_ERR_NULL or SMLP_ERR_ARG (invalid model or T). */
int shared_mlp_layout_times(const smlp_layout_model* model, int64_t T, double* t_rep_us,
                            double* t_shard_us);

/* *sharded = 1 when the sharded layout is predicted faster for T tokens, else 0. */
int shared_mlp_choose_layout(const smlp_layout_model* model, int64_t T, int* sharded);

/* Smallest T in [1, T_max] at which the step does not shard (0 if it shards at every
 * T up to T_max).  1 <= T_max <= 2^24. */
int shared_mlp_layout_crossover(const smlp_layout_model* model, int64_t T_max, int64_t* T_cross);

#ifdef __cplusplus
}
#endif
#endif /* SMLP_LAYOUT_H */
