/*
 * smlp_tuning.h -- tuning hook of libsmlp's M-dispatch planner (not needed for use).
 *
 * The weight-streaming (small-M) stages are parameterised by the kernel kind (kind:
 * 2 = operands loaded directly in the MFMA layout; 3 = operands streamed into a
 * wave-private LDS ring, M <= 32 only), the number of 16-feature blocks per
 * workgroup (nb), waves per workgroup (waves), u (kind 2: 64-element K steps per wave
 * per pipeline stage; kind 3: LDS ring stages) and the K split over workgroups
 * (ksplit).  By default the planner picks them from M, N and K.  This hook pins any
 * of them (0 = automatic) for subsequent plans, process-wide, so a benchmark can sweep
 * them.  Results are the same up to fp32 summation order.
 */
#ifndef SMLP_TUNING_H
#define SMLP_TUNING_H
#ifdef __cplusplus
extern "C" {
#endif

/* stage: 0 = gate_up, 1 = down, 2 = the plain projection of smlp_latent.h (kind 3
 * only).  kind in {0,2,3}; nb in {0,...,4}; waves in {0,4,8}; u in {0,...,8};
 * 0 <= ksplit <= 1024.  Returns SMLP_OK or SMLP_ERR_ARG.  A pinned combination that is
 * not a compiled kernel makes later plans fail with SMLP_ERR_ARG.  With nb, waves or u
 * pinned, a K-split stage is reduced by a separate finalize launch instead of in its own
 * launch (a pinned ksplit alone keeps the in-launch reduction): a sweep of pinned
 * streaming shapes with K splits once ended in an unexplained GPU memory fault, and the
 * in-launch form is tested only with the planner's own shapes. */
int shared_mlp_tune_skinny(int stage, int kind, int nb, int waves, int u, int ksplit);

/* The LDS-tiled (large-M) stages (stage 2: the plain projection, planned like down):
 * tile of bm tokens x bn weight rows (0 and 0 =
 * automatic; bm in {64 (with bn 64 on a 2 x 2 wave grid), 128, 256}, bn in
 * {32 (down only), 64, 128, 256}), the wave grid
 * wm x wn over the tile (0 and 0 = automatic; each in {1, 2, 4}), the number of LDS
 * stages ns (0 = automatic, <= 8) and the K split over workgroups (0 = automatic,
 * <= 1024).  Returns SMLP_OK or SMLP_ERR_ARG; a pinned combination that is not compiled
 * makes later plans fail with SMLP_ERR_ARG. */
int shared_mlp_tune_gemm(int stage, int bm, int bn, int wm, int wn, int ns, int ksplit);

/* Planes of the intermediate h on the small-M (weight-streaming) path: 1 = one bf16
 * plane (h rounded once to bf16, as the serving stack stores it; the down stage then
 * runs the projection kernel, M <= 32 only), 2 = two planes hi + lo (h effectively
 * unrounded), 0 = automatic (one plane for M <= 32 and I >= 256, else two).
 * Process-wide, for subsequent plans.  Returns SMLP_OK or SMLP_ERR_ARG. */
int shared_mlp_tune_h_planes(int planes);

/* Format of the intermediate h on the LDS-tiled (large-M) path: 0 = automatic (two bf16
 * planes hi + lo when I < 256, else one fp16 plane for a bf16 output and one bf16 plane
 * for an fp32 partial), 1 = one bf16 plane, 2 = two bf16 planes, 3 = one fp16 plane.  One bf16 plane rounds h to 8 significant bits, which can
 * take a bf16-output layer past the parity bound over a large output; it is here for
 * timing comparisons.  Process-wide, for subsequent plans.  Returns SMLP_OK or
 * SMLP_ERR_ARG. */
int shared_mlp_tune_h_format(int fmt);

/* Gate_up stage of the tiled path (33 <= M <= 256) as the weight-streaming kernel split
 * over 16- or 32-token tiles, full K per workgroup, SiLU-and-mul fused (no K-split
 * partials): 0 = automatic, 1 = wherever it applies (at most 4 MFMA tiles of features per
 * workgroup), 2 = never.  The small-M overrides of stage 0 (nb, waves, u) apply to it.
 * Process-wide, for subsequent plans.  Returns SMLP_OK or SMLP_ERR_ARG. */
int shared_mlp_tune_token_split(int mode);

/* Token count from which a tiled down stage that reads fp16 h converts w_down to an fp16
 * copy in the workspace once (one streaming pass, counted in the workspace size and the
 * kernel count) instead of converting its weight fragments in registers (default 1024;
 * 1 = always, a value above any M = never).  Results are identical either way (the
 * conversion is exact).  Returns the previous value, or -1 (SMLP_ERR_ARG) if min_m < 1.
 * Process-wide, for subsequent plans. */
int64_t shared_mlp_tune_weight_convert(int64_t min_m);

/* One-launch decode layer: where shared_mlp_forward's plan runs the weight-streaming
 * stages with one plane of h at M <= 32 (the configurations the fused kernel is built
 * for), both stages go into one grid: the gate_up workgroups first, then the down
 * workgroups, which take each compute unit as a gate_up workgroup leaves it, issue
 * their first weight loads and wait (bounded) for all of h before loading it.  mode:
 * 0 = automatic, 1 = wherever it applies, 2 = never (two launches).  poll_limit: polls
 * a down workgroup makes before it gives up, writes NaN and flags the error; 0 = the
 * default (2^18, a fraction of a second), negative = give up at once (to exercise the
 * failure path).  Results are identical with and without the fusion.  Process-wide,
 * for subsequent calls.  Returns SMLP_OK or SMLP_ERR_ARG. */
int shared_mlp_tune_layer_fusion(int mode, int poll_limit);

#ifdef __cplusplus
}
#endif
#endif /* SMLP_TUNING_H */
