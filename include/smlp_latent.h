/*
 * smlp_latent.h -- the tensor-parallel merged MLA latent projection in libsmlp.so.
 *
 * The operation (vLLM PR 345, "[II] TP-shard Kimi MLA latent projections", sections
 * "Behavior", "Technical reason", "Compatibility" and "Validation"): each MLA layer
 * has one merged projection whose output columns are the q_a range followed by the
 * kv_a range (2112 x 7168 bf16 for Kimi-K3).  Under tensor parallelism the weight is
 * stored as column shards: every range is cut into tp equal contiguous pieces and
 * rank r holds piece r of each range, in range order.  A forward pass computes the
 * rank's local output y_r = x . W_r^T, gathers the rank outputs (rank by rank, the
 * order of a merged-column collective) and restores the logical layout -- all of
 * range 0, then all of range 1, ... -- before the latents are used.  Every range size
 * must divide by tp, and a gathered width that does not match the ranges is rejected.
 *
 * The gather itself is a collective and is not part of this library.  A caller that
 * gathers in place can let shared_mlp_linear write each rank's output straight into
 * its slot of the gathered buffer (ldy = the gathered row length, y = the slot).
 *
 * Conventions are those of smlp.h: device pointers, caller-owned buffers, work
 * enqueued on `stream` without synchronisation, SMLP_* status codes with a detail
 * string from shared_mlp_last_error(), every validation done on the host before any
 * HIP call, and no fallback to another computation.
 */
#ifndef SMLP_LATENT_H
#define SMLP_LATENT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "smlp.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest number of logical ranges shared_mlp_restore_logical accepts. */
#define SMLP_MAX_RANGES 8

/* Plan of shared_mlp_linear for these sizes (host-only; no HIP call).  Fills path
 * (SMLP_PATH_SMALL_M: weight-streaming kernel, M < min(threshold, 33);
 * SMLP_PATH_LARGE_M: LDS-tiled MFMA kernel; SMLP_PATH_NONE: M == 0),
 * workspace_bytes, down_ksplit / down_blocks (the projection's K split and
 * workgroups) and kernels; the gate_up fields are zero and h_dtype is SMLP_BF16. */
int shared_mlp_linear_plan(int64_t M, int64_t K, int64_t N, smlp_plan* plan);

/* Bytes of workspace shared_mlp_linear needs for these sizes (host-only; 0 when the
 * plan has no K split over workgroups). */
int shared_mlp_linear_workspace_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes);

/*
 * y[m, n] = sum_k x[m, k] w[n, k]: the rank-local (or, at tp = 1, the replicated)
 * merged latent projection; no bias, no activation.  bf16 operands, fp32
 * accumulation, y rounded once to bf16 (nearest even) or written as fp32.
 *   x          [M, K]  bf16, row-major, 16-byte aligned
 *   w          [N, K]  bf16, row-major ([out, in]), 16-byte aligned
 *   y          M rows of N elements, row m at y + m * ldy; bf16 (out_fp32 == 0,
 *              8-byte aligned) or fp32 (out_fp32 == 1, 16-byte aligned)
 *   sizes      K % 8 == 0, K >= 8; N % 4 == 0, N >= 4; ldy >= N, ldy % 4 == 0;
 *              M*K, N*K and M*ldy < 2^31; M == 0 is a no-op
 *   workspace  >= shared_mlp_linear_workspace_bytes(...) bytes, 256-byte aligned (may
 *              be NULL when that is 0); contents on entry ignored, on exit unspecified
 * y must not overlap x, w or the workspace; elements of y between row ends and the
 * next row (columns N .. ldy-1) are not written.  One or two kernels are enqueued.
 */
int shared_mlp_linear(const void* x, const void* w, void* y, int64_t M, int64_t K, int64_t N,
                      int64_t ldy, int out_fp32, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Restore the logical column order of a gathered merged-column output
 * (PR 345, "Behavior" and "Technical reason"):
 *   gathered  [M, n_gathered], rank-major: row m is rank 0's tp-local output, then rank
 *             1's, ...; rank r's local output is piece r of range 0, piece r of range
 *             1, ... (piece length sizes[t] / tp)
 *   out       [M, n_gathered], logical: range 0, then range 1, ...; out column
 *             o_t + r * sizes[t]/tp + c  =  gathered column r * n_gathered/tp + o_t/tp + c
 *             (o_t = sizes[0] + ... + sizes[t-1], 0 <= c < sizes[t]/tp)
 *   sizes     host array of nsizes range widths, 1 <= nsizes <= SMLP_MAX_RANGES
 *   elem_bytes 2 (bf16) or 4 (fp32); both pointers aligned to elem_bytes
 * Errors (PR 345, "Compatibility" and "Validation"): tp < 1 or a range size that is
 * not a positive multiple of tp -> SMLP_ERR_SHAPE; n_gathered different from the sum
 * of sizes (a truncated or oversized gather) -> SMLP_ERR_SHAPE; nsizes out of range
 * or elem_bytes not 2 or 4 -> SMLP_ERR_ARG; out overlapping gathered -> SMLP_ERR_ALIAS.
 * M * n_gathered < 2^31.  A bit-exact copy; one kernel is enqueued (none for M == 0).
 */
int shared_mlp_restore_logical(const void* gathered, void* out, int64_t M, int64_t n_gathered,
                               const int64_t* sizes, int nsizes, int tp, int elem_bytes,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SMLP_LATENT_H */
