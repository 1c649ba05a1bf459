/*
 * smlp.h -- C ABI of the MI355X (gfx950) shared-expert SwiGLU MLP library (libsmlp.so).
 *
 * The operation (vLLM PR 50656, "[Kimi-K3] Add option to shard the shared expert
 * instead of replicating", sections "Problem" and "Change"; the equivalence test in
 * the prhub.com.cn digest of that PR, section 关键源码片段):
 *
 *     G   = x . Wg^T            Wg = w_gate_up rows [0, I)       (gate_up_proj)
 *     U   = x . Wu^T            Wu = w_gate_up rows [I, 2I)
 *     h   = SiLU(G) * U         SiLU(g) = g / (1 + e^-g)          (SiluAndMul)
 *     out = h . Wd^T            Wd = w_down, stored [H, I]        (down_proj)
 *
 * Replicated layout: the caller passes the full weights (I = 6144 for Kimi-K3) and
 * gets the layer output.  TP-sharded layout: the caller passes one rank's shard
 * ([gate_r; up_r] and the matching column block of Wd, I = I_full / tp) and asks for
 * an fp32 output, which is that rank's partial over its intermediate slice -- the
 * tensor the sharded block hands to its reduce-scatter (down_proj with the
 * reduction turned off, digest section 实现拆解 step 3).
 *
 * Conventions for every entry point
 *  - Layouts are row-major [out, in]: x [M, H], w_gate_up [2I, H], w_down [H, I],
 *    out [M, H].  Element type is given by `dtype` (SMLP_BF16 or SMLP_FP32).
 *  - Device pointers only (memory from hipMalloc or any allocator of the same
 *    device).  The caller owns every buffer; the library keeps no pointer after a
 *    call returns and allocates no device memory.
 *  - Work is enqueued on `stream` (0 = the legacy default stream) and the call
 *    returns without synchronising.  The library never synchronises a stream.
 *  - Return value: SMLP_OK (0) or an error status.  On any error nothing was
 *    launched; shared_mlp_last_error() gives a detail string (thread-local).
 *    Argument validation happens on the host before any HIP call, so every
 *    validation error is reported without touching a GPU.
 *  - There is no silent fallback: an unsupported shape or layout is an error, never
 *    a different computation.
 *  - M == 0 is a valid no-op (nothing is launched).  H and I must be >= 1.
 *  - Size limits: M*H, M*I and 2*I*H must each be < 2^31 elements.
 *  - SMLP_BF16: H % 8 == 0, I % 8 == 0 and every pointer 16-byte aligned.
 *    Accumulation is fp32; the bf16 output is rounded once, to nearest even.
 *  - SMLP_FP32: any sizes; pointers 4-byte aligned; out is fp32.
 *  - Output buffers must not overlap any input buffer or the workspace.
 *  - Calls that share a workspace must not run concurrently.
 */
#ifndef SMLP_H
#define SMLP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  SMLP_BF16_HILO and SMLP_FP16 only describe the intermediate h in a
 * workspace: two bf16 planes [M, I] (hi first, then lo) whose sum is the fp32 value, or
 * one fp16 plane [M, I] (rounded once to nearest even; |h| must stay below 65504). */
enum { SMLP_BF16 = 0, SMLP_FP32 = 1, SMLP_BF16_HILO = 2, SMLP_FP16 = 3 };

/* Status codes. */
enum {
  SMLP_OK = 0,
  SMLP_ERR_NULL = 1,      /* a required pointer is NULL                                  */
  SMLP_ERR_SHAPE = 2,     /* a size is out of range or breaks a divisibility rule        */
  SMLP_ERR_ALIGN = 3,     /* a pointer is not aligned as the dtype requires              */
  SMLP_ERR_ALIAS = 4,     /* an output overlaps an input or the workspace                */
  SMLP_ERR_WORKSPACE = 5, /* workspace_bytes is smaller than shared_mlp_workspace_bytes  */
  SMLP_ERR_DTYPE = 6,     /* unknown dtype, or a flag the dtype does not support         */
  SMLP_ERR_HIP = 7,       /* a HIP runtime call or kernel launch failed                  */
  SMLP_ERR_ARG = 8        /* another argument is out of range (tp, rank, threshold)     */
};

/* Kernel path chosen by the M-dispatch. */
enum {
  SMLP_PATH_NONE = 0,     /* M == 0                                                       */
  SMLP_PATH_FP32 = 1,     /* fp32 inputs: plain fp32 kernels, any shape                   */
  SMLP_PATH_SMALL_M = 2,  /* bf16, M < large-M threshold: weight-streaming kernels        */
  SMLP_PATH_LARGE_M = 3   /* bf16, M >= threshold: LDS-tiled bf16 MFMA GEMM kernels       */
};

/* Static name of a status code. */
const char* shared_mlp_status_string(int status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* shared_mlp_last_error(void);

/* Dispatch plan of one forward call.  Filled by shared_mlp_plan (host-only). */
typedef struct {
  int path;               /* SMLP_PATH_*                                                  */
  int h_dtype;            /* storage type of the intermediate h in the workspace          */
  size_t h_offset;        /* byte offset of h [M, I] (row-major) inside the workspace     */
  size_t workspace_bytes; /* bytes of workspace the call needs                            */
  int gate_up_ksplit;     /* K-split factor of the gate_up stage (1 = none)              */
  int down_ksplit;        /* K-split factor of the down stage                             */
  int gate_up_blocks;     /* workgroups of the gate_up stage's main kernel                */
  int down_blocks;        /* workgroups of the down stage's main kernel                   */
  int kernels;            /* kernel launches per forward call (1 for the one-launch      */
                          /* decode layer, 2 there on a stream past the 16th per device;  */
                          /* 1 for a small fp32 layer, M*I <= 4096 and M*H*I <= 2^20)      */
} smlp_plan;

/* Plan of shared_mlp_forward for these sizes.  Host-only; no HIP call. */
int shared_mlp_plan(int64_t M, int64_t H, int64_t I, int dtype, int partial_fp32,
                    smlp_plan* plan);

/* Bytes of workspace shared_mlp_forward needs for these sizes (host-only). */
int shared_mlp_workspace_bytes(int64_t M, int64_t H, int64_t I, int dtype, size_t* bytes);

/*
 * Forward pass of the SwiGLU MLP (formula above).
 *   x            [M, H]   dtype
 *   w_gate_up    [2I, H]  dtype, rows [0, I) gate, rows [I, 2I) up
 *   w_down       [H, I]   dtype
 *   out          [M, H]   fp32 if dtype == SMLP_FP32 or partial_fp32 != 0, else bf16
 *   partial_fp32 nonzero: write fp32 (a TP rank's partial sum); zero: bf16 output
 *   workspace    device scratch of >= shared_mlp_workspace_bytes(...) bytes, 256-byte
 *                aligned; contents on entry are ignored, on exit unspecified
 * One to five kernels are enqueued on `stream` (see smlp_plan.kernels).  At M <= 32
 * with bf16 weights the two stages run as one launch whose down workgroups wait
 * (bounded) for the gate_up workgroups of the same launch; it keeps a few counters per
 * stream in a static device array (16 streams per GPU; further streams get the
 * two-launch form).  Calls on one stream, and on different streams, may run as usual;
 * two replays of one captured graph must not run at the same time (they share the
 * capturing stream's counters).  If a down workgroup ever gives up waiting, its output
 * rows are NaN.  A small fp32 layer (M * I <= 4096, M * H * I <= 2^20) runs both stages
 * in one single-workgroup launch with h in LDS; the workspace is still required.
 */
int shared_mlp_forward(const void* x, const void* w_gate_up, const void* w_down, void* out,
                       int64_t M, int64_t H, int64_t I, int dtype, int partial_fp32,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * shared_mlp_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The intermediate h and any K-split
 * partial sums live in a static device array of SMLP_NOALLOC_SCRATCH_BYTES bytes
 * (32 MiB), one per GPU, held from library load until the process ends.  A call whose
 * plan needs more (shared_mlp_plan's workspace_bytes; e.g. the M = 8192 prefill) returns
 * SMLP_ERR_WORKSPACE before any HIP call.  Every call on one GPU uses that GPU's array:
 * calls that overlap on one GPU (concurrent streams or threads) race and must be
 * serialised by the caller.  The array keeps the last call's contents; nothing in it
 * needs to start at zero.  Arguments and results are those of shared_mlp_forward.
 */
#define SMLP_NOALLOC_SCRATCH_BYTES (32u << 20)
int shared_mlp_forward_noalloc(const void* x, const void* w_gate_up, const void* w_down, void* out,
                               int64_t M, int64_t H, int64_t I, int dtype, int partial_fp32,
                               hipStream_t stream);

/*
 * The two halves of shared_mlp_forward, for callers that time or test them apart.
 * shared_mlp_gate_up_act computes h = SiLU(x Wg^T) * (x Wu^T) into the workspace
 * (at smlp_plan.h_offset, as smlp_plan.h_dtype); shared_mlp_down then computes out
 * from that h.  Both calls must get the same M, H, I, dtype, partial_fp32 and
 * workspace; together they equal one shared_mlp_forward.
 */
int shared_mlp_gate_up_act(const void* x, const void* w_gate_up, int64_t M, int64_t H,
                           int64_t I, int dtype, int partial_fp32, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);
int shared_mlp_down(const void* w_down, void* out, int64_t M, int64_t H, int64_t I, int dtype,
                    int partial_fp32, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * M-dispatch threshold: bf16 calls with M >= threshold take the LDS-tiled MFMA path,
 * smaller M the weight-streaming path (which serves at most 128 tokens, so M > 128
 * always takes the tiled path).  The initial value is 33, or the value of the
 * environment variable SMLP_LARGE_M_MIN (an integer in [1, 129]) read at library
 * load.  Returns the previous threshold, or -1 (SMLP_ERR_ARG detail) if threshold is
 * outside [1, 129].  Process-wide; not synchronised with calls in flight on other
 * threads.
 */
int64_t shared_mlp_set_large_m_threshold(int64_t threshold);

/*
 * Shard-gating predicate (prhub digest of PR 50656, section 实现拆解 step 2): returns
 * 1 when the MLP should be TP-sharded -- the opt-in flag is on, sequence
 * parallelism is on, the call site is eligible, tp > 1, and H and I both divide
 * by tp -- and 0 when it stays replicated.  Pure host function; it is the only
 * place where "replicate instead" is an answer, and it is an explicit query.
 */
int shared_mlp_shard_eligible(int flag_on, int use_sequence_parallel, int caller_eligible,
                              int tp, int64_t H, int64_t I);

/*
 * Copy rank `rank`'s shard out of full weights (digest section 关键源码片段): with
 * s = I / tp, w_gate_up_r [2s, H] = [gate rows r*s..(r+1)*s ; up rows I+r*s..I+(r+1)*s]
 * and w_down_r [H, s] = columns r*s..(r+1)*s of w_down [H, I].  Requires I % tp == 0
 * and 0 <= rank < tp (else SMLP_ERR_ARG); bit-exact copy; destination buffers must
 * not overlap the sources.  Same pointer and alignment rules as the forward call.
 */
int shared_mlp_slice_rank(const void* w_gate_up, const void* w_down, void* w_gate_up_r,
                          void* w_down_r, int64_t H, int64_t I, int tp, int rank, int dtype,
                          hipStream_t stream);

/*
 * Rank `rank`'s fp32 partial of the TP-sharded layer, computed straight from the full
 * weights without copying a shard (the slice of shared_mlp_slice_rank, read in place):
 * with s = I / tp, gate rows [r*s, (r+1)*s) and up rows I + [r*s, (r+1)*s) of w_gate_up
 * [2I, H], and columns [r*s, (r+1)*s) of w_down [H, I] (row stride I).  Lets a caller
 * that keeps the replicated weights resident run the sharded layout on any step.
 *   x [M, H], out [M, H] fp32 (always the partial); workspace as for
 *   shared_mlp_workspace_bytes(M, H, I / tp, dtype).  Requires I % tp == 0 and
 *   0 <= rank < tp (else SMLP_ERR_ARG), and for bf16 s % 8 == 0 (SMLP_ERR_SHAPE).
 * Equal, up to fp32 summation order, to shared_mlp_forward(partial_fp32 = 1) on the
 * copied shard.
 */
int shared_mlp_forward_rank(const void* x, const void* w_gate_up, const void* w_down, void* out,
                            int64_t M, int64_t H, int64_t I, int tp, int rank, int dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Per-token rescale to unit RMS, the glue between the layers of a stacked-layer
 * chain: out[m, :] = bf16_rne(in[m, :] / sqrt(mean_k in[m, k]^2)), computed in fp32.
 *   in   [M, H] fp32 (e.g. a partial output), out [M, H] bf16; no epsilon: a row
 *   whose RMS is zero yields NaN.  Pointers 16-byte aligned, H % 4 == 0, out must
 *   not overlap in.
 */
int shared_mlp_rms_rescale(const float* in, void* out, int64_t M, int64_t H,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SMLP_H */
