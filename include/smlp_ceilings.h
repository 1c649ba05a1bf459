/*
 * smlp_ceilings.h -- measurement kernels of libsmlp (not part of the MLP path).
 *
 * Microbenchmarks of the ceilings that the MLP kernels are held against, measured on
 * the GPU the library runs on rather than taken from a data sheet:
 *   - the cost of one dependent kernel launch (an empty kernel, launched back to back);
 *   - the rate of a plain streaming read of distinct buffers (HBM), and of a read that
 *     every workgroup makes of one shared, L2-resident region;
 *   - the bf16 matrix-core rate of an MFMA-only loop, and the shader clock it runs at;
 *   - the LDS read rate of a compute unit (bytes per shader clock);
 *   - the cost of one grid-wide barrier between two streaming phases of one kernel
 *     (the alternative to a second launch when fusing two dependent stages).
 * Conventions are those of smlp.h: device pointers, work enqueued on `stream`, host
 * validation before any HIP call, SMLP_OK or an error status.  The caller times the
 * launches (for example with HIP events around a captured graph of many launches).
 */
#ifndef SMLP_CEILINGS_H
#define SMLP_CEILINGS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* An empty kernel of `blocks` workgroups of 64 threads (1 <= blocks <= 65535). */
int shared_mlp_ceiling_empty(int blocks, hipStream_t stream);

/*
 * Streaming read: workgroup b (of `blocks`, 512 threads each, one per compute unit's
 * worth of LDS) reads bytes_per_block bytes into LDS with 16-byte direct-to-LDS loads,
 * eight 1 KB loads in flight per wave.  shared == 0: block b reads
 * [src + b * bytes_per_block, +bytes_per_block) (blocks * bytes_per_block <= src_bytes);
 * shared != 0: every block reads [src, src + bytes_per_block) (a region that L2 holds
 * after the first touch).  bytes_per_block is a multiple of 1024 in [1024, 2^30];
 * src 16-byte aligned.  sink [blocks] fp32 receives one value per block so the loads
 * cannot be elided.
 */
int shared_mlp_ceiling_read(const void* src, size_t src_bytes, int blocks, size_t bytes_per_block,
                            int shared, float* sink, hipStream_t stream);

/*
 * MFMA-only loop: `blocks` workgroups of 8 waves, each wave issuing `iters` rounds of
 * four independent 32x32x16 bf16 MFMAs on register operands (4 * 32768 flops per round).
 * cycles [blocks]: shader-clock cycles of wave 0's loop; ticks [blocks]: the same span
 * on the constant 100 MHz counter (their ratio is the clock).  sink [blocks] keeps the
 * accumulators live.  1 <= blocks <= 65535, 1 <= iters <= 2^24.
 */
int shared_mlp_ceiling_mfma(int blocks, int iters, float* sink, uint64_t* cycles, uint64_t* ticks,
                            hipStream_t stream);

/*
 * LDS-read-only loop: `blocks` workgroups of 8 waves and 64 KB of LDS each; every wave
 * issues `iters` rounds of eight independent 16-byte-per-lane LDS reads (8 KB per wave per
 * round) at bank-conflict-free addresses.  cycles [blocks]: shader-clock cycles of wave
 * 0's loop (bytes per clock per compute unit = 8 waves * 8 KB * iters / cycles with one
 * workgroup per compute unit).  sink [blocks * 512] fp32 is written only where needed to
 * keep the reads live (its contents carry no meaning).  1 <= blocks <= 65535,
 * 1 <= iters <= 2^24.
 */
int shared_mlp_ceiling_lds(int blocks, int iters, float* sink, uint64_t* cycles, hipStream_t stream);

/*
 * Two streaming phases of bytes_per_block each per workgroup (distinct regions of src,
 * 2 * blocks * bytes_per_block <= src_bytes), separated by nothing (barrier == 0), by a
 * grid-wide barrier on one counter (barrier == 1), or by a two-level barrier whose
 * workgroups arrive on 16 group counters and the groups on one more (barrier == 2).  The
 * counters, a generation word and an error word live in bar_state (SMLP_CEILING_BAR_WORDS
 * uint32, 16-byte aligned, zero before the first call and left reusable by every call),
 * updated with device-scope atomics; a workgroup waits a bounded time for the others and
 * then sets bar_state[128] = 1 and goes on, so a launch whose workgroups are not all
 * resident at once ends with that flag set instead of hanging.  blocks <= 256 (one
 * workgroup per compute unit of MI355X).
 */
#define SMLP_CEILING_BAR_WORDS 1280
int shared_mlp_ceiling_two_phase(const void* src, size_t src_bytes, int blocks, size_t bytes_per_block,
                                 int barrier, uint32_t* bar_state, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SMLP_CEILINGS_H */
