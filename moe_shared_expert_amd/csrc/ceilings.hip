// Measurement kernels (smlp_ceilings.h): launch cost, streaming-read rates, the bf16
// matrix-core rate and clock, the LDS read rate, and the cost of a grid-wide barrier.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "smlp.h"
#include "smlp_ceilings.h"

namespace smlp {
int set_error(int status, const char* msg);
}

namespace {

using namespace smlp;

constexpr int kWaves = 8;     // waves per streaming workgroup
constexpr int kDepth = 8;     // 1 KB loads in flight per wave
constexpr int kPad = 32768;   // extra LDS so that one workgroup holds a compute unit's share

__global__ void empty_kernel(float* never) {
  if (never && threadIdx.x > 1024) never[0] = 0.f;
}

// Stream `bytes` bytes of `base` into a wave-private LDS ring, kDepth loads in flight.
__device__ __forceinline__ void stream_region(const char* base, uint32_t bytes, char* ring) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, bytes);
  const int n = (int)(bytes / 1024);
  int c = 0;
  for (int k = wave; k < n; k += kWaves, ++c) {
    buf_ld_lds_nt(r, ring + (c % kDepth) * 1024, (uint32_t)k * 1024u + (uint32_t)lane * 16u);
    wait_vmcnt<kDepth - 1>();
  }
  wait_vmcnt<0>();
}

__global__ __launch_bounds__(kWaves * 64) void read_kernel(const char* src, uint32_t per_block, int shared,
                                                           float* sink) {
  __shared__ __attribute__((aligned(1024))) char lds[kWaves * kDepth * 1024 + kPad];
  const char* base = src + (shared ? (size_t)0 : (size_t)blockIdx.x * per_block);
  char* ring = lds + (threadIdx.x >> 6) * kDepth * 1024;
  stream_region(base, per_block, ring);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)(unsigned char)lds[blockIdx.x & 1023];
}

__global__ __launch_bounds__(512) void mfma_kernel(int iters, float* sink, uint64_t* cycles, uint64_t* ticks) {
  const int lane = threadIdx.x & 63;
  u32x4 a, b;
  for (int i = 0; i < 4; ++i) {
    // small finite bf16 values (about 2^-10 .. 2^-9), different per lane
    const uint32_t v = 0x3a80u + (uint32_t)((lane + i) & 15);
    a[i] = v | (v << 16);
    b[i] = (v + 1u) | ((v + 2u) << 16);
  }
  f32x16 acc[4];
  for (int t = 0; t < 4; ++t)
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  __syncthreads();
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = mfma32x32x16(a, b, acc[t]);
  }
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  float s = 0.f;
  for (int t = 0; t < 4; ++t)
    for (int e = 0; e < 16; ++e) s += acc[t][e];
  if (threadIdx.x == 0) {
    sink[blockIdx.x] = s;
    cycles[blockIdx.x] = c1 - c0;
    ticks[blockIdx.x] = w1 - w0;
  }
}

// LDS read loop: each wave reads 8 KB of a 64 KB LDS array per round with eight
// independent 16-byte-per-lane reads (consecutive lanes, consecutive 16-byte slots: no
// bank conflicts), the block of each read rotating with the round.
__global__ __launch_bounds__(512) void lds_kernel(int iters, float* sink, uint64_t* cycles) {
  __shared__ __attribute__((aligned(1024))) u32x4 lds[4096];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4096; i += 512) {
    const uint32_t v = (uint32_t)i * 2654435761u;
    lds[i] = u32x4{v, v ^ 1u, v ^ 2u, v ^ 3u};
  }
  __syncthreads();
  u32x4 x = {0u, 0u, 0u, 0u};
  const uint64_t c0 = clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = (wave * 8 + j + i) & 63;
      const u32x4 v = lds[blk * 64 + lane];
      x[0] ^= v[0];
      x[1] += v[1];
      x[2] ^= v[2];
      x[3] += v[3];
    }
  }
  const uint64_t c1 = clock64();
  if (threadIdx.x == 0) cycles[blockIdx.x] = c1 - c0;
  const uint32_t s = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (s == 0x9e3779b9u) sink[blockIdx.x * 512 + threadIdx.x] = 1.f;  // keeps the reads live
  else if (threadIdx.x == 0) sink[blockIdx.x * 512] = (float)(s & 1023u);
}

// Grid barriers over all workgroups, on the words of bar_state (uint32, 64 apart so each
// counter has its own 256-byte block): [0] flat count, [64] generation, [128] error flag,
// [192] group count, [256 + 64 g] arrivals of group g.  Every wait is bounded: after
// `limit` polls a workgroup sets the error flag and goes on.
constexpr int kGroups = 16;  // hierarchical barrier: workgroup b arrives in group b % kGroups

__device__ bool wait_generation(uint32_t* gen_p, uint32_t gen, int limit) {
  for (int n = 0; __hip_atomic_load(gen_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen;) {
    __builtin_amdgcn_s_sleep(1);
    if (++n >= limit) return false;
  }
  return true;
}

// Flat: every workgroup adds to one counter; the last arrival resets it and advances the
// generation, the others wait for the generation to change.
__device__ void grid_barrier_flat(uint32_t* st, int limit) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t gen = __hip_atomic_load(&st[64], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    const uint32_t prev = __hip_atomic_fetch_add(&st[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
    if (prev == gridDim.x - 1) {
      __hip_atomic_store(&st[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      __hip_atomic_fetch_add(&st[64], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      ok = wait_generation(&st[64], gen, limit);
    }
    if (!ok) __hip_atomic_store(&st[128], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// Hierarchical: workgroups arrive on kGroups counters in parallel; the last arrival of a
// group arrives on the group counter, whose last arrival advances the generation.  The
// atomics on one word are serialised where the memory side performs them, so 16 words
// of 16 arrivals each take about half the time of one word of 256.
__device__ void grid_barrier_groups(uint32_t* st, int limit) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int g = blockIdx.x % kGroups;
    const uint32_t members = gridDim.x / kGroups + (g < (int)(gridDim.x % kGroups) ? 1u : 0u);
    const uint32_t groups = gridDim.x < (unsigned)kGroups ? gridDim.x : (uint32_t)kGroups;
    const uint32_t gen = __hip_atomic_load(&st[64], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    const uint32_t prev = __hip_atomic_fetch_add(&st[256 + 64 * g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
    if (prev == members - 1) {
      __hip_atomic_store(&st[256 + 64 * g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      const uint32_t top = __hip_atomic_fetch_add(&st[192], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (top == groups - 1) {
        __hip_atomic_store(&st[192], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        __hip_atomic_fetch_add(&st[64], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        ok = wait_generation(&st[64], gen, limit);
      }
    } else {
      ok = wait_generation(&st[64], gen, limit);
    }
    if (!ok) __hip_atomic_store(&st[128], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

__global__ __launch_bounds__(kWaves * 64) void two_phase_kernel(const char* src, uint32_t per_block, int barrier,
                                                                uint32_t* st, float* sink) {
  __shared__ __attribute__((aligned(1024))) char lds[kWaves * kDepth * 1024 + kPad];
  char* ring = lds + (threadIdx.x >> 6) * kDepth * 1024;
  stream_region(src + (size_t)blockIdx.x * per_block, per_block, ring);
  if (barrier == 1) grid_barrier_flat(st, 1 << 20);
  if (barrier == 2) grid_barrier_groups(st, 1 << 20);
  stream_region(src + ((size_t)gridDim.x + blockIdx.x) * per_block, per_block, ring);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)(unsigned char)lds[blockIdx.x & 1023];
}

int status(hipError_t e, const char* what) {
  if (e == hipSuccess) return smlp::set_error(SMLP_OK, "");
  char buf[256];
  snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
  return smlp::set_error(SMLP_ERR_HIP, buf);
}

bool bad_region(size_t per_block) { return per_block < 1024 || per_block % 1024 || per_block > ((size_t)1 << 30); }

}  // namespace

extern "C" {

int shared_mlp_ceiling_empty(int blocks, hipStream_t stream) {
  if (blocks < 1 || blocks > 65535) return smlp::set_error(SMLP_ERR_ARG, "blocks outside [1, 65535]");
  (void)hipGetLastError();
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(64), 0, stream, nullptr);
  return status(hipGetLastError(), "empty launch");
}

int shared_mlp_ceiling_read(const void* src, size_t src_bytes, int blocks, size_t bytes_per_block, int shared,
                            float* sink, hipStream_t stream) {
  if (!src || !sink) return smlp::set_error(SMLP_ERR_NULL, "src and sink must be non-NULL");
  if ((uintptr_t)src % 16) return smlp::set_error(SMLP_ERR_ALIGN, "src must be 16-byte aligned");
  if (blocks < 1 || blocks > 65535 || bad_region(bytes_per_block))
    return smlp::set_error(SMLP_ERR_ARG, "blocks outside [1, 65535] or bytes_per_block not a multiple of 1024 in [1 KB, 1 GB]");
  const size_t need = shared ? bytes_per_block : (size_t)blocks * bytes_per_block;
  if (need > src_bytes) return smlp::set_error(SMLP_ERR_SHAPE, "the read runs past src_bytes");
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kWaves * 64), 0, stream, static_cast<const char*>(src),
                     (uint32_t)bytes_per_block, shared ? 1 : 0, sink);
  return status(hipGetLastError(), "read launch");
}

int shared_mlp_ceiling_mfma(int blocks, int iters, float* sink, uint64_t* cycles, uint64_t* ticks,
                            hipStream_t stream) {
  if (!sink || !cycles || !ticks) return smlp::set_error(SMLP_ERR_NULL, "sink, cycles and ticks must be non-NULL");
  if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 24))
    return smlp::set_error(SMLP_ERR_ARG, "blocks outside [1, 65535] or iters outside [1, 2^24]");
  (void)hipGetLastError();
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(512), 0, stream, iters, sink, cycles, ticks);
  return status(hipGetLastError(), "mfma launch");
}

int shared_mlp_ceiling_lds(int blocks, int iters, float* sink, uint64_t* cycles, hipStream_t stream) {
  if (!sink || !cycles) return smlp::set_error(SMLP_ERR_NULL, "sink and cycles must be non-NULL");
  if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 24))
    return smlp::set_error(SMLP_ERR_ARG, "blocks outside [1, 65535] or iters outside [1, 2^24]");
  (void)hipGetLastError();
  hipLaunchKernelGGL(lds_kernel, dim3(blocks), dim3(512), 0, stream, iters, sink, cycles);
  return status(hipGetLastError(), "lds launch");
}

int shared_mlp_ceiling_two_phase(const void* src, size_t src_bytes, int blocks, size_t bytes_per_block,
                                 int barrier, uint32_t* bar_state, float* sink, hipStream_t stream) {
  if (!src || !sink || (barrier && !bar_state))
    return smlp::set_error(SMLP_ERR_NULL, "src, sink (and bar_state with a barrier) must be non-NULL");
  if (barrier < 0 || barrier > 2) return smlp::set_error(SMLP_ERR_ARG, "barrier outside {0, 1, 2}");
  if ((uintptr_t)src % 16 || (bar_state && (uintptr_t)bar_state % 16))
    return smlp::set_error(SMLP_ERR_ALIGN, "src and bar_state must be 16-byte aligned");
  if (blocks < 1 || blocks > 256 || bad_region(bytes_per_block))
    return smlp::set_error(SMLP_ERR_ARG, "blocks outside [1, 256] or bytes_per_block not a multiple of 1024 in [1 KB, 1 GB]");
  if (2 * (size_t)blocks * bytes_per_block > src_bytes)
    return smlp::set_error(SMLP_ERR_SHAPE, "the two phases run past src_bytes");
  (void)hipGetLastError();
  hipLaunchKernelGGL(two_phase_kernel, dim3(blocks), dim3(kWaves * 64), 0, stream, static_cast<const char*>(src),
                     (uint32_t)bytes_per_block, barrier, bar_state, sink);
  return status(hipGetLastError(), "two-phase launch");
}

}  // extern "C"
