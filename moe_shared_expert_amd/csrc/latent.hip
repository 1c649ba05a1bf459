// Restore of the logical column order of a gathered merged-column projection output
// (vLLM PR 345, "[II] TP-shard Kimi MLA latent projections", Behavior and Technical
// reason).
//
// The merged projection's output columns are R logical ranges (q_a, then kv_a).  Rank r
// holds piece r of every range (each range cut into tp equal pieces), in range order,
// so a gathered row is laid out rank by rank.  Logical column o_t + r p_t + c (range t
// at offset o_t, piece length p_t = size_t / tp) comes from gathered column
// r (N / tp) + o_t / tp + c.
//
// A pure copy bound by HBM bandwidth: each thread moves one unit of U bytes, the
// largest power of two up to 16 that divides every piece (and both base addresses), so
// the writes are coalesced full-width stores and the reads are contiguous within a
// piece.
#include "device_common.h"
#include "internal.h"
#include "smlp_latent.h"

namespace smlp {

namespace {

struct RestoreArgs {
  const char* src;
  char* dst;
  int M;
  int row_units;   // units of U bytes per row
  int rank_units;  // units per rank block of a gathered row (N / tp columns)
  int nr;          // ranges
  int lo[SMLP_MAX_RANGES];     // first logical unit of range t
  int piece[SMLP_MAX_RANGES];  // units per piece of range t
  int src0[SMLP_MAX_RANGES];   // first unit of range t's piece inside a rank block
};

template <typename T>
__global__ __launch_bounds__(256) void restore_kernel(RestoreArgs a) {
  const T* src = reinterpret_cast<const T*>(a.src);
  T* dst = reinterpret_cast<T*>(a.dst);
  const size_t total = (size_t)a.M * a.row_units;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(e / a.row_units), u = (int)(e % a.row_units);
    int t = 0;
#pragma unroll
    for (int j = 1; j < SMLP_MAX_RANGES; ++j)
      if (j < a.nr && u >= a.lo[j]) t = j;
    const int q = u - a.lo[t];
    const int r = q / a.piece[t], c = q - r * a.piece[t];
    const size_t row = (size_t)m * a.row_units;
    dst[row + u] = src[row + (size_t)r * a.rank_units + a.src0[t] + c];
  }
}

}  // namespace

int launch_restore_logical(const void* src, void* dst, int64_t M, int64_t N, const int64_t* sizes,
                           int nr, int tp, int elem_bytes, hipStream_t s) {
  // Unit: the largest power of two <= 16 bytes dividing every piece and both addresses.
  int64_t g = 0;
  for (int t = 0; t < nr; ++t) {
    int64_t v = sizes[t] / tp * elem_bytes, a = g;
    while (v) {  // g = gcd(g, v)
      const int64_t r = a % v;
      a = v;
      v = r;
    }
    g = a;
  }
  int U = 16;
  while (U > elem_bytes && (g % U || (uintptr_t)src % U || (uintptr_t)dst % U)) U /= 2;
  RestoreArgs a{};
  a.src = static_cast<const char*>(src);
  a.dst = static_cast<char*>(dst);
  a.M = (int)M;
  a.row_units = (int)(N * elem_bytes / U);
  a.rank_units = (int)(N / tp * elem_bytes / U);
  a.nr = nr;
  int64_t off = 0;
  for (int t = 0; t < nr; ++t) {
    a.lo[t] = (int)(off * elem_bytes / U);
    a.piece[t] = (int)(sizes[t] / tp * elem_bytes / U);
    a.src0[t] = (int)(off / tp * elem_bytes / U);
    off += sizes[t];
  }
  const size_t total = (size_t)M * a.row_units;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  switch (U) {
    case 16: hipLaunchKernelGGL(restore_kernel<u32x4>, dim3(blocks), dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(restore_kernel<u32x2>, dim3(blocks), dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(restore_kernel<uint32_t>, dim3(blocks), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(restore_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, a); break;
  }
  return (int)hipGetLastError();
}

}  // namespace smlp
