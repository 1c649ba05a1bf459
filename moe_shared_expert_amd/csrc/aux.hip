// fp32 path (plain fp32 kernels for any shape), the per-rank weight slice copy, and the
// per-token RMS rescale used between the layers of a stacked chain.
#include "device_common.h"
#include "internal.h"
#include "smlp.h"

namespace smlp {

// h[m, i] = SiLU(sum_k x[m,k] Wg[i,k]) * (sum_k x[m,k] Wu[i,k]), fp32, one thread per (m, i).
__global__ __launch_bounds__(256) void fp32_gate_up_kernel(const float* __restrict__ x,
                                                           const float* __restrict__ w, int M,
                                                           int H, int I, int up_off,
                                                           float* __restrict__ h) {
  const size_t total = (size_t)M * I;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t m = e / I, i = e % I;
    const float* xr = x + m * H;
    const float* gr = w + i * H;
    const float* ur = w + ((size_t)up_off + i) * H;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < H; ++k) {
      g = fmaf(xr[k], gr[k], g);
      u = fmaf(xr[k], ur[k], u);
    }
    h[e] = silu_mul(g, u);
  }
}

// out[m, n] = sum_i h[m, i] Wd[n, i], fp32, one thread per (m, n).
__global__ __launch_bounds__(256) void fp32_down_kernel(const float* __restrict__ h,
                                                        const float* __restrict__ wd, int M,
                                                        int H, int I, int ldw,
                                                        float* __restrict__ out) {
  const size_t total = (size_t)M * H;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t m = e / H, n = e % H;
    const float* hr = h + m * I;
    const float* wr = wd + n * ldw;
    float acc = 0.f;
    for (int i = 0; i < I; ++i) acc = fmaf(hr[i], wr[i], acc);
    out[e] = acc;
  }
}

// The whole fp32 layer in one workgroup when h fits in LDS (the small equivalence-test
// shapes, where two dependent launches cost more than the arithmetic): the same
// per-element loops as the two kernels above (fmaf over k, then over i, in order), so
// the same bits, with h held in LDS between the stages.
__global__ __launch_bounds__(256) void fp32_layer_small_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               const float* __restrict__ wd, int M, int H,
                                                               int I, int up_off, int ldw,
                                                               float* __restrict__ out) {
  __shared__ float h[kFp32SmallH];
  for (int e = threadIdx.x; e < M * I; e += blockDim.x) {
    const int m = e / I, i = e % I;
    const float* xr = x + (size_t)m * H;
    const float* gr = w + (size_t)i * H;
    const float* ur = w + ((size_t)up_off + i) * H;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < H; ++k) {
      g = fmaf(xr[k], gr[k], g);
      u = fmaf(xr[k], ur[k], u);
    }
    h[e] = silu_mul(g, u);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < M * H; e += blockDim.x) {
    const int m = e / H, n = e % H;
    const float* hr = h + m * I;
    const float* wr = wd + (size_t)n * ldw;
    float acc = 0.f;
    for (int i = 0; i < I; ++i) acc = fmaf(hr[i], wr[i], acc);
    out[e] = acc;
  }
}

int launch_fp32_layer(const Plan& p, const float* x, const float* w_gate_up, const float* w_down, float* out,
                      hipStream_t s) {
  if (!fp32_small_layer(p.M, p.H, p.I)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(fp32_layer_small_kernel, dim3(1), dim3(256), 0, s, x, w_gate_up, w_down, (int)p.M,
                     (int)p.H, (int)p.I, (int)p.up_off, (int)p.ldwd, out);
  return (int)hipGetLastError();
}

static int grid_for(size_t total) {
  size_t b = (total + 255) / 256;
  return (int)(b > 8192 ? 8192 : (b < 1 ? 1 : b));
}

int launch_fp32_gate_up(const Plan& p, const float* x, const float* w_gate_up, void* ws,
                        hipStream_t s) {
  float* h = reinterpret_cast<float*>(static_cast<char*>(ws) + p.h_offset);
  hipLaunchKernelGGL(fp32_gate_up_kernel, dim3(grid_for((size_t)p.M * p.I)), dim3(256), 0, s, x,
                     w_gate_up, (int)p.M, (int)p.H, (int)p.I, (int)p.up_off, h);
  return (int)hipGetLastError();
}

int launch_fp32_down(const Plan& p, const float* w_down, float* out, void* ws, hipStream_t s) {
  const float* h = reinterpret_cast<const float*>(static_cast<const char*>(ws) + p.h_offset);
  hipLaunchKernelGGL(fp32_down_kernel, dim3(grid_for((size_t)p.M * p.H)), dim3(256), 0, s, h,
                     w_down, (int)p.M, (int)p.H, (int)p.I, (int)p.ldwd, out);
  return (int)hipGetLastError();
}

// Rank slice copy, element by element (T = uint16_t for bf16, uint32_t for fp32).
//   dst_gu[j, k]     = src_gu[r*s + j, k]         j <  s
//   dst_gu[s + j, k] = src_gu[I + r*s + j, k]     j <  s
//   dst_wd[n, j]     = src_wd[n, r*s + j]
template <typename T>
__global__ __launch_bounds__(256) void slice_rank_kernel(const T* __restrict__ gu,
                                                         const T* __restrict__ wd,
                                                         T* __restrict__ gu_r,
                                                         T* __restrict__ wd_r, int64_t H,
                                                         int64_t I, int64_t s, int64_t r) {
  const int64_t n_gu = 2 * s * H, n_wd = H * s;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n_gu + n_wd;
       e += (int64_t)gridDim.x * blockDim.x) {
    if (e < n_gu) {
      const int64_t row = e / H, k = e % H;
      const int64_t src_row = row < s ? r * s + row : I + r * s + (row - s);
      gu_r[e] = gu[src_row * H + k];
    } else {
      const int64_t f = e - n_gu;
      const int64_t n = f / s, j = f % s;
      wd_r[f] = wd[n * I + r * s + j];
    }
  }
}

int launch_slice_rank(const void* wgu, const void* wd, void* wgu_r, void* wd_r, int64_t H,
                      int64_t I, int tp, int rank, int elem_bytes, hipStream_t s) {
  const int64_t sl = I / tp;
  const size_t total = (size_t)(3 * sl * H);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(slice_rank_kernel<uint16_t>, dim3(grid_for(total)), dim3(256), 0, s,
                       (const uint16_t*)wgu, (const uint16_t*)wd, (uint16_t*)wgu_r,
                       (uint16_t*)wd_r, H, I, sl, (int64_t)rank);
  else
    hipLaunchKernelGGL(slice_rank_kernel<uint32_t>, dim3(grid_for(total)), dim3(256), 0, s,
                       (const uint32_t*)wgu, (const uint32_t*)wd, (uint32_t*)wgu_r,
                       (uint32_t*)wd_r, H, I, sl, (int64_t)rank);
  return (int)hipGetLastError();
}

// out[m, :] = bf16(in[m, :] * (1 / sqrt(mean(in[m, :]^2)))), one workgroup per row.
__global__ __launch_bounds__(256) void rms_rescale_kernel(const float* __restrict__ in,
                                                          uint16_t* __restrict__ out, int H) {
  const int m = blockIdx.x;
  const float4* row = reinterpret_cast<const float4*>(in + (size_t)m * H);
  const int nv = H / 4;
  float ss = 0.f;
  for (int v = threadIdx.x; v < nv; v += blockDim.x) {
    const float4 q = row[v];
    ss = fmaf(q.x, q.x, ss);
    ss = fmaf(q.y, q.y, ss);
    ss = fmaf(q.z, q.z, ss);
    ss = fmaf(q.w, q.w, ss);
  }
  // wave reduction then across the 4 waves
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float total = part[0] + part[1] + part[2] + part[3];
  const float scale = 1.0f / sqrtf(total / (float)H);
  u32x2* orow = reinterpret_cast<u32x2*>(out + (size_t)m * H);
  for (int v = threadIdx.x; v < nv; v += blockDim.x) {
    const float4 q = row[v];
    orow[v] = u32x2{pack_bf2(q.x * scale, q.y * scale), pack_bf2(q.z * scale, q.w * scale)};
  }
}

// Rows of up to 8192 elements: the row is held in registers (one 16-byte load per thread
// per 2048 elements, all in flight at once), reduced in a fixed order (per thread,
// across the wave, across the 8 waves), then scaled and stored from the registers.
template <int VPT>
__global__ __launch_bounds__(512) void rms_rescale_reg_kernel(const float* __restrict__ in,
                                                              uint16_t* __restrict__ out, int H) {
  const int m = blockIdx.x;
  const float4* row = reinterpret_cast<const float4*>(in + (size_t)m * H);
  const int nv = H / 4;
  float4 q[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = threadIdx.x + i * 512;
    q[i] = v < nv ? row[v] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    ss = fmaf(q[i].x, q[i].x, ss);
    ss = fmaf(q[i].y, q[i].y, ss);
    ss = fmaf(q[i].z, q[i].z, ss);
    ss = fmaf(q[i].w, q[i].w, ss);
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  __shared__ float part[8];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) total += part[w];
  const float scale = 1.0f / sqrtf(total / (float)H);
  u32x2* orow = reinterpret_cast<u32x2*>(out + (size_t)m * H);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = threadIdx.x + i * 512;
    if (v < nv)
      orow[v] = u32x2{pack_bf2(q[i].x * scale, q[i].y * scale), pack_bf2(q[i].z * scale, q[i].w * scale)};
  }
}

int launch_rms_rescale(const float* in, uint16_t* out, int64_t M, int64_t H, hipStream_t s) {
  if (H <= 2048)
    hipLaunchKernelGGL(rms_rescale_reg_kernel<1>, dim3((unsigned)M), dim3(512), 0, s, in, out, (int)H);
  else if (H <= 4096)
    hipLaunchKernelGGL(rms_rescale_reg_kernel<2>, dim3((unsigned)M), dim3(512), 0, s, in, out, (int)H);
  else if (H <= 8192)
    hipLaunchKernelGGL(rms_rescale_reg_kernel<4>, dim3((unsigned)M), dim3(512), 0, s, in, out, (int)H);
  else
    hipLaunchKernelGGL(rms_rescale_kernel, dim3((unsigned)M), dim3(256), 0, s, in, out, (int)H);
  return (int)hipGetLastError();
}

}  // namespace smlp

namespace smlp {

// bf16 -> fp16 copy of a weight matrix (rows x cols, source row stride ld_src elements,
// destination dense), eight elements per thread; exact for every value in the fp16
// normal range (see bf16x8_to_f16x8).
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                          int64_t rows, int64_t cols, uint16_t* __restrict__ dst) {
  const int64_t c8 = cols / 8, total = rows * c8;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / c8, c = (e % c8) * 8;
    const u32x4 v = ld_stream(src + r * ld_src + c);
    *reinterpret_cast<u32x4*>(dst + r * cols + c) = bf16x8_to_f16x8(v);
  }
}

int launch_bf16_to_f16(const void* src, int64_t ld_src, int64_t rows, int64_t cols, void* dst, hipStream_t s) {
  if (cols % 8 || ld_src % 8) return (int)hipErrorInvalidValue;
  const int64_t total = rows * (cols / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(bf16_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const uint16_t*>(src),
                     ld_src, rows, cols, static_cast<uint16_t*>(dst));
  return (int)hipGetLastError();
}

}  // namespace smlp
