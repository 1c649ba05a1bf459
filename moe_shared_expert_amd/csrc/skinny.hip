// Weight-streaming kernels for small token counts (decode): the gate_up projection
// with the SiLU-and-mul epilogue, and the down projection.
//
// Shape of the work: C[M, N] = A[M, K] . W[N, K]^T with M small (<= 128) and W large.
// Every weight byte is used by all M tokens and by nothing else, so the kernels are
// bound by streaming W from HBM once.  Each wave owns a block of 16 output features
// (for gate_up: 16 gate rows and the 16 matching up rows) and a slice of K; it loads
// 16-byte pieces of W straight into registers in the layout the 16x16x32 bf16 MFMA
// takes as its B operand, loads the matching pieces of A (L2-resident) as the A
// operand, and accumulates in fp32.  K is split over the waves of a workgroup
// (reduced through LDS) and optionally over workgroups (reduced by a second,
// elementwise kernel that also applies the epilogue).
#include "device_common.h"
#include "internal.h"
#include "smlp.h"

namespace smlp {

struct SkArgs {
  const void* act;     // [M, K]: bf16 (x) or fp32 (h)
  const uint16_t* w;   // [rows, K] bf16
  int M, K, N;         // N: output features per row group (I for gate_up, H for down)
  int up_off;          // gate_up: first row of the up projection (= I)
  int kslice;          // K elements per workgroup (multiple of 64)
  void* out;           // ksplit == 1: final output [M, N]
  float* part;         // ksplit > 1: partial sums [ksplit][M][P*N]
  int out_f32;         // down: fp32 (1) or bf16 (0) output
};

// AF32: activations are fp32 and are fed to the MFMA as bf16 hi + bf16 lo parts
// (hi = rne(v), lo = rne(v - hi)), which keeps ~16 mantissa bits of h.
// GU: gate_up stage (two row groups per feature block, SiLU-and-mul epilogue).
template <int MT, int NB, int WAVES, int U, bool AF32, bool GU>
__global__ __launch_bounds__(WAVES * 64) void skinny_kernel(SkArgs a) {
  constexpr int P = GU ? 2 : 1;
  constexpr int AB = AF32 ? 4 : 2;  // bytes per activation element
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = a.K;

  const char* wrow[P][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int n = (blockIdx.x * NB + nb) * 16 + ln;
    n = n < a.N ? n : a.N - 1;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      int row = p ? a.up_off + n : n;
      wrow[p][nb] = reinterpret_cast<const char*>(a.w) + ((size_t)row * K + lg * 8) * 2;
    }
  }
  const char* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int m = mt * 16 + ln;
    m = m < a.M ? m : a.M - 1;
    arow[mt] = reinterpret_cast<const char*>(a.act) + ((size_t)m * K + lg * 8) * AB;
  }

  f32x4 acc[P][NB][MT];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[p][nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kbeg = blockIdx.y * a.kslice;
  const int kend = min(K, kbeg + a.kslice);
  constexpr int STEP = 64 * WAVES * U;

  for (int kit = kbeg; kit < kend; kit += STEP) {
    u32x4 bw[U][2][P][NB];
    u32x4 av[U][2][MT][AF32 ? 2 : 1];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int koff = kit + (u * WAVES + wave) * 64 + j * 32;  // + lg*8 folded in pointers
        const bool valid = koff + lg * 8 < kend;
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            bw[u][j][p][nb] = valid ? ld_stream(wrow[p][nb] + (size_t)koff * 2) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (AF32) {
            av[u][j][mt][0] = valid ? ld16(arow[mt] + (size_t)koff * 4) : u32x4{0, 0, 0, 0};
            av[u][j][mt][AF32 ? 1 : 0] =
                valid ? ld16(arow[mt] + (size_t)koff * 4 + 16) : u32x4{0, 0, 0, 0};
          } else {
            av[u][j][mt][0] = valid ? ld16(arow[mt] + (size_t)koff * 2) : u32x4{0, 0, 0, 0};
          }
        }
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          u32x4 ahi, alo;
          if (AF32) {
            const u32x4 v0 = av[u][j][mt][0], v1 = av[u][j][mt][AF32 ? 1 : 0];
            float f[8] = {__uint_as_float(v0.x), __uint_as_float(v0.y), __uint_as_float(v0.z),
                          __uint_as_float(v0.w), __uint_as_float(v1.x), __uint_as_float(v1.y),
                          __uint_as_float(v1.z), __uint_as_float(v1.w)};
            uint32_t hb[8], lb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              hb[e] = f2bf(f[e]);
              lb[e] = f2bf(f[e] - __uint_as_float(hb[e] << 16));
            }
            ahi = u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16),
                        hb[6] | (hb[7] << 16)};
            alo = u32x4{lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16),
                        lb[6] | (lb[7] << 16)};
          } else {
            ahi = av[u][j][mt][0];
          }
#pragma unroll
          for (int p = 0; p < P; ++p)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              acc[p][nb][mt] = mfma16x16x32(ahi, bw[u][j][p][nb], acc[p][nb][mt]);
              if (AF32) acc[p][nb][mt] = mfma16x16x32(alo, bw[u][j][p][nb], acc[p][nb][mt]);
            }
        }
  }

  // Reduce the WAVES K-slices of the workgroup through LDS, in wave order.
  constexpr int NF = P * NB * MT;
  if constexpr (WAVES > 1) {
    __shared__ f32x4 red[WAVES][NF][64];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[wave][(p * NB + nb) * MT + mt][lane] = acc[p][nb][mt];
    __syncthreads();
    // Output unit q = (nb, mt) is finished by wave q % WAVES.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (((nb * MT + mt) % WAVES) != wave) continue;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          f32x4 s = red[0][(p * NB + nb) * MT + mt][lane];
#pragma unroll
          for (int w = 1; w < WAVES; ++w) s += red[w][(p * NB + nb) * MT + mt][lane];
          acc[p][nb][mt] = s;
        }
      }
  }

  const int ksplit = gridDim.y;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (WAVES > 1 && ((nb * MT + mt) % WAVES) != wave) continue;
      const int n = (blockIdx.x * NB + nb) * 16 + ln;
      if (n >= a.N) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = mt * 16 + lg * 4 + j;
        if (m >= a.M) continue;
        if (ksplit > 1) {
          float* dst = a.part + ((size_t)blockIdx.y * a.M + m) * (size_t)(P * a.N) + n;
          dst[0] = acc[0][nb][mt][j];
          if (GU) dst[a.N] = acc[P - 1][nb][mt][j];
        } else if (GU) {
          reinterpret_cast<float*>(a.out)[(size_t)m * a.N + n] =
              silu_mul(acc[0][nb][mt][j], acc[P - 1][nb][mt][j]);
        } else if (a.out_f32) {
          reinterpret_cast<float*>(a.out)[(size_t)m * a.N + n] = acc[0][nb][mt][j];
        } else {
          reinterpret_cast<uint16_t*>(a.out)[(size_t)m * a.N + n] =
              (uint16_t)f2bf(acc[0][nb][mt][j]);
        }
      }
    }
}

// Sum the ksplit partials in slice order and apply the stage's epilogue.
template <bool GU>
__global__ __launch_bounds__(256) void skinny_finalize(const float* __restrict__ part,
                                                       int ksplit, int M, int N, void* out,
                                                       int out_f32) {
  const int P = GU ? 2 : 1;
  const size_t total = (size_t)M * N;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const size_t m = e / N, n = e % N;
    float g = 0.f, u = 0.f;
    for (int s = 0; s < ksplit; ++s) {
      const float* src = part + ((size_t)s * M + m) * (size_t)(P * N) + n;
      g += src[0];
      if (GU) u += src[N];
    }
    if (GU)
      reinterpret_cast<float*>(out)[e] = silu_mul(g, u);
    else if (out_f32)
      reinterpret_cast<float*>(out)[e] = g;
    else
      reinterpret_cast<uint16_t*>(out)[e] = (uint16_t)f2bf(g);
  }
}

template <bool AF32, bool GU>
static int launch_stage(const SkinnyPlan& sp, const SkArgs& a, hipStream_t s) {
  dim3 grid(sp.blocks / sp.ksplit, sp.ksplit);
  dim3 block(sp.waves * 64);
#define SMLP_SK(MT_, NB_, U_)                                                             \
  if (sp.mt == MT_ && sp.nb == NB_ && sp.waves == 4) {                                   \
    hipLaunchKernelGGL((skinny_kernel<MT_, NB_, 4, U_, AF32, GU>), grid, block, 0, s, a); \
    return (int)hipGetLastError();                                                       \
  }
  SMLP_SK(1, 1, 2) SMLP_SK(2, 1, 2) SMLP_SK(4, 1, 1) SMLP_SK(8, 1, 1)
  SMLP_SK(1, 2, 2) SMLP_SK(2, 2, 2) SMLP_SK(4, 2, 1) SMLP_SK(8, 2, 1)
#undef SMLP_SK
  return (int)hipErrorInvalidConfiguration;
}

static int finalize(bool gu, const float* part, int ksplit, int M, int N, void* out, int out_f32,
                    hipStream_t s) {
  const size_t total = (size_t)M * N;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (gu)
    hipLaunchKernelGGL(skinny_finalize<true>, dim3(blocks), dim3(256), 0, s, part, ksplit, M, N,
                       out, out_f32);
  else
    hipLaunchKernelGGL(skinny_finalize<false>, dim3(blocks), dim3(256), 0, s, part, ksplit, M, N,
                       out, out_f32);
  return (int)hipGetLastError();
}

int launch_skinny_gate_up(const Plan& p, const void* x, const void* w_gate_up, void* ws,
                          hipStream_t s) {
  SkArgs a;
  a.act = x;
  a.w = reinterpret_cast<const uint16_t*>(w_gate_up);
  a.M = (int)p.M;
  a.K = (int)p.H;
  a.N = (int)p.I;
  a.up_off = (int)p.I;
  a.kslice = p.gu.kslice;
  a.out = static_cast<char*>(ws) + p.h_offset;
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_offset);
  a.out_f32 = 1;
  int rc = launch_stage<false, true>(p.gu, a, s);
  if (rc || p.gu.ksplit == 1) return rc;
  return finalize(true, a.part, p.gu.ksplit, a.M, a.N, a.out, 1, s);
}

int launch_skinny_down(const Plan& p, const void* w_down, void* out, void* ws, hipStream_t s) {
  SkArgs a;
  a.act = static_cast<const char*>(ws) + p.h_offset;
  a.w = reinterpret_cast<const uint16_t*>(w_down);
  a.M = (int)p.M;
  a.K = (int)p.I;
  a.N = (int)p.H;
  a.up_off = 0;
  a.kslice = p.dn.kslice;
  a.out = out;
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_offset);
  a.out_f32 = p.partial_fp32 ? 1 : 0;
  int rc = launch_stage<true, false>(p.dn, a, s);
  if (rc || p.dn.ksplit == 1) return rc;
  return finalize(false, a.part, p.dn.ksplit, a.M, a.N, out, a.out_f32, s);
}

}  // namespace smlp
