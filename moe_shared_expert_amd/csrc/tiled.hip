// LDS-tiled bf16 MFMA GEMM kernels for large token counts (prefill).
//
// C[M, N] = A[M, K] . B[N, K]^T with both operands K-contiguous.  A workgroup of 4
// waves computes a 128 x 128 tile of C; the A and B tiles for a 64-wide K step are
// staged in LDS (double-buffered, XOR-swizzled 16-byte chunks to avoid bank
// conflicts) and fed to 16x16x32 bf16 MFMAs.  For the gate_up stage the 128 B rows
// of a tile are 64 gate rows and the 64 matching up rows, so each wave holds gate
// and up accumulators for the same (token, feature) pairs and applies SiLU-and-mul
// in registers; h is stored once, as bf16, or (for small intermediate sizes, where
// one rounding of h would not average out over the down contraction) as two bf16
// planes hi + lo, which the down stage multiplies with two MFMAs per fragment.
#include "device_common.h"
#include "internal.h"
#include "smlp.h"

namespace smlp {

namespace {

constexpr int BM = 128, BN = 128, BK = 64, THREADS = 256;
constexpr int CHUNKS = BK / 8;  // 16-byte chunks per tile row

struct TArgs {
  const uint16_t* a;   // [M, K] bf16 (down with two planes: the hi plane)
  const uint16_t* a_lo;  // down with two planes: the lo plane
  const uint16_t* b;   // [rows, K] bf16
  int M, K;
  int N;               // output features (h columns for gate_up, H for down)
  int up_off;          // gate_up: first up row (= I)
  int tiles_m;
  void* out;           // gate_up: h bf16 [M, N] (plus the lo plane); down: out [M, N]
  int out_f32;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * CHUNKS + (chunk ^ (row & 7)); }

// HL: gate_up stores h as hi + lo planes / down reads them.
template <bool GU, bool HL>
__global__ __launch_bounds__(THREADS) void tiled_kernel(TArgs t) {
  constexpr int NA = (!GU && HL) ? 2 : 1;
  __shared__ u32x4 lds_a[NA][2][BM * CHUNKS];
  __shared__ u32x4 lds_b[2][BN * CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const int tile_m = blockIdx.x % t.tiles_m;
  const int tile_n = blockIdx.x / t.tiles_m;
  const int K = t.K;

  // Global -> LDS copy assignment: each thread moves 4 chunks of A and 4 of B.
  const char* ga[NA][4];
  const char* gb[4];
  int lrow[4], lchk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * THREADS;      // 0..1023
    lrow[i] = c / CHUNKS;
    lchk[i] = c % CHUNKS;
    int m = tile_m * BM + lrow[i];
    m = m < t.M ? m : t.M - 1;
#pragma unroll
    for (int q = 0; q < NA; ++q)
      ga[q][i] = reinterpret_cast<const char*>(q ? t.a_lo : t.a) + ((size_t)m * K + lchk[i] * 8) * 2;
    int brow;
    if (GU) {
      const int half = lrow[i] >> 6, r = lrow[i] & 63;
      int n = tile_n * (BN / 2) + r;
      n = n < t.N ? n : t.N - 1;
      brow = half ? t.up_off + n : n;
    } else {
      int n = tile_n * BN + lrow[i];
      brow = n < t.N ? n : t.N - 1;
    }
    gb[i] = reinterpret_cast<const char*>(t.b) + ((size_t)brow * K + lchk[i] * 8) * 2;
  }

  // B row tiles of this wave (16 rows each), as row offsets inside the B tile.
  int btile[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) btile[q] = GU ? ((q >> 1) * 64 + wn * 32 + (q & 1) * 16) : (wn * 64 + q * 16);

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[NA][4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool v = k0 + lchk[i] * 8 < K;
#pragma unroll
      for (int q = 0; q < NA; ++q) ra[q][i] = v ? ld16(ga[q][i] + (size_t)k0 * 2) : u32x4{0, 0, 0, 0};
      rb[i] = v ? ld16(gb[i] + (size_t)k0 * 2) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < NA; ++q) lds_a[q][buf][swz(lrow[i], lchk[i])] = ra[q][i];
      lds_b[buf][swz(lrow[i], lchk[i])] = rb[i];
    }
  };

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 fa[NA][4], fb[4];
#pragma unroll
      for (int qa = 0; qa < NA; ++qa)
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[qa][i] = lds_a[qa][buf][swz(wm * 64 + i * 16 + ln, ks * 4 + lg)];
#pragma unroll
      for (int q = 0; q < 4; ++q) fb[q] = lds_b[buf][swz(btile[q] + ln, ks * 4 + lg)];
#pragma unroll
      for (int qa = 0; qa < NA; ++qa)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][q] = mfma16x16x32(fa[qa][i], fb[q], acc[i][q]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = tile_m * BM + wm * 64 + i * 16 + lg * 4 + j;
      if (m >= t.M) continue;
      if (GU) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int n = tile_n * (BN / 2) + wn * 32 + q * 16 + ln;
          if (n < t.N) {
            const float hv = silu_mul(acc[i][q][j], acc[i][q + 2][j]);
            const uint32_t hi = f2bf(hv);
            uint16_t* hp = reinterpret_cast<uint16_t*>(t.out);
            hp[(size_t)m * t.N + n] = (uint16_t)hi;
            if (HL) hp[(size_t)t.M * t.N + (size_t)m * t.N + n] = (uint16_t)f2bf(hv - __uint_as_float(hi << 16));
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = tile_n * BN + wn * 64 + q * 16 + ln;
          if (n >= t.N) continue;
          if (t.out_f32)
            reinterpret_cast<float*>(t.out)[(size_t)m * t.N + n] = acc[i][q][j];
          else
            reinterpret_cast<uint16_t*>(t.out)[(size_t)m * t.N + n] = (uint16_t)f2bf(acc[i][q][j]);
        }
      }
    }
}

}  // namespace

int launch_tiled_gate_up(const Plan& p, const void* x, const void* w_gate_up, void* ws,
                         hipStream_t s) {
  TArgs t;
  t.a = reinterpret_cast<const uint16_t*>(x);
  t.b = reinterpret_cast<const uint16_t*>(w_gate_up);
  t.M = (int)p.M;
  t.K = (int)p.H;
  t.N = (int)p.I;
  t.up_off = (int)p.I;
  t.tiles_m = (int)((p.M + BM - 1) / BM);
  t.a_lo = nullptr;
  t.out = static_cast<char*>(ws) + p.h_offset;
  t.out_f32 = 0;
  if (p.h_dtype == SMLP_BF16_HILO)
    hipLaunchKernelGGL((tiled_kernel<true, true>), dim3(p.tgu.blocks), dim3(THREADS), 0, s, t);
  else
    hipLaunchKernelGGL((tiled_kernel<true, false>), dim3(p.tgu.blocks), dim3(THREADS), 0, s, t);
  return (int)hipGetLastError();
}

int launch_tiled_down(const Plan& p, const void* w_down, void* out, void* ws, hipStream_t s) {
  TArgs t;
  t.a = reinterpret_cast<const uint16_t*>(static_cast<const char*>(ws) + p.h_offset);
  t.a_lo = t.a + (size_t)p.M * p.I;
  t.b = reinterpret_cast<const uint16_t*>(w_down);
  t.M = (int)p.M;
  t.K = (int)p.I;
  t.N = (int)p.H;
  t.up_off = 0;
  t.tiles_m = (int)((p.M + BM - 1) / BM);
  t.out = out;
  t.out_f32 = p.partial_fp32 ? 1 : 0;
  if (p.h_dtype == SMLP_BF16_HILO)
    hipLaunchKernelGGL((tiled_kernel<false, true>), dim3(p.tdn.blocks), dim3(THREADS), 0, s, t);
  else
    hipLaunchKernelGGL((tiled_kernel<false, false>), dim3(p.tdn.blocks), dim3(THREADS), 0, s, t);
  return (int)hipGetLastError();
}

}  // namespace smlp
