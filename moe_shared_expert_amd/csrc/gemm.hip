// LDS-tiled bf16 MFMA GEMM for the gate_up and down stages at larger token counts.
//
// C[M, N] = A[M, K] . B[N, K]^T with both operands K-contiguous (A = x or h, B = the
// weight rows).  A workgroup computes a BM x BN tile of C over a K slice; WM x WN waves
// each own a (BM/WM) x (BN/WN) sub-tile built from 32x32x16 bf16 MFMAs with fp32
// accumulation.
//
// Operands reach LDS by direct buffer-to-LDS loads: one 16-byte load instruction of a
// wave fills a 1 KB block of LDS with 8 tile rows x 128 bytes (one 64-element K step),
// lane p writing slot p.  Lanes pick their global chunk so that slot s of row r holds
// K chunk (s % 8) ^ ((r / 2) % 8); a wave's 8 lanes of a row still cover that row's
// whole 128-byte line, and the sixteen rows read by a quarter-wave for one MFMA
// fragment fall in distinct LDS banks.  No staging registers are needed, so a wave can
// hold a 128 x 128 accumulator tile.  LDS is a ring of NS stages: the loads for step
// k+NS-1 are issued right after the barrier that opens step k, so NS-1 steps of loads
// are in flight while step k is multiplied.
// Rows past M or N and K past the slice use out-of-range buffer offsets, which load
// zeros and move no bytes.
//
// gate_up: the B rows of each wave hold a block of gate rows followed by the matching
// up rows, so a feature's gate and up sums land in the same lane and element of two
// MFMA tiles and SiLU-and-mul is a register operation.  down: A is h as one fp16 plane
// (the weight fragments are converted from bf16 to fp16 after their LDS read, exactly,
// and multiplied with fp16 MFMAs of the same rate), as one bf16 plane (the plain
// projection, A = x), or as two bf16 planes hi + lo (two MFMAs per fragment).  With a K
// split over workgroups the raw fp32 sums go to a partial buffer and a finalize kernel
// applies the epilogue.
//
// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2; the
// (K slice, tile) order gives each XCD a contiguous run, walked in groups of GROUP_M
// token tiles, so the workgroups resident on one XCD share A and B tiles in its L2
// and a K slice of the activations is fetched by one XCD only.
#include "device_common.h"
#include "internal.h"
#include "smlp.h"
#include "tile_configs.h"

namespace smlp {

namespace {


enum { GM_GATE_UP = 0, GM_DOWN_BF16 = 1, GM_DOWN_HILO = 2, GM_DOWN_F16 = 3, GM_DOWN_F16W = 4 };
// Mode flag: weight (B) loads carry the non-temporal bit.  Where every workgroup streams
// its weights exactly once (one token tile, long K, wide weights: the replicated layer at
// M <= 128) this keeps them from displacing the activations that all workgroups re-read
// (replicated gate_up at M = 40 / 64 / 128: 40.2 -> 37.1-38.4, 43.2 -> 39.2-40.8,
// 49.1 -> 45.7 us).  TP shards (short K) and larger M were slower with it.
constexpr int GM_NTB = 8;

struct GArgs {
  const uint16_t* a;      // [M, K] bf16 (down, two planes: hi)
  const uint16_t* a_lo;   // down, two planes: lo plane
  const uint16_t* b;      // [rows, K] bf16
  int M, K;
  int N;                  // output features: h columns (gate_up) or H (down)
  int up_off;             // gate_up: first up row (= I)
  int b_rows;             // rows of b
  int ldb;                // elements between consecutive rows of b (>= K)
  int tiles_m, tiles_n;
  int kslice;             // K elements per workgroup slice (gridDim.y slices)
  void* out;              // gate_up: h plane(s); down: out [M, N] bf16 or fp32
  int ldo;                // down: elements between output rows (>= N)
  float* part;            // gridDim.y > 1: fp32 partial sums [slices][M][P*N]
  int out_f32;
  int h_fmt;              // gate_up: h as one bf16 plane (1), bf16 hi + lo (2) or fp16 (3)
  int ldh;                // gate_up: elements between rows of h (>= N; planes are M * ldh apart)
};

// Format code of h in the kernels: one bf16 plane (1), bf16 hi + lo (2), fp16 (3).
int h_format(int h_dtype) { return h_dtype == SMLP_BF16_HILO ? 2 : h_dtype == SMLP_FP16 ? 3 : 1; }

constexpr int BK = 64;      // K elements per step (128 bytes of a row)
constexpr int GROUP_M = 8;  // token tiles per group in the tile order
constexpr int XCDS = 8;

__device__ __forceinline__ void put_h(void* base, int M, int ld, int m, int n, float h, int fmt) {
  uint16_t* p = reinterpret_cast<uint16_t*>(base);
  if (fmt == 3) {
    p[(size_t)m * ld + n] = (uint16_t)f2h(h);
    return;
  }
  const uint32_t hi = f2bf(h);
  p[(size_t)m * ld + n] = (uint16_t)hi;
  if (fmt == 2) p[(size_t)M * ld + (size_t)m * ld + n] = (uint16_t)f2bf(h - __uint_as_float(hi << 16));
}

// Swizzle of the 16-byte chunks within tile row r.
__device__ __forceinline__ int chunk_swz(int r) { return (r >> 1) & 7; }

// Workgroup -> (K slice, tile_m, tile_n).  Workgroups are dispatched in grid order
// (x fastest) round-robin over the XCDs; the flattened (slice, tile) order is cut into
// one contiguous run per XCD, so an XCD holds whole K slices (the activation slice is
// fetched into one L2 only) and, within a slice, walks GROUP_M token tiles down each
// column of weight tiles before moving right.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn, int& slice) {
  const int tiles = tiles_m * tiles_n;
  const int total = tiles * gridDim.y;
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int per = total / XCDS, rem = total % XCDS;
  const int xcd = lin % XCDS, idx = lin / XCDS;
  // XCD x owns the run starting at x*per + min(x, rem), of length per + (x < rem).
  const int f = xcd * per + (xcd < rem ? xcd : rem) + idx;
  slice = f / tiles;
  const int t = f - slice * tiles;
  const int group = GROUP_M * tiles_n;
  const int gi = t / group;
  const int first = gi * GROUP_M;
  const int gsize = min(tiles_m - first, GROUP_M);
  const int in = t - gi * group;
  tm = first + in % gsize;
  tn = in / gsize;
}

// Workgroup barrier without the memory fence of __syncthreads(), whose release
// semantics would wait for every load in flight, the later steps' LDS loads included.
// The LDS reads of a step are all consumed by its MFMAs (so complete) before the
// barrier; the empty asm statements keep the compiler from moving memory accesses
// across it, and the scheduling barriers keep the multiplies of a step on their side.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Wait until at most `later` steps of LPS loads each are still in flight.
template <int LPS, int MAXL>
__device__ __forceinline__ void wait_steps(int later) {
  if constexpr (MAXL == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= MAXL) wait_vmcnt<MAXL * LPS>();
    else wait_steps<LPS, MAXL - 1>(later);
  }
}

template <int BM, int BN, int WM, int WN, int NS, int MODE>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(GArgs g) {
  constexpr int BASE = MODE & 7;
  constexpr bool NTB = (MODE & GM_NTB) != 0;
  constexpr bool GU = BASE == GM_GATE_UP;
  constexpr bool F16 = BASE == GM_DOWN_F16;      // fp16 h, bf16 weights converted in registers
  constexpr bool F16W = BASE == GM_DOWN_F16W;    // fp16 h, fp16 weights (converted beforehand)
  constexpr int NA = BASE == GM_DOWN_HILO ? 2 : 1;
  constexpr int W = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 32x32 MFMA tiles per wave
  constexpr int AL = BM / 8 / W, BL = BN / 8 / W;      // 1 KB block loads per wave per step
  static_assert(AL * W * 8 == BM && BL * W * 8 == BN, "tile / wave mismatch");
  static_assert(!GU || TN % 2 == 0 || TN == 1, "gate_up pairs gate and up MFMA tiles or columns");
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int STAGE = NA * A_BYTES + B_BYTES;
  constexpr int LPS = NA * AL + BL;  // load instructions per wave per step
  static_assert(NS >= 2 && LPS * (NS - 2) < 64, "stage count");
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  int tile_m, tile_n, slice;
  tile_coords(g.tiles_m, g.tiles_n, tile_m, tile_n, slice);
  const int K = g.K;
  const int kbeg = slice * g.kslice;
  const int kend = min(K, kbeg + g.kslice);
  const int nk = (kend - kbeg + BK - 1) / BK;

  const uint32_t abytes = (uint32_t)g.M * (uint32_t)K * 2u;
  const uint32_t bbytes = ((uint32_t)(g.b_rows - 1) * (uint32_t)g.ldb + (uint32_t)K) * 2u;
  const __amdgpu_buffer_rsrc_t arsc[2] = {make_rsrc(g.a, abytes), make_rsrc(NA == 2 ? g.a_lo : g.a, abytes)};
  const __amdgpu_buffer_rsrc_t brsc = make_rsrc(g.b, bbytes);

  // This lane's slot in each 1 KB block: row p/8, holding global chunk (p%8) ^ swizzle.
  // Block i of this wave covers tile rows (i*W + wave)*8 .. +7.
  const int prow = lane >> 3;
  uint32_t aoff[AL], boff[BL];
  int achk[AL], bchk[BL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int r = (i * W + wave) * 8 + prow;
    achk[i] = (lane & 7) ^ chunk_swz(r);
    const int m = tile_m * BM + r;
    aoff[i] = m < g.M ? (uint32_t)m * (uint32_t)K * 2u + achk[i] * 16 : abytes;
  }
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    const int r = (i * W + wave) * 8 + prow;
    bchk[i] = (lane & 7) ^ chunk_swz(r);
    int row;
    bool ok;
    if (GU) {
      // Each wave column's 32*TN rows: 16*TN gate rows, then the matching up rows.
      const int wc = r / (32 * TN), rr = r % (32 * TN);
      const int f = tile_n * (BN / 2) + wc * 16 * TN + rr % (16 * TN);
      ok = f < g.N;
      row = rr < 16 * TN ? f : g.up_off + f;
    } else {
      row = tile_n * BN + r;
      ok = row < g.N;
    }
    boff[i] = ok ? (uint32_t)row * (uint32_t)g.ldb * 2u + bchk[i] * 16 : bbytes;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Issue load l of one step (of the LPS per wave: A plane q block i at l = q*AL + i,
  // then B block i) into stage `buf` (K elements k0 .. k0+63 of the slice).
  auto issue_one = [&](int buf, int k0, int l) {
    char* st = lds + buf * STAGE;
    const uint32_t kb = (uint32_t)k0 * 2u;
    if (l < NA * AL) {
      const int q = l / AL, i = l % AL;
      const bool ok = aoff[i] != abytes && k0 + achk[i] * 8 < kend;
      buf_ld_lds(arsc[q], st + q * A_BYTES + (i * W + wave) * 1024, ok ? aoff[i] + kb : abytes);
    } else {
      const int i = l - NA * AL;
      const bool ok = boff[i] != bbytes && k0 + bchk[i] * 8 < kend;
      if constexpr (NTB) buf_ld_lds_nt(brsc, st + NA * A_BYTES + (i * W + wave) * 1024, ok ? boff[i] + kb : bbytes);
      else buf_ld_lds(brsc, st + NA * A_BYTES + (i * W + wave) * 1024, ok ? boff[i] + kb : bbytes);
    }
  };
  auto issue = [&](int buf, int k0) {
#pragma unroll
    for (int l = 0; l < LPS; ++l) issue_one(buf, k0, l);
  };

  // 32x32x16 fragments: lane l reads tile row (base + l%32), K chunk 2*ks + l/32.
  // Fragment t of a sub-step: A tiles (plane q, row block i) for t < NA*TM, then B tiles.
  const int fr = lane & 31, fh = lane >> 5;
  const int fsw = chunk_swz(fr);  // row bases are multiples of 32
  constexpr int NFRAG = NA * TM + TN;
  constexpr int NMFMA = NA * TM * TN;
  // Wave tiles with at least as many MFMAs as fragment reads per sub-step (the 256-wide
  // tiles and 128 x 128 on 4 waves) run the pinned schedule below; thinner wave tiles,
  // with too few MFMAs to hide the reads behind, keep the compiler's schedule.
  constexpr bool PINNED = NMFMA >= NFRAG;
  auto mma = [](u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16 || F16W) return mfma32x32x16_f16(a, b, c);
    else return mfma32x32x16(a, b, c);
  };
  u32x4 fa[2][NA][TM], fb[2][TN];
  // Read fragment t of sub-step ks of stage `stage` into slot `slot`.
  auto read_frag = [&](int stage, int slot, int ks, int t) __attribute__((always_inline)) {
    const char* st = lds + stage * STAGE;
    const int coff = ((2 * ks + fh) ^ fsw) * 16;
    if (t < NA * TM) {
      const int q = t / TM, i = t % TM;
      fa[slot][q][i] = *reinterpret_cast<const u32x4*>(st + q * A_BYTES + ((wm * TM + i) * 32 + fr) * 128 + coff);
    } else {
      const int j = t - NA * TM;
      fb[slot][j] = *reinterpret_cast<const u32x4*>(st + NA * A_BYTES + ((wn * TN + j) * 32 + fr) * 128 + coff);
    }
  };

  if constexpr (PINNED) {
    // Pinned schedule, pipelined across K steps.  Each sub-step's MFMAs (fragment slot
    // `cur`) are interleaved with the reads of the next sub-step's fragments into the
    // other slot, two reads ahead of each MFMA, so every read has most of a sub-step of
    // MFMAs to land (left to the compiler, the reads drifted next to their MFMAs and each
    // waited out an LDS round trip: prefill gate_up 1219 -> 1175 us, down 674 -> 657 us).
    // The barrier of step kt sits before its last sub-step, once every wave holds that
    // sub-step's fragments in registers: the last sub-step's MFMAs then cover the barrier
    // skew, the reads of step kt + 1's first fragments and the global loads of step
    // kt + NS into the stage just released.  Those loads are spread one or two per MFMA
    // over that sub-step and the next step's first one (issued in a burst, the eight
    // waves' 64 loads per compute unit overflowed the texture address queue and held
    // up MFMA issue).  Loads stay a full step ahead.  M = 8192: gate_up 1173 -> 1148 us,
    // down 702 -> 688 us against a barrier at the top of each step with the loads in one
    // burst; spread over three sub-steps instead of two, the last loads came too close
    // to the barrier that waits for them (1231 us).
    constexpr int CONV_AT = (NFRAG - 1) / 2 + 3 < NMFMA ? (NFRAG - 1) / 2 + 3 : NMFMA - 1;
    // MFMAs of slot cur; reads of sub-step rks of stage rstage into slot cur ^ 1; loads
    // lo .. hi-1 of the step at lk0 into stage lstage (if ld_on), spread over the MFMAs.
    auto run = [&](int cur, int rstage, int rks, bool ld_on, int lstage, int lk0, int lo, int hi)
        __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < NA; ++q)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int m = (q * TM + i) * TN + j;
#pragma unroll
            for (int r = 0; r < 2; ++r)
              if (2 * m + r < NFRAG) read_frag(rstage, cur ^ 1, rks, 2 * m + r);
            acc[i][j] = mma(fa[cur][q][i], fb[cur][j], acc[i][j]);
            if constexpr (F16) {
              // fp16 mode: the weight fragments just read are converted a few MFMAs
              // after their reads, overlapping the matrix core.
              if (m == CONV_AT) {
#pragma unroll
                for (int jj = 0; jj < TN; ++jj) fb[cur ^ 1][jj] = bf16x8_to_f16x8(fb[cur ^ 1][jj]);
              }
            }
            if (ld_on) {
#pragma unroll
              for (int l = 0; l < LPS; ++l)
                if (l >= lo && l < hi && (l - lo) * NMFMA / (hi - lo) == m) issue_one(lstage, lk0, l);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
      for (int t = 2 * NMFMA; t < NFRAG; ++t) read_frag(rstage, cur ^ 1, rks, t);
      __builtin_amdgcn_sched_barrier(0);
    };
    // Steps 0 .. NS-1 fill the ring; step 0 lands; its first fragments.
#pragma unroll
    for (int st = 0; st < NS; ++st)
      if (st < nk) issue(st, kbeg + st * BK);
    wait_steps<LPS, NS - 1>(min(NS - 1, nk - 1));
    block_barrier();
#pragma unroll
    for (int t = 0; t < NFRAG; ++t) read_frag(0, 0, 0, t);
    if constexpr (F16) {
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[0][j] = bf16x8_to_f16x8(fb[0][j]);
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int HALF = LPS / 2;  // loads issued in the last sub-step; the rest in the next step's first
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt % NS;
      // The second half of step kt + NS - 1's loads (its first half went out in the last
      // sub-step of step kt - 1; the prologue issued steps 0 .. NS-1 whole).
      const bool rest = kt >= 1 && kt + NS - 1 < nk;
      run(0, st, 1, rest, (kt + NS - 1) % NS, kbeg + (kt + NS - 1) * BK, HALF, LPS);
      run(1, st, 2, false, 0, 0, 0, 1);
      run(0, st, 3, false, 0, 0, 0, 1);
      // Every wave holds its last fragments of stage st (lgkmcnt 0) and has step kt + 1
      // in LDS (vmcnt: steps kt + 2 .. kt + NS - 1 may still be in flight); after the
      // barrier, stage st takes step kt + NS.  (After the last step the reads fetch
      // fragments of a stage that are never used, and the barrier is a spare one.)
      __builtin_amdgcn_s_waitcnt(0xc07f);
      wait_steps<LPS, NS - 2>(min(NS - 2, nk - 2 - kt));
      block_barrier();
      run(1, (kt + 1) % NS, 0, kt + NS < nk, st, kbeg + (kt + NS) * BK, 0, HALF);
    }
  } else {
    // One K step: the hook issues the next stage's loads, then the compiler schedules
    // each sub-step's MFMAs with the next sub-step's reads, one read ahead of a share of
    // the MFMAs.
    auto compute = [&](int buf, auto&& hook) {
      hook();
#pragma unroll
      for (int t = 0; t < NFRAG; ++t) read_frag(buf, 0, 0, t);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int cur = ks & 1;
        if (ks < 3) {
#pragma unroll
          for (int t = 0; t < NFRAG; ++t) read_frag(buf, cur ^ 1, ks + 1, t);
        }
        if constexpr (F16) {
#pragma unroll
          for (int j = 0; j < TN; ++j) fb[cur][j] = bf16x8_to_f16x8(fb[cur][j]);
        }
#pragma unroll
        for (int q = 0; q < NA; ++q)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = mma(fa[cur][q][i], fb[cur][j], acc[i][j]);
        if (ks < 3) {
          // Interleave: one fragment read, then a share of the MFMAs.
#pragma unroll
          for (int t = 0; t < NFRAG; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                    // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, NA * TM * TN / NFRAG, 0);  // MFMA
          }
        }
      }
    };
    // NS-stage ring: step kt lives in stage kt % NS; loads run NS-1 steps ahead.
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      if (st < nk) issue(st, kbeg + st * BK);
    for (int kt = 0; kt < nk; ++kt) {
      // Step kt's loads have landed (this wave: vmcnt, allowing the later steps' loads
      // to stay in flight; all waves: the barrier), and no wave still reads the stage
      // that the next loads overwrite (it held step kt-1).
      wait_steps<LPS, NS - 2>(min(NS - 2, nk - 1 - kt));
      block_barrier();
      compute(kt % NS, [&] {
        if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kbeg + (kt + NS - 1) * BK);
      });
    }
  }

  // Epilogue.  32x32 output: lane l, element e -> row 8*(e/4) + 4*(l/32) + e%4, col l%32.
  // K-split partials (read once, by the finalize) and the down output (read once, by the
  // caller) are stored non-temporally, and the finalize loads the partials non-temporally:
  // with weights from HBM, TP16 layers at M = 64 / 128 / 256 18.4 -> 17.7, 19.3 -> 18.1,
  // 23.1 -> 21.2 us, TP8 at M = 256 30.9 -> 29.0 us, replicated at M = 64 / 512 81 -> 75,
  // 213 -> 202 us.  h stays a normal store (the down stage re-reads it).
  // gate_up: MFMA tile j holds gate features and tile j + TN/2 the matching up rows; with
  // one MFMA tile column per wave (TN = 1) its columns 0-15 are gate features and 16-31
  // the matching up rows, brought together by exchanging lanes l and l ^ 16.
  const bool split = gridDim.y > 1;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      // One output row at a time keeps the accumulators from all moving to VGPRs at once.
      __builtin_amdgcn_sched_barrier(0);
      const int m = tile_m * BM + (wm * TM + i) * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
      if constexpr (GU && TN == 1) {
        const float v = acc[i][0][e];
        const float other = __shfl_xor(v, 16);  // every lane, before any lane leaves
        if (m >= g.M) continue;
        const int f = tile_n * (BN / 2) + wn * 16 + (fr & 15);
        if (f >= g.N) continue;
        if (split) {
          float* row = g.part + ((size_t)slice * g.M + m) * (size_t)(2 * g.N);
          __builtin_nontemporal_store(v, &row[(fr < 16 ? 0 : g.N) + f]);
        } else if (fr < 16) {
          put_h(g.out, g.M, g.ldh, m, f, silu_mul(v, other), g.h_fmt);
        }
        continue;
      }
      if (m >= g.M) continue;
      if (GU) {
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
          const int f = tile_n * (BN / 2) + wn * 16 * TN + j * 32 + fr;
          if (f >= g.N) continue;
          const float gate = acc[i][j][e], up = acc[i][j + TN / 2][e];
          if (split) {
            float* row = g.part + ((size_t)slice * g.M + m) * (size_t)(2 * g.N);
            __builtin_nontemporal_store(gate, &row[f]);
            __builtin_nontemporal_store(up, &row[g.N + f]);
          } else {
            put_h(g.out, g.M, g.ldh, m, f, silu_mul(gate, up), g.h_fmt);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = tile_n * BN + (wn * TN + j) * 32 + fr;
          if (n >= g.N) continue;
          const float v = acc[i][j][e];
          if (split)
            __builtin_nontemporal_store(v, &g.part[((size_t)slice * g.M + m) * (size_t)g.N + n]);
          else if (g.out_f32)
            __builtin_nontemporal_store(v, &reinterpret_cast<float*>(g.out)[(size_t)m * g.ldo + n]);
          else
            __builtin_nontemporal_store((uint16_t)f2bf(v), &reinterpret_cast<uint16_t*>(g.out)[(size_t)m * g.ldo + n]);
        }
      }
    }
}

template <int MODE>
int launch_mode(const GemmPlan& gp, const GArgs& a, hipStream_t s) {
  const dim3 grid(gp.tiles, gp.ksplit);
#define SMLP_G(BM_, BN_, WM_, WN_, NS_)                                                          \
  if (gp.bm == BM_ && gp.bn == BN_ && gp.wm == WM_ && gp.wn == WN_ && gp.ns == NS_) {              \
    hipLaunchKernelGGL((gemm_kernel<BM_, BN_, WM_, WN_, NS_, MODE>), grid, dim3(WM_ * WN_ * 64), 0, s, a); \
    return (int)hipGetLastError();                                                               \
  }
  if constexpr ((MODE & GM_NTB) != 0) {
    SMLP_GEMM_NT_CONFIGS(SMLP_G)
  } else {
    if constexpr (MODE != GM_DOWN_HILO && MODE != GM_DOWN_F16W) {
      if (gp.ntb) return launch_mode<MODE | GM_NTB>(gp, a, s);
    }
    if constexpr (MODE == GM_DOWN_HILO) {
      SMLP_GEMM_HILO_CONFIGS(SMLP_G)
    } else {
      SMLP_GEMM_CONFIGS(SMLP_G)
      if constexpr (MODE == GM_DOWN_BF16 || MODE == GM_DOWN_F16 || MODE == GM_DOWN_F16W) {
        SMLP_GEMM_DN_CONFIGS(SMLP_G)
      }
    }
  }
#undef SMLP_G
  return (int)hipErrorInvalidConfiguration;
}

}  // namespace

int launch_gemm_gate_up(const Plan& p, const void* x, const void* w_gate_up, void* ws, hipStream_t s) {
  GArgs a{};
  a.a = reinterpret_cast<const uint16_t*>(x);
  a.a_lo = nullptr;
  a.b = reinterpret_cast<const uint16_t*>(w_gate_up);
  a.M = (int)p.M;
  a.K = (int)p.H;
  a.N = (int)p.I;
  a.up_off = (int)p.up_off;
  a.b_rows = (int)(p.up_off + p.I);
  a.ldb = (int)p.H;
  a.tiles_m = p.ggu.tiles_m;
  a.tiles_n = p.ggu.tiles / p.ggu.tiles_m;
  a.kslice = p.ggu.kslice;
  a.out = static_cast<char*>(ws) + p.h_offset;
  a.ldo = a.N;
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_offset);
  a.out_f32 = 0;
  a.h_fmt = h_format(p.h_dtype);
  a.ldh = a.N;
  if (p.gu_split) {
    // Features [0, gu_split) with the main tile, then the rest with the tail tile: each
    // launch sees its own gate rows (its up rows up_off further on) and h columns.
    if (a.h_fmt == 2 || p.ggu.ksplit != 1 || p.ggu_tail.ksplit != 1) return (int)hipErrorInvalidConfiguration;
    a.N = (int)p.gu_split;
    int rc = launch_mode<GM_GATE_UP>(p.ggu, a, s);
    if (rc) return rc;
    GArgs t = a;
    t.b = a.b + (size_t)p.gu_split * a.ldb;
    t.N = (int)(p.I - p.gu_split);
    t.b_rows = t.up_off + t.N;
    t.tiles_m = p.ggu_tail.tiles_m;
    t.tiles_n = p.ggu_tail.tiles / p.ggu_tail.tiles_m;
    t.kslice = p.ggu_tail.kslice;
    t.out = static_cast<char*>(a.out) + (size_t)p.gu_split * 2;
    return launch_mode<GM_GATE_UP>(p.ggu_tail, t, s);
  }
  int rc = launch_mode<GM_GATE_UP>(p.ggu, a, s);
  if (rc || p.ggu.ksplit == 1) return rc;
  return launch_finalize(true, a.part, p.ggu.ksplit, a.M, a.N, a.out, a.N, 0, a.h_fmt, s);
}

int launch_gemm_down(const Plan& p, const void* w_down, void* out, void* ws, hipStream_t s) {
  GArgs a{};
  const uint16_t* h = reinterpret_cast<const uint16_t*>(static_cast<const char*>(ws) + p.h_offset);
  a.a = h;
  a.a_lo = h + (size_t)p.M * p.I;
  a.b = reinterpret_cast<const uint16_t*>(w_down);
  a.M = (int)p.M;
  a.K = (int)p.I;
  a.N = (int)p.H;
  a.up_off = 0;
  a.b_rows = (int)p.H;
  a.ldb = (int)p.ldwd;
  a.tiles_m = p.gdn.tiles_m;
  a.tiles_n = p.gdn.tiles / p.gdn.tiles_m;
  a.kslice = p.gdn.kslice;
  a.out = out;
  a.ldo = a.N;
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_offset);
  a.out_f32 = p.partial_fp32 ? 1 : 0;
  a.h_fmt = h_format(p.h_dtype);
  if (p.wd16_bytes) {
    // fp16 h against an fp16 copy of the weights, converted once before the GEMM
    int rc = launch_bf16_to_f16(w_down, p.ldwd, p.H, p.I, static_cast<char*>(ws) + p.wd16_offset, s);
    if (rc) return rc;
    a.b = reinterpret_cast<const uint16_t*>(static_cast<const char*>(ws) + p.wd16_offset);
    a.ldb = (int)p.I;
  }
  // one plane of h: fp16 (weights fp16 already, or converted in registers) or bf16
  auto one_plane = [&](const GemmPlan& gp, const GArgs& args) {
    if (p.h_dtype != SMLP_FP16) return launch_mode<GM_DOWN_BF16>(gp, args, s);
    return p.wd16_bytes ? launch_mode<GM_DOWN_F16W>(gp, args, s) : launch_mode<GM_DOWN_F16>(gp, args, s);
  };
  if (p.dn_split) {
    // Columns [0, dn_split) with the main tile, then the rest with the tail tile: each
    // launch sees its own weight rows and output columns (row stride H).  Planned for
    // one plane of h only.
    if (p.h_dtype == SMLP_BF16_HILO || p.gdn.ksplit != 1 || p.gdn_tail.ksplit != 1)
      return (int)hipErrorInvalidConfiguration;
    a.N = (int)p.dn_split;
    a.b_rows = a.N;
    a.ldo = (int)p.H;
    int rc = one_plane(p.gdn, a);
    if (rc) return rc;
    GArgs t = a;
    t.b = a.b + (size_t)p.dn_split * a.ldb;
    t.N = (int)(p.H - p.dn_split);
    t.b_rows = t.N;
    t.tiles_m = p.gdn_tail.tiles_m;
    t.tiles_n = p.gdn_tail.tiles / p.gdn_tail.tiles_m;
    t.kslice = p.gdn_tail.kslice;
    t.out = static_cast<char*>(out) + (size_t)p.dn_split * (a.out_f32 ? 4 : 2);
    return one_plane(p.gdn_tail, t);
  }
  int rc = p.h_dtype == SMLP_BF16_HILO ? launch_mode<GM_DOWN_HILO>(p.gdn, a, s) : one_plane(p.gdn, a);
  if (rc || p.gdn.ksplit == 1) return rc;
  return launch_finalize(false, a.part, p.gdn.ksplit, a.M, a.N, out, a.N, a.out_f32, 1, s);
}

// A plain projection y = x . w^T runs the down stage's one-plane kernel with A = x.
int launch_gemm_linear(const GemmPlan& gp, const void* x, const void* w, void* y, int M, int K,
                       int N, int ldy, int out_f32, float* part, hipStream_t s) {
  GArgs a{};
  a.a = reinterpret_cast<const uint16_t*>(x);
  a.a_lo = nullptr;
  a.b = reinterpret_cast<const uint16_t*>(w);
  a.M = M;
  a.K = K;
  a.N = N;
  a.up_off = 0;
  a.b_rows = N;
  a.ldb = K;
  a.tiles_m = gp.tiles_m;
  a.tiles_n = gp.tiles / gp.tiles_m;
  a.kslice = gp.kslice;
  a.out = y;
  a.ldo = ldy;
  a.part = part;
  a.out_f32 = out_f32;
  a.h_fmt = 1;
  int rc = launch_mode<GM_DOWN_BF16>(gp, a, s);
  if (rc || gp.ksplit == 1) return rc;
  return launch_finalize(false, part, gp.ksplit, M, N, y, ldy, out_f32, 1, s);
}

}  // namespace smlp
