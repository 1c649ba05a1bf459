// Weight-streaming kernels for small token counts (decode): the gate_up projection
// with the SiLU-and-mul epilogue, the down projection, and a plain projection y = x.w^T
// (the merged MLA latent projection, streaming kind only).
//
// Shape of the work: C[M, N] = A[M, K] . W[N, K]^T with M small (<= 128) and W large.
// Every weight byte is used by all M tokens and by nothing else, so the kernels are
// bound by streaming W from HBM once.  A wave owns NB blocks of 16 output features
// (for gate_up: each block is 16 gate rows plus the 16 matching up rows) and a share
// of K, and accumulates with 16x16x32 bf16 MFMAs in fp32.
//
// Memory access: the MFMA operand layout puts 16 different rows in the 16 lanes of
// each lane group, so loading operands directly in that layout makes every load
// instruction touch 16 cache lines (64 bytes of each).  Measured on MI355X that caps
// streaming at ~4-5 TB/s; loading 8 rows x 128 contiguous bytes per instruction (8
// full lines) streams at the rate of a plain linear read.  For M <= 32 the streaming
// kernel therefore moves each 64-element K step of a wave's weight and activation
// rows in that 8-row layout straight into a wave-private LDS ring (direct
// buffer-to-LDS loads, chunks XOR-swizzled so the MFMA fragment reads are free of
// bank conflicts) and keeps several K steps in flight with explicit vmcnt waits.  For
// larger M the direct kernel loads MFMA operands straight into registers.  The K
// range of a workgroup is interleaved over its waves in 64-element steps and reduced
// through LDS in a fixed tree order; a K split over workgroups (for shapes with few
// feature blocks) is reduced by a second, elementwise kernel that also applies the
// epilogue.
//
// The intermediate h is handed from gate_up to down either as one bf16 plane (rounded
// once; the down stage is then the one-plane projection mode) or as two bf16 planes,
// hi = rne(h) and lo = rne(h - hi), which together carry ~16 significant bits; with
// two planes the down kernel multiplies both (two MFMAs per fragment), so h is
// effectively not rounded.  The planner picks one plane unless the down contraction
// is short.
#include <mutex>

#include "device_common.h"
#include "internal.h"
#include "smlp.h"
#include "tile_configs.h"

namespace smlp {

// Kernel modes: the gate_up stage, the down stage reading h as two bf16 planes, and a
// plain projection (one bf16 activation plane, no epilogue; streaming kind only).
enum { MODE_GATE_UP = 0, MODE_DOWN_HILO = 1, MODE_LINEAR = 2 };

struct SkArgs {
  const uint16_t* a_hi;  // [M, K] bf16 activations (x), or the hi plane of h
  const uint16_t* a_lo;  // [M, K] lo plane of h (down stage only)
  const uint16_t* w;     // [rows, K] bf16
  int M, K, N;           // N: output features per row group (I for gate_up, H for down)
  int up_off;            // gate_up: first row of the up projection (= I)
  int kslice;            // K elements per workgroup (multiple of 64)
  void* out;             // ksplit == 1: gate_up -> h planes, down -> out [M, N]
  int ldo;               // down / projection: elements between output rows (>= N)
  float* part;           // ksplit > 1: partial sums [ksplit][M][P*N]
  int out_f32;           // down: fp32 (1) or bf16 (0) output
  int h_planes;          // gate_up (and its finalize): h planes to store (1 or 2)
  int fpw;               // LDS kernel: features (gate_up) or rows (down) per workgroup
  int w_rows;            // rows of w
  int ldw;               // elements between consecutive rows of w (>= K)
  // ksplit > 1: per-column arrival counters (16 words apart, zero between launches) with
  // which the last-arriving slice of a column sums the partials and applies the epilogue
  // in the same launch; null: a finalize launch does that.
  uint32_t* red_cnt;
};

// Store element (m, n) of h: rne(h) in the first plane and, with two planes, the
// rounding remainder rne(h - hi) in the second.
__device__ __forceinline__ void store_h(void* base, int M, int N, int m, int n, float h,
                                        int planes) {
  uint16_t* p = reinterpret_cast<uint16_t*>(base);
  if (planes == 3) {  // one fp16 plane (the format the tiled down stage reads for bf16 outputs)
    p[(size_t)m * N + n] = (uint16_t)f2h(h);
    return;
  }
  const uint32_t hi = f2bf(h);
  p[(size_t)m * N + n] = (uint16_t)hi;
  if (planes == 2) p[(size_t)M * N + (size_t)m * N + n] = (uint16_t)f2bf(h - __uint_as_float(hi << 16));
}

// One bf16 plane of h stored agent-coherent (write-through past this XCD's L2), for a
// consumer on another XCD in the same launch.
__device__ __forceinline__ void store_h_coherent(void* base, int M, int N, int m, int n, float h) {
  (void)M;
  __hip_atomic_store(reinterpret_cast<uint16_t*>(base) + (size_t)m * N + n, (uint16_t)f2bf(h), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Direct buffer-to-LDS load that misses in this XCD's L2 when the line may be stale
// (agent-coherent), to read data another XCD wrote in the same launch.
__device__ __forceinline__ void buf_ld_lds_coherent(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)off, 0, 0, 16);
}

// LDS bytes the cross-wave reduction needs.
template <int MT, int NB, int WAVES, bool GU>
constexpr int lds_red_bytes() {
  return WAVES > 1 ? (WAVES / 2) * (GU ? 2 : 1) * NB * MT * 64 * 16 : 16;
}

// Reduce the WAVES K-shares of a workgroup as a fixed binary tree through LDS, then
// let wave 0 write the partial sums (K split) or apply the stage's epilogue.
// `lds` is a 16-byte aligned buffer of at least lds_red_bytes<...>() bytes.
template <int MT, int NB, int WAVES, bool GU>
__device__ __forceinline__ void finish_workgroup(const SkArgs& a,
                                                 f32x4 (&acc)[GU ? 2 : 1][NB][MT], char* lds) {
  constexpr int P = GU ? 2 : 1;
  constexpr int NF = P * NB * MT;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  if constexpr (WAVES > 1) {
    f32x4* red = reinterpret_cast<f32x4*>(lds);
    __syncthreads();
#pragma unroll
    for (int half = WAVES / 2; half >= 1; half /= 2) {
      if (wave >= half && wave < 2 * half) {
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              red[((wave - half) * NF + (p * NB + nb) * MT + mt) * 64 + lane] = acc[p][nb][mt];
      }
      __syncthreads();
      if (wave < half) {
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[p][nb][mt] += red[(wave * NF + (p * NB + nb) * MT + mt) * 64 + lane];
      }
      __syncthreads();
    }
  }
  if (wave != 0) return;

  const int ksplit = gridDim.y;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
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
          store_h(a.out, a.M, a.N, m, n, silu_mul(acc[0][nb][mt][j], acc[P - 1][nb][mt][j]), a.h_planes);
        } else if (a.out_f32) {
          reinterpret_cast<float*>(a.out)[(size_t)m * a.ldo + n] = acc[0][nb][mt][j];
        } else {
          reinterpret_cast<uint16_t*>(a.out)[(size_t)m * a.ldo + n] = (uint16_t)f2bf(acc[0][nb][mt][j]);
        }
      }
    }
}

// Streaming kernel (M <= 32).  A workgroup owns the contiguous feature range
// [col * fpw, +fpw) and a K slice; the range is cut into NT 16-row MFMA tiles.
// gate_up tiles pack 8 features: rows 0-7 are their gate rows and rows 8-15 their up
// rows; down tiles are 16 consecutive rows.  The K slice is interleaved over the waves
// in 64-element steps.  Each operand block reaches a wave-private LDS ring by direct
// buffer-to-LDS loads: a
// 16-byte load per lane fills 1 KB with 8 rows x 128 bytes (one 64-element K step),
// lane p writing slot p, the lane choosing its global chunk so that slot s of row r
// holds chunk (s % 8) ^ ((r / 2) % 8) and the 16-row fragment reads are free of bank
// conflicts.  No registers hold loads in flight, so the ring can keep STAGES - 1 K
// steps of loads in flight per wave, with explicit vmcnt waits; the ring is private
// to the wave, so the loop needs no barrier.  Steps past the slice load zeros (no
// memory traffic), so the loop issues ahead without branches.
template <int MT, int NT, int WAVES, int STAGES, int MODE>
constexpr int stream_lds_bytes() {
  constexpr int NA = MODE == MODE_DOWN_HILO ? 2 : 1;
  constexpr int WAVE_LDS = STAGES * (NT + NA * MT) * 2048;
  constexpr int RED_LDS = lds_red_bytes<MT, NT, WAVES, false>();
  return WAVES * WAVE_LDS > RED_LDS ? WAVES * WAVE_LDS : RED_LDS;
}

// s_waitcnt vmcnt(n) for an n known only after unrolling (0 <= n <= MAX).
template <int MAX>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if constexpr (MAX == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAX) wait_vmcnt<MAX>();
    else wait_vmcnt_le<MAX - 1>(n);
  }
}

// Role of a streaming stage inside the one-launch decode layer (decode_layer_kernel):
// none (a stage of its own), the gate_up producer (h stored agent-coherent), or the
// down consumer (weight loads issued before h is ready; h loaded agent-coherent).
enum { FUSE_NONE = 0, FUSE_PRODUCER = 1, FUSE_CONSUMER = 2 };

struct StreamSync {
  const uint32_t* ready;  // consumer: its ready flag
  uint32_t target;        // consumer: the flag value that means h is complete
  int limit;              // consumer: polls before giving up
  int* flag;              // consumer: an LDS word outside the ring
};

// Wait (thread 0 polling, the workgroup behind a barrier) until *sy.ready holds
// sy.target, for at most sy.limit polls; returns false if it gave up.
__device__ __forceinline__ bool wait_ready(const StreamSync& sy) {
  if (threadIdx.x == 0) {
    bool ok = false;
    for (int n = 0; n < sy.limit; ++n) {
      if (__hip_atomic_load(sy.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == sy.target) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    *reinterpret_cast<volatile int*>(sy.flag) = ok;
  }
  __syncthreads();
  return *reinterpret_cast<volatile int*>(sy.flag) != 0;
}

template <int MT, int NT, int WAVES, int STAGES, int MODE, int FUSE>
__device__ __forceinline__ void stream_body(const SkArgs& a, char* lds, int col, int slice, int ksplit,
                                            int m0, const StreamSync& sy) {
  constexpr bool GU = MODE == MODE_GATE_UP;
  constexpr int NA = MODE == MODE_DOWN_HILO ? 2 : 1;  // activation planes: x, or h hi + lo
  constexpr int TA = NA * MT;           // activation tiles per K step
  constexpr int TT = NT + TA;           // 2 KB tiles per K step
  constexpr int SLOT = TT * 2048;       // one ring slot: one K step of this wave
  constexpr int WAVE_LDS = STAGES * SLOT;
  constexpr int LW = 2 * NT, LA = 2 * TA;  // 1 KB weight / activation loads per K step
  constexpr int LPS = LW + LA;             // 1 KB loads per K step
  constexpr int LDS_BYTES = stream_lds_bytes<MT, NT, WAVES, STAGES, MODE>();
  static_assert(STAGES >= 2 && LPS * (STAGES - 1) < 64, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS per workgroup");
  static_assert(FUSE != FUSE_CONSUMER || (LPS * STAGES < 64 && MODE != MODE_GATE_UP), "consumer ring");
  static_assert(FUSE != FUSE_PRODUCER || MODE == MODE_GATE_UP, "producer stage");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int lr = lane >> 3;  // row within a 1 KB block
  const int K = a.K;
  char* my = lds + wave * WAVE_LDS;

  const int f0 = col * a.fpw;
  const int fend = min(a.N, f0 + a.fpw);
  const uint32_t wbytes = ((uint32_t)(a.w_rows - 1) * (uint32_t)a.ldw + (uint32_t)K) * 2u;
  const uint32_t abytes = (uint32_t)a.M * (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, wbytes);
  const __amdgpu_buffer_rsrc_t ar[2] = {make_rsrc(a.a_hi, abytes), make_rsrc(NA == 2 ? a.a_lo : a.a_hi, abytes)};

  // Block h of a tile holds tile rows 8h .. 8h+7; this lane loads row 8h + lr, chunk
  // ch[h].  Per-lane row byte offsets (chunk included) or the out-of-range marker.
  int ch[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) ch[h] = (lane & 7) ^ (((8 * h + lr) >> 1) & 7);
  uint32_t wo[NT][2], ao[TA][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int row;
      bool ok;
      if (GU) {
        const int f = f0 + 8 * t + lr;  // rows 0-7: gate rows, rows 8-15: the matching up rows
        ok = f < fend;
        row = h ? a.up_off + f : f;
      } else {
        row = f0 + 16 * t + 8 * h + lr;
        ok = row < fend;
      }
      wo[t][h] = ok ? (uint32_t)row * (uint32_t)a.ldw * 2u + ch[h] * 16 : wbytes;
    }
#pragma unroll
  for (int q = 0; q < NA; ++q)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = m0 + mt * 16 + 8 * h + lr;
        ao[q * MT + mt][h] = m < a.M ? (uint32_t)m * (uint32_t)K * 2u + ch[h] * 16 : abytes;
      }

  f32x4 acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kbeg = slice * a.kslice;
  const int kend = min(K, kbeg + a.kslice);
  constexpr int STEP = 64 * WAVES;
  const int nst = (kend - kbeg + STEP - 1) / STEP;

  // Issue the weight or activation loads of K step i of this wave into ring slot `slot`.
  auto issue_w = [&](int slot, int i) {
    const int k = kbeg + (i * WAVES + wave) * 64;
    const uint32_t kb = (uint32_t)k * 2u;
    char* sl = my + slot * SLOT;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        buf_ld_lds_nt(wr, sl + t * 2048 + h * 1024,
                      (k + ch[h] * 8 < kend && wo[t][h] != wbytes) ? wo[t][h] + kb : wbytes);
  };
  auto issue_a = [&](int slot, int i) {
    const int k = kbeg + (i * WAVES + wave) * 64;
    const uint32_t kb = (uint32_t)k * 2u;
    char* sl = my + slot * SLOT;
#pragma unroll
    for (int t = 0; t < TA; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t off = (k + ch[h] * 8 < kend && ao[t][h] != abytes) ? ao[t][h] + kb : abytes;
        if constexpr (FUSE == FUSE_CONSUMER) buf_ld_lds_coherent(ar[t / MT], sl + (NT + t) * 2048 + h * 1024, off);
        else buf_ld_lds(ar[t / MT], sl + (NT + t) * 2048 + h * 1024, off);
      }
  };
  auto issue = [&](int slot, int i) {
    issue_w(slot, i);
    issue_a(slot, i);
  };
  // Multiply the K step in ring slot `slot`: 16x16x32 fragments, lane (ln, lg) reads
  // tile row ln, chunk 4j + lg.
  const int fsw = (ln >> 1) & 7;
  auto compute = [&](int slot) {
    const char* sl = my + slot * SLOT;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int off = ln * 128 + (((4 * j + lg) ^ fsw) * 16);
      u32x4 fb[NT], fa[TA];
#pragma unroll
      for (int t = 0; t < NT; ++t) fb[t] = *reinterpret_cast<const u32x4*>(sl + t * 2048 + off);
#pragma unroll
      for (int t = 0; t < TA; ++t) fa[t] = *reinterpret_cast<const u32x4*>(sl + (NT + t) * 2048 + off);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < NA; ++q)
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t][mt] = mfma16x16x32(fa[q * MT + mt], fb[t], acc[t][mt]);
    }
  };

  int slot = 0;  // ring slot of step i
  int i0 = 0;
  bool ready = true;
  if constexpr (FUSE == FUSE_CONSUMER) {
    // The weights do not depend on h: the weight blocks of the first STAGES steps (the
    // whole ring) go out before the wait, then the matching h blocks.  Loads complete in
    // issue order, so step i < STAGES - 1 waits with the h blocks of steps i + 1 ..
    // STAGES - 1 and the i steps issued since still in flight; from step STAGES - 1 on,
    // the loop below runs as usual.
#pragma unroll
    for (int p = 0; p < STAGES; ++p) issue_w(p, p);
    ready = wait_ready(sy);
#pragma unroll
    for (int p = 0; p < STAGES; ++p) issue_a(p, p);
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i) {
      if (i >= 1) issue(i - 1, i + STAGES - 1);
      wait_vmcnt_le<LPS * (STAGES - 1)>((STAGES - 1 - i) * LA + i * LPS);
      if (i < nst) compute(i);
    }
    slot = STAGES - 1;
    i0 = STAGES - 1;
  } else {
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p) issue(p, p);
  }
  for (int i = i0; i < nst; ++i) {
    // The slot of step i - 1 (multiplied in the previous iteration) takes step
    // i + STAGES - 1; then wait until step i has landed, STAGES - 1 later steps may
    // stay in flight.
    issue(slot == 0 ? STAGES - 1 : slot - 1, i + STAGES - 1);
    wait_vmcnt<LPS * (STAGES - 1)>();
    compute(slot);
    slot = slot == STAGES - 1 ? 0 : slot + 1;
  }
  wait_vmcnt<0>();  // the loads issued past the end write zeros into the ring

  // Reduce the WAVES K-shares of the workgroup through LDS (reusing the ring), as a
  // fixed binary tree.
  if constexpr (WAVES > 1) {
    f32x4* red = reinterpret_cast<f32x4*>(lds);
    __syncthreads();
#pragma unroll
    for (int half = WAVES / 2; half >= 1; half /= 2) {
      if (wave >= half && wave < 2 * half) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) red[((wave - half) * NT * MT + t * MT + mt) * 64 + lane] = acc[t][mt];
      }
      __syncthreads();
      if (wave < half) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[t][mt] += red[(wave * NT * MT + t * MT + mt) * 64 + lane];
      }
      __syncthreads();
    }
  }
  // With a K split reduced in this launch, every wave stays for the last-arriving
  // workgroup's reduction below.
  const bool reduce_here = ksplit > 1 && a.red_cnt != nullptr;
  if (wave != 0 && !reduce_here) return;

  // Epilogue.  MFMA output: lane (ln, lg), element j = (token mt*16 + 4*lg + j, column ln).
  // A consumer whose wait gave up writes NaN.  K-split partial sums are stored
  // agent-coherent when the last-arriving slice reads them in this launch.
  const float poison = ready ? 0.f : __builtin_nanf("");
  if (wave == 0) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + mt * 16 + lg * 4 + j;
        const float v = acc[t][mt][j];
        if (GU) {
          const float up = __shfl_xor(v, 8, 64);  // column ln ^ 8 of the same row
          const int f = f0 + 8 * t + (ln & 7);
          if (m >= a.M || f >= fend) continue;
          if (ksplit > 1) {
            // lanes 0-7 hold gate columns, lanes 8-15 the matching up columns
            float* dst = a.part + ((size_t)slice * a.M + m) * (size_t)(2 * a.N) + (ln < 8 ? f : a.N + f);
            if (reduce_here) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *dst = v;
          } else if (ln < 8) {
            if constexpr (FUSE == FUSE_PRODUCER) store_h_coherent(a.out, a.M, a.N, m, f, silu_mul(v, up));
            else store_h(a.out, a.M, a.N, m, f, silu_mul(v, up), a.h_planes);
          }
        } else {
          const int n = f0 + 16 * t + ln;
          if (m >= a.M || n >= fend) continue;
          if (ksplit > 1) {
            float* dst = a.part + ((size_t)slice * a.M + m) * (size_t)a.N + n;
            if (reduce_here) __hip_atomic_store(dst, v + poison, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *dst = v + poison;
          } else if (a.out_f32) {
            reinterpret_cast<float*>(a.out)[(size_t)m * a.ldo + n] = v + poison;
          } else {
            reinterpret_cast<uint16_t*>(a.out)[(size_t)m * a.ldo + n] = (uint16_t)f2bf(v + poison);
          }
        }
      }
  }
  if (!reduce_here) return;

  // In-launch reduction of the K split: once its stores are complete, wave 0 counts this
  // slice on the column's counter; the last slice to arrive clears the counter and, with
  // all its waves, sums every slice's partials in slice order (agent-coherent loads; the
  // same order and arithmetic as the finalize kernel) and applies the epilogue.
  wait_vmcnt<0>();
  __syncthreads();
  int* const last_flag = reinterpret_cast<int*>(lds);  // the rings and the tree are done with
  if (threadIdx.x == 0) {
    uint32_t* c = a.red_cnt + 16 * col;
    const uint32_t prev = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == (uint32_t)ksplit - 1;
    if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *reinterpret_cast<volatile int*>(last_flag) = last;
  }
  __syncthreads();
  if (!*reinterpret_cast<volatile int*>(last_flag)) return;
  constexpr int P = GU ? 2 : 1;
  const uint32_t pbytes = (uint32_t)ksplit * (uint32_t)a.M * (uint32_t)(P * a.N) * 4u;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.part, pbytes);
  const uint32_t sstride = (uint32_t)a.M * (uint32_t)(P * a.N) * 4u;
  constexpr int COLS = GU ? 8 * NT : 16 * NT;  // outputs per token row of this workgroup
  constexpr int SB = 16;                       // slices in flight per batch
  for (int e = threadIdx.x; e < 16 * MT * COLS; e += WAVES * 64) {
    const int m = m0 + e / COLS, c = f0 + e % COLS;
    if (m >= a.M || c >= fend) continue;
    const uint32_t base = ((uint32_t)m * (uint32_t)(P * a.N) + (uint32_t)c) * 4u;
    float g = 0.f, u = 0.f;
    for (int s0 = 0; s0 < ksplit; s0 += SB) {
      float pg[SB], pu[SB];
#pragma unroll
      for (int q = 0; q < SB; ++q)
        if (s0 + q < ksplit) {
          const uint32_t o = base + (uint32_t)(s0 + q) * sstride;
          pg[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (int)o, 0, 16));
          if (GU) pu[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (int)(o + 4u * a.N), 0, 16));
        }
#pragma unroll
      for (int q = 0; q < SB; ++q)
        if (s0 + q < ksplit) {
          g += pg[q];
          if (GU) u += pu[q];
        }
    }
    if (GU) {
      store_h(a.out, a.M, a.N, m, c, silu_mul(g, u), a.h_planes);
    } else if (a.out_f32) {
      reinterpret_cast<float*>(a.out)[(size_t)m * a.ldo + c] = g;
    } else {
      reinterpret_cast<uint16_t*>(a.out)[(size_t)m * a.ldo + c] = (uint16_t)f2bf(g);
    }
  }
}

template <int MT, int NT, int WAVES, int STAGES, int MODE>
__global__ __launch_bounds__(WAVES * 64) void skinny_stream_kernel(SkArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[stream_lds_bytes<MT, NT, WAVES, STAGES, MODE>()];
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).  With
  // a K split, the (slice, column) order is cut into one contiguous run per XCD, so an
  // XCD holds whole K slices and fetches only its slices of the activations.
  int col = blockIdx.x, slice = blockIdx.y;
  if (gridDim.y > 1) {
    const int total = gridDim.x * gridDim.y;
    const int lin = blockIdx.y * gridDim.x + blockIdx.x;
    const int xcd = lin % 8, per = total / 8, rem = total % 8;
    const int t = xcd * per + min(xcd, rem) + lin / 8;
    slice = t / gridDim.x;
    col = t % gridDim.x;
  }
  // Token split (gridDim.z > 1): workgroup z takes tokens [16 MT z, 16 MT (z + 1)); the
  // workgroups of one feature range are 8 apart in dispatch order when gridDim.x % 8 == 0,
  // so they share an XCD and its L2 copy of the weights.
  stream_body<MT, NT, WAVES, STAGES, MODE, FUSE_NONE>(a, lds, col, slice, gridDim.y, blockIdx.z * 16 * MT,
                                                     StreamSync{});
}

// One-launch decode layer: the gate_up stage (producers, blockIdx.x < producers, 4
// waves) and the down projection over one bf16 plane of h (consumers, 8 waves) in one
// grid.  Workgroups are dispatched in index order, so every producer has been placed
// on a compute unit before any consumer, and a consumer only waits for producers,
// which wait for nothing: the launch cannot deadlock, whatever else shares the GPU.
// A consumer starts on a compute unit as soon as a producer leaves it, issues its
// first weight loads, and waits until h is complete before it loads h.  Producers
// store h agent-coherent and count themselves once their stores are complete;
// consumers load h agent-coherent.
//
// Counters (one slot per stream, words 256 bytes apart so that no memory channel takes
// all the traffic): [64 g] producers of group g done (g < 16, producer b in group
// b % 16), [64 * 16] groups done, [64 * (17 + f)] ready flag f (f < 16, consumer c polls
// flag c % 16), [64 * 33] consumers done, [64 * 34] the slot's generation G.  Every
// workgroup reads G when it starts; G only changes when the last consumer ends, after
// every workgroup has read it.  The last producer of a group clears the group's count,
// the last group clears the groups' count and stores G + 1 in every ready flag, and the
// last consumer clears the consumers' count and stores G + 1 in the generation, so the
// slot is ready for the next launch on the same stream without being cleared from the
// host.  A consumer that gives up waiting (limit polls) writes NaN.
constexpr int kSyncGroups = 16;
constexpr int kSyncWords = 64 * 35;

template <int MT, int NTG, int SG, int NTD, int SD, int WD>
__global__ __launch_bounds__((WD > 4 ? WD : 4) * 64) void decode_layer_kernel(SkArgs gu, SkArgs dn, uint32_t* sync,
                                                                            int producers, int limit) {
  constexpr int LG = stream_lds_bytes<MT, NTG, 4, SG, MODE_GATE_UP>();
  constexpr int LD = stream_lds_bytes<MT, NTD, WD, SD, MODE_LINEAR>();
  // The consumer's ready flag sits in a 1 KB pad after the rings: a workgroup LDS size
  // that is not a whole number of KB (a separate 4-byte variable) slowed the streaming
  // loops by ~10% on MI355X (gate_up phase 26.6 -> 29.8 us at M = 16).
  constexpr int RING = LG > LD ? LG : LD;
  __shared__ __attribute__((aligned(1024))) char lds[RING + 1024];
  int& flag = *reinterpret_cast<int*>(lds + RING);
  uint32_t* const gen_word = sync + 64 * 34;
  if ((int)blockIdx.x < producers) {
    if (threadIdx.x >= 256) return;
    uint32_t gen = 0;
    if (threadIdx.x == 0) gen = __hip_atomic_load(gen_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stream_body<MT, NTG, 4, SG, MODE_GATE_UP, FUSE_PRODUCER>(gu, lds, blockIdx.x, 0, 1, 0, StreamSync{});
    if (threadIdx.x < 64) {  // wave 0 wrote h
      wait_vmcnt<0>();
      if (threadIdx.x == 0) {
        const int g = blockIdx.x % kSyncGroups;
        const uint32_t members = producers / kSyncGroups + (g < producers % kSyncGroups ? 1u : 0u);
        const uint32_t groups = producers < kSyncGroups ? producers : kSyncGroups;
        const uint32_t prev = __hip_atomic_fetch_add(sync + 64 * g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == members - 1) {
          __hip_atomic_store(sync + 64 * g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t top =
              __hip_atomic_fetch_add(sync + 64 * kSyncGroups, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (top == groups - 1) {
            __hip_atomic_store(sync + 64 * kSyncGroups, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int f = 0; f < kSyncGroups; ++f)
              __hip_atomic_store(sync + 64 * (17 + f), gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    return;
  }
  const int c = blockIdx.x - producers;
  const uint32_t consumers = gridDim.x - (uint32_t)producers;
  // Thread 0 polls and ends the workgroup's part, so only it reads the generation.
  uint32_t gen = 0;
  if (threadIdx.x == 0) gen = __hip_atomic_load(gen_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const StreamSync sy{sync + 64 * (17 + c % kSyncGroups), gen + 1u, limit, &flag};
  if (threadIdx.x >= WD * 64) return;
  stream_body<MT, NTD, WD, SD, MODE_LINEAR, FUSE_CONSUMER>(dn, lds, c, 0, 1, 0, sy);
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(sync + 64 * 33, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == consumers - 1) {
      __hip_atomic_store(sync + 64 * 33, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(gen_word, gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Counter slots of the one-launch decode layer (one per stream that uses it, per device).
__device__ uint32_t g_layer_sync[kLayerSyncSlots * kSyncWords];

// Direct-load variant for larger token tiles (MT >= 4), where staging every
// activation tile through LDS per wave would not fit: operands are loaded straight
// into registers in the MFMA layout.
template <int MT, int NB, int WAVES, int U, int MODE>
__global__ __launch_bounds__(WAVES * 64) void skinny_direct_kernel(SkArgs a) {
  constexpr bool GU = MODE == MODE_GATE_UP;
  constexpr int P = GU ? 2 : 1;                      // row groups per feature block
  constexpr int NA = GU ? 1 : 2;                      // activation planes: x, or h hi + lo
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
      const int row = p ? a.up_off + n : n;
      wrow[p][nb] = reinterpret_cast<const char*>(a.w) + ((size_t)row * a.ldw + lg * 8) * 2;
    }
  }
  const char* arow[NA][MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int m = mt * 16 + ln;
    m = m < a.M ? m : a.M - 1;
#pragma unroll
    for (int q = 0; q < NA; ++q)
      arow[q][mt] = reinterpret_cast<const char*>(q ? a.a_lo : a.a_hi) + ((size_t)m * K + lg * 8) * 2;
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

  struct Stage {
    u32x4 w[U][2][P][NB];
    u32x4 x[U][2][NA][MT];
  };
  auto load = [&](Stage& s, int kit) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const size_t off = (size_t)(kit + (u * WAVES + wave) * 64 + j * 32) * 2;
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s.w[u][j][p][nb] = ld_stream(wrow[p][nb] + off);
#pragma unroll
        for (int q = 0; q < NA; ++q)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) s.x[u][j][q][mt] = ld16(arow[q][mt] + off);
      }
  };
  auto load_masked = [&](Stage& s, int kit) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int koff = kit + (u * WAVES + wave) * 64 + j * 32;
        const bool valid = koff + lg * 8 < kend;
        const size_t off = valid ? (size_t)koff * 2 : 0;
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const u32x4 v = ld_stream(wrow[p][nb] + off);
            s.w[u][j][p][nb] = valid ? v : u32x4{0, 0, 0, 0};
          }
#pragma unroll
        for (int q = 0; q < NA; ++q)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const u32x4 v = ld16(arow[q][mt] + off);
            s.x[u][j][q][mt] = valid ? v : u32x4{0, 0, 0, 0};
          }
      }
  };
  auto compute = [&](const Stage& s) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int q = 0; q < NA; ++q)
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                acc[p][nb][mt] = mfma16x16x32(s.x[u][j][q][mt], s.w[u][j][p][nb], acc[p][nb][mt]);
  };

  const int nfull = (kend - kbeg) / STEP;
  Stage s0, s1;
  int kit = kbeg;
  if (nfull > 0) {
    load(s0, kit);
    int i = 0;
    for (; i + 2 < nfull; i += 2) {
      load(s1, kit + STEP);
      __builtin_amdgcn_sched_barrier(0);
      compute(s0);
      __builtin_amdgcn_sched_barrier(0);
      load(s0, kit + 2 * STEP);
      __builtin_amdgcn_sched_barrier(0);
      compute(s1);
      __builtin_amdgcn_sched_barrier(0);
      kit += 2 * STEP;
    }
    if (i + 1 < nfull) {
      load(s1, kit + STEP);
      __builtin_amdgcn_sched_barrier(0);
      compute(s0);
      compute(s1);
      kit += 2 * STEP;
    } else {
      compute(s0);
      kit += STEP;
    }
  }
  if (kit < kend) {
    load_masked(s0, kit);
    compute(s0);
  }
  __shared__ __attribute__((aligned(16))) char red[lds_red_bytes<MT, NB, WAVES, GU>()];
  finish_workgroup<MT, NB, WAVES, GU>(a, acc, red);
}

// Sum the ksplit partials in slice order and apply the stage's epilogue.
template <bool GU>
__global__ __launch_bounds__(256) void skinny_finalize(const float* __restrict__ part,
                                                       int ksplit, int M, int N, void* out,
                                                       int ldo, int out_f32, int h_fmt) {
  // Four consecutive features per thread (N % 4 == 0): 16-byte partial loads, up to
  // sixteen slices in flight at a time, summed in slice order.  Down and projection outputs
  // have row stride ldo (a multiple of 4).  The partials (read once) are loaded and an fp32
  // output stored non-temporally, as the tiled kernel stores them.
  constexpr int P = GU ? 2 : 1;
  const int N4 = N >> 2;
  const size_t total = (size_t)M * N4;
  const size_t sstride = (size_t)M * P * N;  // floats per slice
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(e / N4), n = (int)(e % N4) * 4;
    const float* base = part + (size_t)m * P * N + n;
    f32x4 g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
    // SB slices per batch, all loads of a batch in flight together (the last batch
    // takes the remaining slices), summed in slice order.
    constexpr int SB = 16;
    for (int s = 0; s < ksplit; s += SB) {
      f32x4 a[SB], b[SB];
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        if (s + q < ksplit) {
          a[q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base + (size_t)(s + q) * sstride));
          if (GU) b[q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base + (size_t)(s + q) * sstride + N));
        }
      }
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        if (s + q < ksplit) {
          g += a[q];
          if (GU) u += b[q];
        }
      }
    }
    const size_t o = (size_t)m * (GU ? N : ldo) + n;
    if (GU) {
      // h as one bf16 plane (h_fmt 1), bf16 hi + lo planes (2) or one fp16 plane (3)
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float h = silu_mul(g[j], u[j]);
        if (h_fmt == 3) {
          hi[j] = f2h(h);
        } else {
          hi[j] = f2bf(h);
          lo[j] = f2bf(h - __uint_as_float(hi[j] << 16));
        }
      }
      uint16_t* hp = reinterpret_cast<uint16_t*>(out);
      *reinterpret_cast<u32x2*>(hp + o) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
      if (h_fmt == 2)
        *reinterpret_cast<u32x2*>(hp + (size_t)M * N + o) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
    } else if (out_f32) {
      __builtin_nontemporal_store(g, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + o));
    } else {
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + o) =
          u32x2{f2bf(g[0]) | (f2bf(g[1]) << 16), f2bf(g[2]) | (f2bf(g[3]) << 16)};
    }
  }
}

template <int MODE>
static int launch_stage(const SkinnyPlan& sp, const SkArgs& a, hipStream_t s) {
  constexpr bool GU = MODE == MODE_GATE_UP;
  const int tt = sp.ttiles > 1 ? sp.ttiles : 1;
  dim3 grid(sp.blocks / (sp.ksplit * tt), sp.ksplit, tt);
  dim3 block(sp.waves * 64);
#define SMLP_SK(KERNEL)                                                                  \
  if (sp.mt == MT_ && sp.nb == NB_ && sp.waves == W_ && sp.u == U_) {                    \
    hipLaunchKernelGGL((KERNEL<MT_, NB_, W_, U_, MODE>), grid, block, 0, s, a);          \
    return (int)hipGetLastError();                                                       \
  }
#define SMLP_SK_D(MT__, NB__, W__, U__) { constexpr int MT_ = MT__, NB_ = NB__, W_ = W__, U_ = U__; SMLP_SK(skinny_direct_kernel) }
#define SMLP_SK_S(MT__, NB__, W__, U__)                                                     \
  if (sp.mt == MT__ && sp.nb == NB__ && sp.waves == W__ && sp.u == U__) {                   \
    hipLaunchKernelGGL((skinny_stream_kernel<MT__, NB__, W__, U__, MODE>), grid, block, 0, s, a); \
    return (int)hipGetLastError();                                                          \
  }
  if constexpr (GU) {
    if (sp.kind == SKINNY_DIRECT16) { SMLP_SK_GU_DIRECT16(SMLP_SK_D) }
    if (sp.kind == SKINNY_STREAM16) { SMLP_SK_GU_STREAM16(SMLP_SK_S) }
  } else if constexpr (MODE == MODE_LINEAR) {
    if (sp.kind == SKINNY_STREAM16) { SMLP_SK_LIN_STREAM16(SMLP_SK_S) }
  } else {
    if (sp.kind == SKINNY_DIRECT16) { SMLP_SK_DN_DIRECT16(SMLP_SK_D) }
    if (sp.kind == SKINNY_STREAM16) { SMLP_SK_DN_STREAM16(SMLP_SK_S) }
  }
#undef SMLP_SK_S
#undef SMLP_SK_D
#undef SMLP_SK
  return (int)hipErrorInvalidConfiguration;
}

int launch_finalize(bool gu, const float* part, int ksplit, int M, int N, void* out, int ldo,
                    int out_f32, int h_fmt, hipStream_t s) {
  if (N % 4 != 0 || ldo % 4 != 0) return (int)hipErrorInvalidValue;
  const size_t total = (size_t)M * (N / 4);
  // Small outputs (a decode step's partials) take 64-thread workgroups so that every
  // compute unit pulls a share of the partials.
  const int threads = total >= (size_t)512 * 256 ? 256 : 64;
  size_t blocks = (total + threads - 1) / threads;
  if (blocks > (size_t)2048 * 256 / threads) blocks = (size_t)2048 * 256 / threads;
  if (gu)
    hipLaunchKernelGGL(skinny_finalize<true>, dim3((unsigned)blocks), dim3(threads), 0, s, part, ksplit, M,
                       N, out, ldo, out_f32, h_fmt);
  else
    hipLaunchKernelGGL(skinny_finalize<false>, dim3((unsigned)blocks), dim3(threads), 0, s, part, ksplit,
                       M, N, out, ldo, out_f32, h_fmt);
  return (int)hipGetLastError();
}

int launch_skinny_gate_up(const Plan& p, const void* x, const void* w_gate_up, void* ws,
                          hipStream_t s) {
  SkArgs a;
  a.a_hi = reinterpret_cast<const uint16_t*>(x);
  a.a_lo = nullptr;
  a.w = reinterpret_cast<const uint16_t*>(w_gate_up);
  a.M = (int)p.M;
  a.K = (int)p.H;
  a.N = (int)p.I;
  a.up_off = (int)p.up_off;
  a.kslice = p.gu.kslice;
  a.out = static_cast<char*>(ws) + p.h_offset;
  a.ldo = a.N;
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_offset);
  a.out_f32 = 0;
  a.h_planes = p.h_dtype == SMLP_BF16_HILO ? 2 : p.h_dtype == SMLP_FP16 ? 3 : 1;
  a.fpw = p.gu.fpw;
  a.w_rows = (int)(p.up_off + p.I);
  a.ldw = (int)p.H;
  a.red_cnt = nullptr;
  if (p.gu.ksplit > 1 && p.gu.kind == SKINNY_STREAM16 && p.gu.red_ok)
    a.red_cnt = reduce_counters(s, p.gu.blocks / (p.gu.ksplit * (p.gu.ttiles > 1 ? p.gu.ttiles : 1)));
  int rc = launch_stage<MODE_GATE_UP>(p.gu, a, s);
  if (rc || p.gu.ksplit == 1 || a.red_cnt) return rc;
  return launch_finalize(true, a.part, p.gu.ksplit, a.M, a.N, a.out, a.N, 0, a.h_planes, s);
}

// Per-column arrival counters of the in-launch K-split reduction: one block of
// kRedColumns counters (16 words apart) per stream slot, per device.
constexpr int kRedColumns = 256;
__device__ uint32_t g_red_cnt[kLayerSyncSlots * kRedColumns * 16];

uint32_t* reduce_counters(hipStream_t s, int columns) {
  if (columns > kRedColumns || !fusion_enabled()) return nullptr;
  const int slot = stream_slot(s);
  if (slot < 0) return nullptr;
  static std::mutex mu;
  static uint32_t* base[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev] && hipGetSymbolAddress((void**)&base[dev], HIP_SYMBOL(g_red_cnt)) != hipSuccess) {
    base[dev] = nullptr;
    return nullptr;
  }
  return base[dev] + (size_t)slot * kRedColumns * 16;
}

// Device address of this device's counter slots, looked up once per device.
static int layer_sync_base(uint32_t** out) {
  static std::mutex mu;
  static uint32_t* base[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev]) {
    e = hipGetSymbolAddress((void**)&base[dev], HIP_SYMBOL(g_layer_sync));
    if (e != hipSuccess) {
      base[dev] = nullptr;
      return (int)e;
    }
  }
  *out = base[dev];
  return (int)hipSuccess;
}

// The stage configurations the one-launch layer is built for: one token tile (gate_up
// 3 tiles x 4 waves x 3 stages, down 2 tiles x 8 waves x 3 stages) and two token tiles
// (gate_up 3 x 4 x 3, down 2 x 4 x 4).
bool decode_layer_eligible(const Plan& p) {
  const SkinnyPlan& g = p.gu;
  const SkinnyPlan& d = p.dn;
  if (p.path != SMLP_PATH_SMALL_M || p.h_dtype != SMLP_BF16 || g.kind != SKINNY_STREAM16 ||
      d.kind != SKINNY_STREAM16 || g.ksplit != 1 || d.ksplit != 1 || g.ttiles > 1 || g.mt != d.mt ||
      g.nb != 3 || g.waves != 4 || g.u != 3 || d.nb != 2 || g.blocks + d.blocks > 65535)
    return false;
  return (g.mt == 1 && d.waves == 8 && d.u == 3) || (g.mt == 2 && d.waves == 4 && d.u == 4);
}

int launch_decode_layer(const Plan& p, const void* x, const void* w_gate_up, const void* w_down, void* out,
                        void* ws, int slot, int limit, hipStream_t s) {
  if (!decode_layer_eligible(p) || slot < 0 || slot >= kLayerSyncSlots) return (int)hipErrorInvalidConfiguration;
  SkArgs g;
  g.a_hi = reinterpret_cast<const uint16_t*>(x);
  g.a_lo = nullptr;
  g.w = reinterpret_cast<const uint16_t*>(w_gate_up);
  g.M = (int)p.M;
  g.K = (int)p.H;
  g.N = (int)p.I;
  g.up_off = (int)p.up_off;
  g.kslice = p.gu.kslice;
  g.out = static_cast<char*>(ws) + p.h_offset;
  g.ldo = g.N;
  g.part = nullptr;
  g.out_f32 = 0;
  g.h_planes = 1;
  g.fpw = p.gu.fpw;
  g.w_rows = (int)(p.up_off + p.I);
  g.ldw = (int)p.H;
  g.red_cnt = nullptr;
  SkArgs d;
  d.a_hi = reinterpret_cast<const uint16_t*>(static_cast<const char*>(ws) + p.h_offset);
  d.a_lo = nullptr;
  d.w = reinterpret_cast<const uint16_t*>(w_down);
  d.M = (int)p.M;
  d.K = (int)p.I;
  d.N = (int)p.H;
  d.up_off = 0;
  d.kslice = p.dn.kslice;
  d.out = out;
  d.ldo = (int)p.H;
  d.part = nullptr;
  d.out_f32 = p.partial_fp32 ? 1 : 0;
  d.h_planes = 1;
  d.fpw = p.dn.fpw;
  d.w_rows = (int)p.H;
  d.ldw = (int)p.ldwd;
  d.red_cnt = nullptr;
  uint32_t* sync = nullptr;
  const int rc = layer_sync_base(&sync);
  if (rc != (int)hipSuccess) return rc;
  if (p.gu.mt == 1)
    hipLaunchKernelGGL((decode_layer_kernel<1, 3, 3, 2, 3, 8>), dim3(p.gu.blocks + p.dn.blocks), dim3(512), 0, s,
                       g, d, sync + (size_t)slot * kSyncWords, p.gu.blocks, limit);
  else
    hipLaunchKernelGGL((decode_layer_kernel<2, 3, 3, 2, 4, 4>), dim3(p.gu.blocks + p.dn.blocks), dim3(256), 0, s,
                       g, d, sync + (size_t)slot * kSyncWords, p.gu.blocks, limit);
  return (int)hipGetLastError();
}

int launch_skinny_down(const Plan& p, const void* w_down, void* out, void* ws, hipStream_t s) {
  if (p.h_dtype == SMLP_BF16)  // one plane of h: the plain projection out = h . Wd^T
    return launch_skinny_linear(p.dn, static_cast<const char*>(ws) + p.h_offset, w_down, out, (int)p.M,
                                (int)p.I, (int)p.H, (int)p.H, p.partial_fp32 ? 1 : 0,
                                reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_offset), s,
                                (int)p.ldwd);
  SkArgs a;
  const uint16_t* h = reinterpret_cast<const uint16_t*>(static_cast<const char*>(ws) + p.h_offset);
  a.a_hi = h;
  a.a_lo = p.h_dtype == SMLP_BF16_HILO ? h + (size_t)p.M * p.I : nullptr;
  a.w = reinterpret_cast<const uint16_t*>(w_down);
  a.M = (int)p.M;
  a.K = (int)p.I;
  a.N = (int)p.H;
  a.up_off = 0;
  a.kslice = p.dn.kslice;
  a.out = out;
  a.ldo = a.N;
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_offset);
  a.out_f32 = p.partial_fp32 ? 1 : 0;
  a.h_planes = p.h_dtype == SMLP_BF16_HILO ? 2 : 1;
  a.fpw = p.dn.fpw;
  a.w_rows = (int)p.H;
  a.ldw = (int)p.ldwd;
  a.red_cnt = nullptr;
  if (p.dn.ksplit > 1 && p.dn.kind == SKINNY_STREAM16 && p.dn.red_ok)
    a.red_cnt = reduce_counters(s, p.dn.blocks / p.dn.ksplit);
  int rc = launch_stage<MODE_DOWN_HILO>(p.dn, a, s);
  if (rc || p.dn.ksplit == 1 || a.red_cnt) return rc;
  return launch_finalize(false, a.part, p.dn.ksplit, a.M, a.N, out, a.N, a.out_f32, 1, s);
}

int launch_skinny_linear(const SkinnyPlan& sp, const void* x, const void* w, void* y, int M, int K,
                         int N, int ldy, int out_f32, float* part, hipStream_t s, int ldw) {
  SkArgs a;
  a.a_hi = reinterpret_cast<const uint16_t*>(x);
  a.a_lo = nullptr;
  a.w = reinterpret_cast<const uint16_t*>(w);
  a.M = M;
  a.K = K;
  a.N = N;
  a.up_off = 0;
  a.kslice = sp.kslice;
  a.out = y;
  a.ldo = ldy;
  a.part = part;
  a.out_f32 = out_f32;
  a.h_planes = 1;
  a.fpw = sp.fpw;
  a.w_rows = N;
  a.ldw = ldw > 0 ? ldw : K;
  a.red_cnt = nullptr;
  if (sp.ksplit > 1 && sp.kind == SKINNY_STREAM16 && sp.red_ok) a.red_cnt = reduce_counters(s, sp.blocks / sp.ksplit);
  int rc = launch_stage<MODE_LINEAR>(sp, a, s);
  if (rc || sp.ksplit == 1 || a.red_cnt) return rc;
  return launch_finalize(false, part, sp.ksplit, M, N, y, ldy, out_f32, 1, s);
}

}  // namespace smlp
