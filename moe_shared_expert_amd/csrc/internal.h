// Host-side interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace smlp {

// One weight-streaming (small-M) stage: out-features in blocks of 16, K split into
// `ksplit` slices over workgroups and into `waves` slices inside a workgroup.
struct SkinnyPlan {
  int kind;      // SKINNY_STREAM16 or SKINNY_DIRECT16
  int mt;        // 16-token tiles (M <= 16 * mt)
  int nb;        // output tiles per workgroup (SKINNY_STREAM16: 16-row MFMA tiles holding
                 // 8 gate_up features or 16 down rows; SKINNY_DIRECT16: 16-feature blocks)
  int waves;     // waves per workgroup (they split K)
  int u;         // SKINNY_STREAM16: LDS ring stages; SKINNY_DIRECT16: 64-element K steps
                 // per wave per pipeline stage
  int ksplit;    // workgroups along K (1 = no cross-workgroup reduction)
  int kslice;    // K elements per workgroup slice (multiple of 64)
  int blocks;    // total workgroups
  int fpw;       // SKINNY_STREAM16: features (gate_up) or rows (down) per workgroup
  int ttiles;    // SKINNY_STREAM16 token split: workgroups along M, 16 * mt tokens each
                 // (0 or 1 = none; blocks counts every workgroup)
  int red_ok;    // a K split may be reduced in the same launch (off for a pinned shape)
};

enum { SKINNY_DIRECT16 = 2, SKINNY_STREAM16 = 3 };

// One stage of the LDS-tiled GEMM path (gemm.hip).
struct GemmPlan {
  int bm, bn;    // tile: tokens x weight rows (gate_up: bn/2 features)
  int wm, wn;    // wave grid
  int ns;        // LDS stages
  int tiles_m;   // tiles along M (tiles = tiles_m * tiles along N)
  int tiles;
  int ksplit;    // workgroups along K
  int kslice;    // K elements per slice (multiple of 64)
  int ntb;       // weight loads non-temporal (a tile of SMLP_GEMM_NT_CONFIGS)
};

struct Plan {
  int path;                 // SMLP_PATH_*
  int64_t M, H, I;
  int dtype;
  int partial_fp32;
  int h_dtype;              // SMLP_FP32, SMLP_BF16, SMLP_BF16_HILO or SMLP_FP16
  size_t h_offset, h_bytes;
  size_t part_offset, part_bytes;   // split-K partial sums
  size_t wd16_offset, wd16_bytes;   // fp16 copy of w_down [H, I] (dense) when the down stage
                                    // multiplies fp16 h by pre-converted weights
  size_t workspace_bytes;
  SkinnyPlan gu, dn;
  GemmPlan ggu, gdn;
  // Large-M stages split by output columns: ggu / gdn cover features / rows [0, split)
  // in whole rounds of workgroups and the tail plan the rest (split = 0: no split).
  GemmPlan ggu_tail, gdn_tail;
  int64_t gu_split, dn_split;
  // Large-M path with the gate_up stage run by the weight-streaming kernel split over
  // tokens (plan gu) instead of the tiled GEMM (ggu).
  int gu_tsplit;
  int kernels;
  // Weight views (a rank's slice read in place from full weights): rows between a gate
  // row and its up row in w_gate_up (I for whole weights), and the row stride of w_down
  // in elements (I for whole weights).
  int64_t up_off, ldwd;
};

// Weight-streaming stages (skinny.hip).  Return a hipError_t.
int launch_skinny_gate_up(const Plan& p, const void* x, const void* w_gate_up, void* ws,
                          hipStream_t s);
int launch_skinny_down(const Plan& p, const void* w_down, void* out, void* ws, hipStream_t s);
// One-launch decode layer (both stages in one grid; skinny.hip): whether plan p has the
// stage configurations it is built for, and the launch with counter slot `slot` and a
// consumer wait of at most `limit` polls.  Returns a hipError_t.
constexpr int kLayerSyncSlots = 16;
// Counter slot of `stream` on the current device (api.cpp; -1 when all are taken), and
// whether one-launch forms and in-launch reductions are enabled (shared_mlp_tune_layer_fusion).
int stream_slot(hipStream_t stream);
bool fusion_enabled();
// Per-column counters for an in-launch K-split reduction over `columns` columns on
// `stream`, or null (then a finalize launch reduces) (skinny.hip).
uint32_t* reduce_counters(hipStream_t stream, int columns);
bool decode_layer_eligible(const Plan& p);
int launch_decode_layer(const Plan& p, const void* x, const void* w_gate_up, const void* w_down, void* out,
                        void* ws, int slot, int limit, hipStream_t s);

// Sum K-split partials [ksplit][M][P*N] in slice order and apply the stage epilogue
// (gate_up: SiLU-and-mul into h, h_fmt 1 = one bf16 plane, 2 = bf16 hi + lo, 3 = fp16;
// down: bf16 or fp32 out).
int launch_finalize(bool gate_up, const float* part, int ksplit, int M, int N, void* out,
                    int ldo, int out_f32, int h_fmt, hipStream_t s);

// Plain projection y = x . w^T (bf16 operands; y bf16 or fp32 with row stride ldy):
// the streaming kernel (plan kind SKINNY_STREAM16, M <= 32) or the LDS-tiled kernel,
// with `part` holding ksplit x M x N fp32 partials when the plan splits K.
int launch_skinny_linear(const SkinnyPlan& sp, const void* x, const void* w, void* y, int M, int K,
                         int N, int ldy, int out_f32, float* part, hipStream_t s, int ldw = 0);
int launch_gemm_linear(const GemmPlan& gp, const void* x, const void* w, void* y, int M, int K,
                       int N, int ldy, int out_f32, float* part, hipStream_t s);
// Rank-major -> logical column order of a gathered merged-column output (latent.hip);
// arguments validated by the caller.
int launch_restore_logical(const void* src, void* dst, int64_t M, int64_t N, const int64_t* sizes,
                           int nr, int tp, int elem_bytes, hipStream_t s);

// LDS-tiled GEMM stages (gemm.hip).
int launch_gemm_gate_up(const Plan& p, const void* x, const void* w_gate_up, void* ws, hipStream_t s);
int launch_gemm_down(const Plan& p, const void* w_down, void* out, void* ws, hipStream_t s);

// Device address of this device's static scratch array (noalloc.hip), looked up with
// hipGetSymbolAddress on the first call per device and cached.  Returns a hipError_t.
int noalloc_scratch(void** ptr);

// fp32 stages and helpers (aux.hip).
int launch_fp32_gate_up(const Plan& p, const float* x, const float* w_gate_up, void* ws,
                        hipStream_t s);
int launch_fp32_down(const Plan& p, const float* w_down, float* out, void* ws, hipStream_t s);
// Both fp32 stages in one single-workgroup launch, h in LDS, where M * I <= kFp32SmallH and
// M * H * I <= 2^20 (fp32_small_layer); the same bits as the two launches above.
constexpr int kFp32SmallH = 4096;
inline bool fp32_small_layer(int64_t M, int64_t H, int64_t I) {
  return M * I <= kFp32SmallH && M * H * I <= ((int64_t)1 << 20);
}
int launch_fp32_layer(const Plan& p, const float* x, const float* w_gate_up, const float* w_down, float* out,
                      hipStream_t s);
int launch_slice_rank(const void* wgu, const void* wd, void* wgu_r, void* wd_r, int64_t H,
                      int64_t I, int tp, int rank, int elem_bytes, hipStream_t s);
int launch_rms_rescale(const float* in, uint16_t* out, int64_t M, int64_t H, hipStream_t s);
// bf16 -> fp16 copy of a rows x cols weight matrix (source row stride ld_src) into a dense
// destination (aux.hip).
int launch_bf16_to_f16(const void* src, int64_t ld_src, int64_t rows, int64_t cols, void* dst, hipStream_t s);

}  // namespace smlp
