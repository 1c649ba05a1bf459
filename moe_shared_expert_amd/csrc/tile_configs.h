// Compiled kernel configurations of the weight-streaming (skinny.hip) and LDS-tiled
// (gemm.hip) stages, as X-macro lists, and the host-side queries of those lists that the
// planner (api.cpp) uses.  Host-visible only: no device code.
#pragma once

#include "internal.h"

namespace smlp {

// Instantiated configurations (MT, NB, WAVES, U) per kernel kind (MT = 16-token
// tiles; none spills registers).  Streaming kind: NB = 16-row MFMA tiles, U = ring
// stages, LDS = WAVES x STAGES x (NB + activation tiles) x 2 KB <= 160 KB with
// activation tiles = MT (gate_up) or 2 MT (down).  Direct kind: NB = 16-feature
// blocks, U = 64-element K steps per wave per pipeline stage.
#define SMLP_SK_GU_STREAM16(X)                                                                 \
  X(1, 1, 4, 4) X(1, 1, 8, 4) X(1, 2, 4, 4) X(1, 2, 8, 3) X(1, 3, 4, 3) X(1, 3, 4, 4)          \
  X(1, 3, 4, 5) X(1, 3, 8, 2) X(1, 4, 4, 4) X(2, 1, 4, 4) X(2, 2, 4, 4) X(2, 3, 4, 3)          \
  X(2, 3, 4, 4) X(2, 4, 4, 3)
#define SMLP_SK_DN_STREAM16(X)                                                                 \
  X(1, 1, 4, 4) X(1, 1, 8, 3) X(1, 2, 4, 3) X(1, 2, 4, 4) X(1, 2, 4, 5) X(1, 2, 8, 2)          \
  X(1, 3, 4, 4) X(1, 4, 4, 3) X(2, 1, 4, 4) X(2, 2, 4, 3) X(2, 3, 4, 2) X(2, 4, 4, 2)
// Projection (one activation plane): deeper rings, so that a wave keeps more weight
// bytes in flight when a workgroup holds only one or two 16-row tiles.
#define SMLP_SK_LIN_STREAM16(X)                                                                \
  X(1, 1, 4, 4) X(1, 1, 4, 6) X(1, 1, 4, 8) X(1, 1, 8, 3) X(1, 1, 8, 4) X(1, 1, 8, 5)          \
  X(1, 2, 4, 4) X(1, 2, 4, 6) X(1, 2, 8, 3) X(1, 3, 4, 4) X(1, 4, 4, 4) X(2, 1, 4, 4)          \
  X(2, 1, 4, 6) X(2, 1, 8, 3) X(2, 2, 4, 4) X(2, 2, 8, 2)
#define SMLP_SK_GU_DIRECT16(X) X(4, 1, 4, 1) X(4, 1, 8, 1) X(8, 1, 4, 1) X(8, 1, 8, 1)
#define SMLP_SK_DN_DIRECT16(X) X(4, 1, 4, 1) X(4, 1, 8, 1) X(8, 1, 4, 1)
inline bool skinny_instantiated(int stage, int kind, int mt, int nb, int waves, int u) {
#define SMLP_MATCH(MT_, NB_, W_, U_) \
  if (mt == MT_ && nb == NB_ && waves == W_ && u == U_) return true;
  if (stage == 2) {
    if (kind == SKINNY_STREAM16) { SMLP_SK_LIN_STREAM16(SMLP_MATCH) }
  } else if (stage == 0) {
    if (kind == SKINNY_DIRECT16) { SMLP_SK_GU_DIRECT16(SMLP_MATCH) }
    if (kind == SKINNY_STREAM16) { SMLP_SK_GU_STREAM16(SMLP_MATCH) }
  } else {
    if (kind == SKINNY_DIRECT16) { SMLP_SK_DN_DIRECT16(SMLP_MATCH) }
    if (kind == SKINNY_STREAM16) { SMLP_SK_DN_STREAM16(SMLP_MATCH) }
  }
#undef SMLP_MATCH
  return false;
}


// Tile configurations (BM, BN, WM, WN, stages).  LDS holds stages x (BM + BN) x 128
// bytes (the two-plane down mode: stages x (2 BM + BN) x 128) of the 160 KB per
// workgroup.
#define SMLP_GEMM_CONFIGS(X)                                                                    \
  X(256, 256, 2, 4, 2) X(128, 256, 2, 4, 3) X(128, 256, 2, 2, 3) X(128, 128, 2, 2, 2)           \
  X(128, 128, 2, 2, 4) X(128, 128, 4, 2, 4) X(128, 64, 4, 1, 2) X(128, 64, 4, 1, 4) X(128, 64, 4, 1, 6) \
  X(128, 128, 4, 2, 2) X(128, 128, 4, 2, 3) X(128, 256, 2, 4, 2) X(256, 128, 4, 2, 2) X(256, 128, 4, 2, 3) \
  X(128, 64, 4, 2, 3) X(128, 64, 4, 2, 4) X(64, 64, 2, 2, 4)
// Down only (one MFMA tile column per wave cannot pair gate and up rows).
#define SMLP_GEMM_DN_CONFIGS(X) X(128, 32, 4, 1, 2) X(128, 32, 4, 1, 4)
#define SMLP_GEMM_HILO_CONFIGS(X) X(128, 128, 2, 2, 3) X(128, 64, 4, 1, 2) X(128, 64, 4, 1, 4)
// Tiles also built with non-temporal weight loads (one bf16 plane or fp16 h only), for
// plans whose weights every workgroup streams exactly once: one token tile, long K, wide
// weights (the replicated layer at M <= 128).
#define SMLP_GEMM_NT_CONFIGS(X) X(128, 256, 2, 4, 3) X(128, 128, 4, 2, 2)


inline bool gemm_nt_instantiated(bool hilo, int bm, int bn, int wm, int wn, int ns) {
#define SMLP_GM(BM_, BN_, WM_, WN_, NS_) \
  if (bm == BM_ && bn == BN_ && wm == WM_ && wn == WN_ && ns == NS_) return true;
  if (!hilo) {
    SMLP_GEMM_NT_CONFIGS(SMLP_GM)
  }
#undef SMLP_GM
  return false;
}

inline bool gemm_instantiated(int stage, bool hilo, int bm, int bn, int wm, int wn, int ns) {
#define SMLP_GM(BM_, BN_, WM_, WN_, NS_) \
  if (bm == BM_ && bn == BN_ && wm == WM_ && wn == WN_ && ns == NS_) return true;
  if (stage == 1 && hilo) {
    SMLP_GEMM_HILO_CONFIGS(SMLP_GM)
  } else {
    SMLP_GEMM_CONFIGS(SMLP_GM)
    if (stage == 1) {
      SMLP_GEMM_DN_CONFIGS(SMLP_GM)
    }
  }
#undef SMLP_GM
  return false;
}


}  // namespace smlp
