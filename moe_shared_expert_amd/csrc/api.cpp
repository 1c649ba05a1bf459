// C ABI of libsmlp: host-side validation, M-dispatch planning and kernel dispatch.
// Every check runs on the host before the first HIP call of an entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "internal.h"
#include "tile_configs.h"
#include "smlp.h"
#include "smlp_latent.h"
#include "smlp_tuning.h"

namespace {

thread_local std::string g_last_error;

// Number of compute units the planner sizes grids for (MI355X).
constexpr int kCUs = 256;
// The weight-streaming kernels handle up to 128 tokens per call.
constexpr int64_t kSmallMaxM = 128;
// Default M-dispatch threshold: on MI355X the weight-streaming kernel is fastest up
// to 32 tokens and the LDS-tiled path from 33 on.
constexpr int64_t kDefaultLargeMMin = 33;
constexpr int64_t kLimit = (int64_t)1 << 31;

int64_t initial_threshold() {
  const char* e = std::getenv("SMLP_LARGE_M_MIN");
  if (e && *e) {
    char* end = nullptr;
    long long v = std::strtoll(e, &end, 10);
    if (end && *end == '\0' && v >= 1 && v <= kSmallMaxM + 1) return (int64_t)v;
  }
  return kDefaultLargeMMin;
}
std::atomic<int64_t> g_threshold{initial_threshold()};

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SMLP_OK;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Tuning overrides of the small-M planner (0 = automatic), per stage (0 gate_up, 1 down,
// 2 the plain projection).
struct SkinnyOverride {
  std::atomic<int> kind{0}, nb{0}, waves{0}, u{0}, ksplit{0};
};
SkinnyOverride g_tune[3];

struct GemmOverride {
  std::atomic<int> bm{0}, bn{0}, wm{0}, wn{0}, ns{0}, ksplit{0};
};
GemmOverride g_gtune[3];

// Planes of h on the small-M path (0 = automatic: one for M <= 32 and I >= 256, else
// two), see shared_mlp_tune_h_planes.
std::atomic<int> g_h_planes{0};
// Format of h on the large-M path (0 = automatic), see shared_mlp_tune_h_format.
std::atomic<int> g_h_format{0};
// Token-split gate_up on the tiled path (0 = automatic, 1 = always where it applies,
// 2 = never), see shared_mlp_tune_token_split.
std::atomic<int> g_tsplit{0};

// One-launch decode layer (0 = automatic, 1 = wherever it applies, 2 = never) and the
// consumer's poll limit, see shared_mlp_tune_layer_fusion.
std::atomic<int> g_fuse{0};
std::atomic<int> g_fuse_limit{1 << 18};

int layer_sync_slot(hipStream_t stream) { return smlp::stream_slot(stream); }

// Token count from which a large-M down stage with fp16 h converts w_down to fp16 once
// (into the workspace) instead of converting its weight fragments in registers, see
// shared_mlp_tune_weight_convert.
std::atomic<int64_t> g_wd16_min_m{1024};

// Small-M stage plan.  M <= 32: the streaming kernel, one workgroup per compute unit
// over an equal contiguous share of the features (gate_up) or rows (down), the whole K
// range, waves interleaved over K (short TP shards: whole tiles and a K split, below).
// M > 32: the direct-load kernel over 16-feature
// blocks, with a K split over workgroups when the blocks alone cannot keep about
// three waves per compute unit streaming.  Returns false if a pinned (tuned)
// configuration is not one of the compiled kernels.
// `inst` names the compiled config list the plan must come from (default: the stage's
// own; the down stage with one plane of h runs the projection kernel, list 2).
bool plan_skinny(int stage, int64_t M, int64_t N, int64_t K, smlp::SkinnyPlan* out, int inst = -1) {
  using namespace smlp;
  if (inst < 0) inst = stage;
  const SkinnyOverride& o = g_tune[stage];
  smlp::SkinnyPlan sp{};
  sp.kind = o.kind.load() ? o.kind.load() : (M <= 32 ? SKINNY_STREAM16 : SKINNY_DIRECT16);
  sp.waves = 0;
  if (sp.kind == SKINNY_STREAM16 && M > 32) return false;
  sp.mt = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
  // u: LDS ring stages of the streaming kind, the unroll of the direct kind.
  sp.u = o.u.load() ? o.u.load() : 1;
  const int64_t ksteps = (K + 63) / 64;
  if (sp.kind == SKINNY_STREAM16) {
    const int64_t tile = stage == 0 ? 8 : 16;  // features per 16-row tile
    // Short TP shards (measured on MI355X, H = 7168): gate_up with few features (I_r <= 512,
    // or I_r < 2048 at 17-32 tokens) fills whole tiles, ~48 workgroup columns, and splits
    // K four ways (I_r = 384, M = 16: 8.6 -> 7.7 us; I_r = 768, M = 32: 13.4 -> 11.7 us)
    // instead of spreading a few features over every compute unit; the one-plane down
    // stage with a short K (<= 1024) takes two whole tiles per workgroup with 4 waves and
    // 4 stages (I_r = 768: 6.0 -> 5.5 us; I_r = 384: 4.9 -> 4.5 us).
    const bool auto_shape = !o.nb.load() && !o.ksplit.load() && !o.waves.load() && !o.u.load();
    const bool gu_split = auto_shape && stage == 0 && N < tile * kCUs && (sp.mt == 2 || N <= 512);
    const bool dn_short = auto_shape && stage == 1 && inst == 2 && K <= 1024 && N >= 2048;
    int64_t groups = o.nb.load() ? (N + tile * o.nb.load() - 1) / (tile * o.nb.load()) : kCUs;
    if (groups > N) groups = N;
    int64_t fpw = (N + groups - 1) / groups;
    int64_t nt = (fpw + tile - 1) / tile;
    if (gu_split) {
      nt = (N + 24 * tile) / (48 * tile);  // round(N / (48 * tile)): about 48 columns
      nt = nt < 1 ? 1 : nt > 4 ? 4 : nt;
      fpw = nt * tile;
    } else if (dn_short) {
      nt = 2;
      fpw = 2 * tile;
    }
    if (nt > 4) {
      nt = 4;
      fpw = 4 * tile;
    }
    // Without a pinned tile count, narrow the workgroups (more of them) until some
    // compiled (waves, stages) pair serves the tile count: not every (tokens, tiles)
    // combination is instantiated (two token tiles take at most 2 tiles per workgroup in
    // the projection kernel, for one).
    if (!o.nb.load()) {
      auto served = [&](int64_t t) {
        for (int w : {4, 8})
          for (int st = 2; st <= 8; ++st)
            if (smlp::skinny_instantiated(inst, sp.kind, sp.mt, (int)t, o.waves.load() ? o.waves.load() : w,
                                          o.u.load() ? o.u.load() : st))
              return true;
        return false;
      };
      while (nt > 1 && !served(nt)) {
        --nt;
        fpw = nt * tile;
      }
    }
    groups = (N + fpw - 1) / fpw;
    sp.nb = (int)nt;
    sp.fpw = (int)fpw;
    // Measured on MI355X: gate_up is fastest with 4 waves and a 3-stage ring, down
    // with 8 waves and 2 stages (two planes of h) or 3 stages (one plane); otherwise
    // the first compiled (waves, stages) pair in this order.
    static const int kPrefGU[][2] = {{4, 3}, {4, 4}, {4, 2}, {8, 2}};
    static const int kPrefDN[][2] = {{8, 2}, {8, 3}, {4, 4}, {4, 3}, {4, 2}};
    static const int kPrefDN1[][2] = {{8, 3}, {4, 4}, {8, 2}, {4, 6}};
    const int (*pref)[2] = stage == 0 ? kPrefGU : inst == 2 ? kPrefDN1 : kPrefDN;
    const int npref = stage == 0 ? 4 : inst == 2 ? 4 : 5;
    if ((gu_split || dn_short) && smlp::skinny_instantiated(inst, sp.kind, sp.mt, (int)nt, 4, 4)) {
      sp.waves = 4;
      sp.u = 4;
    } else if (!o.waves.load() || !o.u.load()) {
      for (int c = 0; c < npref; ++c) {
        const int w = o.waves.load() ? o.waves.load() : pref[c][0];
        const int st = o.u.load() ? o.u.load() : pref[c][1];
        if (smlp::skinny_instantiated(inst, sp.kind, sp.mt, (int)nt, w, st)) {
          sp.waves = w;
          sp.u = st;
          break;
        }
      }
    }
    if (!sp.waves && !(o.waves.load() && o.u.load())) {
      // none of the measured preferences is compiled for this tile count: take any pair
      for (int w : {4, 8})
        for (int st = 2; st <= 8 && !sp.waves; ++st)
          if (smlp::skinny_instantiated(inst, sp.kind, sp.mt, (int)nt, o.waves.load() ? o.waves.load() : w,
                                        o.u.load() ? o.u.load() : st)) {
            sp.waves = o.waves.load() ? o.waves.load() : w;
            sp.u = o.u.load() ? o.u.load() : st;
          }
    }
    if (o.waves.load()) sp.waves = o.waves.load();
    if (o.u.load()) sp.u = o.u.load();
    int64_t ks = o.ksplit.load() ? o.ksplit.load() : gu_split ? 4 : 1;
    if (ks > ksteps) ks = ksteps;
    const int64_t kslice = ((K + ks - 1) / ks + 63) / 64 * 64;
    ks = (K + kslice - 1) / kslice;
    sp.ksplit = (int)ks;
    sp.kslice = (int)kslice;
    sp.blocks = (int)(groups * ks);
  } else {
    sp.nb = o.nb.load() ? o.nb.load() : 1;
    sp.waves = o.waves.load() ? o.waves.load() : (sp.mt == 8 ? 4 : 8);
    const int64_t groups = (N + 16 * sp.nb - 1) / (16 * sp.nb);
    const int64_t target_waves = (int64_t)kCUs * 3;
    int64_t ks = o.ksplit.load();
    if (!ks) {
      ks = (target_waves + groups * sp.waves - 1) / (groups * sp.waves);
      const int64_t max_ks = ksteps / (2 * (int64_t)sp.waves * sp.u);  // >= two K steps per wave
      if (ks > max_ks) ks = max_ks;
      if (ks < 1) ks = 1;
    }
    if (ks > ksteps) ks = ksteps;
    const int64_t kslice = ((K + ks - 1) / ks + 63) / 64 * 64;
    ks = (K + kslice - 1) / kslice;
    sp.ksplit = (int)ks;
    sp.kslice = (int)kslice;
    sp.blocks = (int)(groups * ks);
    sp.fpw = 0;
  }
  if (!smlp::skinny_instantiated(inst, sp.kind, sp.mt, sp.nb, sp.waves, sp.u)) return false;
  // The in-launch K-split reduction is used with the planner's own shapes only (a pinned
  // K split alone keeps it); a pinned tile count, wave count or ring depth takes the
  // finalize launch.  A sweep of pinned streaming shapes with K splits (8 waves, 1-4
  // tiles, 3-4 stages) ended in a GPU memory fault whose cause was not found.
  sp.red_ok = !o.nb.load() && !o.waves.load() && !o.u.load();
  *out = sp;
  return true;
}

// Default choice of the token-split gate_up (measured on MI355X, H = 7168): off until
// measured.
bool token_split_default(int64_t M, int64_t N) {
  (void)M;
  (void)N;
  return false;
}

// Token-split gate_up for the tiled path: the weight-streaming kernel over tiles of 16 * mt
// tokens (ttiles workgroups along M) and nt 16-row tiles of 8 features each (along I),
// the full K range per workgroup, so the gate and up sums of a feature never leave
// registers and SiLU-and-mul is the kernel's epilogue (no K-split partials, no finalize
// launch).  The workgroups of one feature range share its weights through their XCD's L2.
// Sized to about one workgroup per compute unit; applies while every workgroup holds at
// most 4 tiles (N up to ~1024 features at M = 128).  Returns false when it does not apply.
bool plan_token_split(int64_t M, int64_t N, int64_t K, smlp::SkinnyPlan* out) {
  using namespace smlp;
  const SkinnyOverride& o = g_tune[0];
  SkinnyPlan sp{};
  sp.kind = SKINNY_STREAM16;
  sp.mt = M > 128 ? 2 : 1;
  const int64_t tok = 16 * sp.mt;
  const int64_t tt = (M + tok - 1) / tok;
  int64_t groups = (kCUs + tt / 2) / tt;
  if (groups < 1) groups = 1;
  int64_t fpw = (N + groups - 1) / groups;
  fpw = (fpw + 7) / 8 * 8;
  int64_t nt = o.nb.load() ? o.nb.load() : fpw / 8;
  if (nt < 1 || nt > 4) return false;
  fpw = 8 * nt;
  groups = (N + fpw - 1) / fpw;
  // measured preferences for the (waves, stages) of the ring, else any compiled pair
  static const int kPref[][2] = {{4, 4}, {4, 3}, {8, 2}, {8, 3}, {8, 4}, {4, 5}};
  sp.nb = (int)nt;
  sp.waves = o.waves.load();
  sp.u = o.u.load();
  for (const auto& c : kPref) {
    const int w = sp.waves ? sp.waves : c[0], st = sp.u ? sp.u : c[1];
    if (skinny_instantiated(0, sp.kind, sp.mt, sp.nb, w, st)) {
      sp.waves = w;
      sp.u = st;
      break;
    }
  }
  if (!sp.waves || !sp.u || !skinny_instantiated(0, sp.kind, sp.mt, sp.nb, sp.waves, sp.u)) return false;
  sp.fpw = (int)fpw;
  sp.ksplit = 1;
  sp.kslice = (int)((K + 63) / 64 * 64);
  sp.ttiles = (int)tt;
  sp.blocks = (int)(groups * tt);
  *out = sp;
  return true;
}

// LDS-tiled GEMM stage plan (measured on MI355X over M = 64 .. 8192, I = 384, 768 and
// 6144).  M > 256: 256 x 256 tiles (8 waves, 128 x 64 per wave) when they fill the chip
// at least twice over and K is long; otherwise 128 x 128 tiles (8 waves) when they fill
// the chip (gate_up) or fill it twice (down), or for a long-K down from half a tile per
// compute unit; down with a short K and few tiles: 128 x 32 tiles without a K split;
// else 128 x 64 tiles with a K split.  Two LDS stages, so that two workgroups share a
// compute unit, and a K split over workgroups when the tiles alone leave compute units
// idle.  M <= 256: the weight-streaming rules below.  N counts gate_up features (two
// weight rows each) or down rows.  Returns false if a pinned tile is not compiled.
// `ov` replaces the stage's tuning overrides (the plain projection plans as down).
bool plan_gemm(int stage, int64_t M, int64_t N, int64_t K, bool hilo, smlp::GemmPlan* out,
               const GemmOverride* ov = nullptr) {
  smlp::GemmPlan gp{};
  const GemmOverride& o = ov ? *ov : g_gtune[stage];
  const int64_t fpr = stage == 0 ? 2 : 1;  // weight rows per output feature
  auto tiles_for = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N * fpr + bn - 1) / bn); };
  // Up to two token tiles (M <= 256) the stage is bound by streaming the weights: one
  // workgroup per compute unit with a deep LDS ring, about 224 workgroups.  gate_up takes
  // 128 x 256 tiles (8 waves, 3 stages) when they reach 160 workgroups with K slices of
  // at least 12 K steps, else the widest of 128 x 128 (8 waves, 4 stages) and 128 x 64
  // (4 waves, 4 stages) that does; down the same without the 256-row tile; a short-K
  // down (the I of a TP shard) takes 64 x 64 tiles on a 2 x 2 wave grid without a K
  // split (each workgroup reads half the tokens' h instead of all of it), and a down
  // whose 128 x 64 tiles would not reach 160 workgroups 128 x 32 tiles.  Measured at
  // M = 64, 128, 256 (graph timings over distinct weight copies): replicated gate_up
  // 45.6 -> 42.1, 51.9 -> 47.2, 78.4 -> 70.7 us and down 29.0 -> 26.5, 32.9 -> 30.3,
  // 45.2 -> 42.5 us against 4-wave 128 x 128 tiles; TP8 down 7.45 -> 7.21, 7.82 -> 7.51,
  // 11.9 -> 9.31 us and TP16 down 5.49 -> 5.34, 5.84 -> 5.64, 7.55 -> 7.02 us against
  // 128 x 32 / 128 x 64 tiles.
  const bool stream_m = !hilo && M <= 256;
  const int64_t ksteps = (K + 63) / 64;
  auto stream_ks = [&](int bn, int bm = 128) {
    int64_t ks = (224 + tiles_for(bm, bn) / 2) / tiles_for(bm, bn);
    if (ks > ksteps / 12) ks = ksteps / 12;
    return ks < 1 ? (int64_t)1 : ks;
  };
  // 256-token tiles only where M fills at least 3/4 of them (gate_up: 85%; M = 400 was
  // 113 -> 117 us on 256 x 128 tiles, 78% full, while its down stage gained 63.5 -> 61.5).
  const int64_t padded256 = (M + 255) / 256 * 256;
  const bool full256 = stage == 0 ? M * 20 >= 17 * padded256 : M * 4 >= 3 * padded256;
  bool narrow_gu = false;  // the narrow gate_up rule below, with its own K split
  bool short_dn = false;   // the short-K down rule below: no K split
  if (o.bm.load() && o.bn.load()) {
    gp.bm = o.bm.load();
    gp.bn = o.bn.load();
  } else if (stream_m) {
    gp.bm = 128;
    gp.bn = 64;
    if (stage == 0 && tiles_for(128, 256) * stream_ks(256) >= 160) {
      gp.bn = 256;
    } else if (tiles_for(128, 128) * stream_ks(128) >= 160) {
      gp.bn = 128;
    } else if (stage == 0 && (M <= 64 || tiles_for(128, 64) * stream_ks(64) < 160)) {
      // 64 x 64 gate_up tiles (one MFMA tile of 16 gate + 16 up columns per wave) where
      // 128-token tiles would be half empty or leave compute units idle: TP8 M = 64
      // 13.0 -> 12.4 us, TP16 M = 64 11.7 -> 11.2 us, TP16 M = 128 13.5 -> 12.2 us
      // (216 workgroups instead of 108).
      gp.bm = 64;
      gp.bn = 64;
    } else if (stage == 1 && K < 2048 && M <= 128) {
      gp.bm = 64;
      gp.bn = 64;
    } else if (stage == 1 && K < 2048) {
      gp.wm = 4;  // two token tiles: 128 x 64 on 8 waves without a K split
      gp.wn = 2;
    } else if (stage == 1 && tiles_for(128, 64) * stream_ks(64) < 160) {
      gp.bn = 32;
    }
  } else if (!hilo && tiles_for(256, 256) >= 2 * kCUs && K >= 4096) {
    gp.bm = 256;
    gp.bn = 256;
  } else if (!hilo && stage == 1 && K >= 4096 && tiles_for(256, 256) * 8 >= 7 * kCUs) {
    // Long-K down stage whose 256 x 256 tiles fill 7/8 of the chip: one tile per compute
    // unit without a K split beats 128 x 128 tiles, whose 32 x 64 wave tiles read three
    // fragments per two MFMAs (M = 2048: 237.7 -> 201.6 us; M = 4096: 418.0 -> 375.2 us).
    gp.bm = 256;
    gp.bn = 256;
  } else if (!hilo && stage == 0 && K >= 4096 && full256 && tiles_for(256, 256) >= kCUs &&
             tiles_for(256, 256) * 10 >= 7 * kCUs * ((tiles_for(256, 256) + kCUs - 1) / kCUs)) {
    // gate_up whose 256 x 256 tiles fill the chip once with rounds at least 70% full
    // (M = 2048, I = 6144: 384 tiles, 376 -> 356 us against 128 x 128 tiles).
    gp.bm = 256;
    gp.bn = 256;
  } else if (!hilo && stage == 0 && K >= 4096 && M > 256 && M <= 384 && !full256 && tiles_for(128, 256) >= 96) {
    // gate_up at three 128-token tiles (M = 257-384) that would leave 256-token tiles
    // part empty: 128 x 256 tiles (8 waves, 3 stages) split K three ways, against 128 x
    // 128 tiles (M = 288 / 320 / 352: 108.2 -> 93.8, 107.9 -> 95.1, 109.0 -> 97.4 us).
    gp.bm = 128;
    gp.bn = 256;
  } else if (!hilo && K >= 4096 && M > 256 && (stage == 1 || full256) && tiles_for(256, 256) >= 48 &&
             (stage == 0 ? tiles_for(256, 256) < 384 : tiles_for(256, 256) <= kCUs)) {
    // Medium M, long K, wide weights: 256 x 256 tiles with the K split that fills about
    // one round (at most 4 slices; gate_up between one and 1.5 rounds takes 2), against
    // 256 x 128 and 128 x 128 tiles (graph timings at I = 6144, H = 7168):
    //   down    M = 384 / 640 / 768 / 896 / 1536 / 1792: 68.0 -> 62.3, 126.1 -> 84.8, 132.5 -> 89.1,
    //           136.9 -> 107.0, 198.8 -> 185.7, 221.9 -> 192.2 us (also with the second token
    //           tile part empty: M = 288 / 320 / 352: 68.3 -> 57.6, 69.5 -> 58.3, 70.3 -> 59.6 us);
    //   gate_up M = 512 / 896 / 1024 / 1280 / 1536: 123.6 -> 111.7, 203.3 -> 184.5, 217.5 -> 187.1,
    //           251.1 -> 196.7, 330.6 -> 316.6 us.
    gp.bm = 256;
    gp.bn = 256;
  } else if (!hilo && K >= 4096 && M <= 1024 && full256 &&
             (stage == 0 ? tiles_for(256, 128) >= kCUs / 2 : tiles_for(128, 128) < kCUs)) {
    // Medium M, long K: 256 x 128 tiles (8 waves, 3 stages) with a K split to about three
    // workgroups per compute unit (gate_up) or two slices (down).  M = 512: gate_up
    // 131.7 -> 122.0 us, down 73.0 -> 63.0 us; M = 1024: gate_up 237 -> 207 us.
    gp.bm = 256;
    gp.bn = 128;
  } else if (!hilo && stage == 0 && K >= 4096 && M > 256 && tiles_for(128, 128) < kCUs) {
    // Narrow gate_up (the I of a TP shard) at medium M streams weights that no cache
    // holds across a stack of layers, as the M <= 256 plans do: 128 x 256 tiles (8 waves,
    // 3 stages, one workgroup per compute unit) with K split to about 224 workgroups (at
    // most 12 slices), or, under 16 such tiles, 128 x 64 tiles on 8 waves split to about
    // 192.  Measured with 24 (TP8) or 48 (TP16) distinct weight copies, so that the weights
    // come from HBM, against 4-wave 128 x 64 tiles split to about 768 workgroups: TP8 M =
    // 512 / 1024 / 1536 35.1 -> 26.3, 45.8 -> 37.0, 52.1 -> 49.7 us; TP16 M = 512 / 1024 /
    // 2048 25.4 -> 20.1, 33.4 -> 26.3, 44.4 -> 37.4 us.
    gp.bm = 128;
    if (tiles_for(128, 256) >= 16) {
      gp.bn = 256;
    } else {
      gp.bn = 64;
      gp.wm = 4;
      gp.wn = 2;
    }
    narrow_gu = true;
  } else if (tiles_for(128, 128) >= (stage == 0 ? kCUs : 2 * kCUs) ||
             (stage == 1 && !hilo && K >= 2048 && tiles_for(128, 128) >= kCUs / 2)) {
    // The long-K down stage also takes 128 x 128 tiles from half a tile per compute
    // unit, K split to fill the chip (M = 512, I = 6144: 87.2 -> 72.2 us against
    // 128 x 64 tiles).
    gp.bm = 128;
    gp.bn = 128;
  } else if (stage == 1 && !hilo && K < 2048 && tiles_for(128, 64) < kCUs) {
    // Down with a short K (the I of a TP shard): 32-row tiles fill the chip without a K
    // split, so no fp32 partials and no finalize pass (half the time at M = 128).
    gp.bm = 128;
    gp.bn = 32;
  } else if (stage == 1 && !hilo && K < 2048 && M > 256) {
    // Short-K down below two rounds of 128 x 128 tiles: those tiles (8 waves, 2 stages)
    // once there are more of them than compute units, else 128 x 64 tiles on 8 waves
    // (3 stages); weights from HBM (24 / 48 distinct copies), against 4-wave 128 x 64
    // tiles: TP8 M = 384 / 640 / 768 24.3 -> 15.2, 21.3 -> 19.1, 22.5 -> 20.7 us; TP16
    // 18.2 -> 10.2, 13.9 -> 13.0, 14.0 -> 14.2 us.  No K split: with a contraction this
    // short the fp32 partials and their finalize pass cost as much as the GEMM (TP8
    // M = 320: 21.5 us with two slices, 11.7 us with one).
    gp.bm = 128;
    gp.bn = tiles_for(128, 128) > kCUs ? 128 : 64;
    gp.wm = 4;
    gp.wn = 2;
    short_dn = true;
  } else {
    gp.bm = 128;
    gp.bn = 64;
  }
  // Waves: 8 for the 128 x 128 and 256-wide tiles (two waves per SIMD overlap one wave's
  // LDS reads and barrier with the other's multiplies: M = 2048 down 225 -> 210 us, TP8
  // gate_up 74.5 -> 71.8 us), 4 for the narrow tiles and the two-plane down tile.
  if (o.wm.load() && o.wn.load()) {
    gp.wm = o.wm.load();
    gp.wn = o.wn.load();
  } else if (gp.wm && gp.wn) {
    // set with the tile above
  } else if (stream_m && stage == 0 && gp.bm == 128 && gp.bn == 64) {
    // 8 waves, each with one 32-column MFMA tile of 16 gate and 16 up columns (TP8 gate_up
    // at M = 64 / 128: 14.1 -> 13.2, 16.0 -> 15.6 us; TP16 13.6 -> 12.5, 14.5 -> 14.0 us)
    gp.wm = 4;
    gp.wn = 2;
  } else if (gp.bm == 256 && gp.bn == 128) {
    gp.wm = 4;
    gp.wn = 2;
  } else if (gp.bm == 256) {
    gp.wm = 2;
    gp.wn = 4;
  } else if (gp.bm == 64) {
    gp.wm = 2;
    gp.wn = 2;
  } else if (gp.bn <= 64) {
    gp.wm = 4;
    gp.wn = 1;
  } else if (gp.bn == 256) {
    gp.wm = 2;
    gp.wn = 4;
  } else if (hilo) {
    gp.wm = 2;
    gp.wn = 2;
  } else {
    gp.wm = 4;
    gp.wn = 2;
  }
  if (o.ns.load()) {
    gp.ns = o.ns.load();
  } else if (stream_m) {
    // the down stage's 128 x 128 tiles take two stages (64 KB, two workgroups per compute
    // unit) and a four-way K split: M = 128 / 192 / 256: 32.8 -> 31.8, 48.0 -> 43.6,
    // 50.8 -> 47.1 us against four stages and two slices
    gp.ns = gp.bn == 256 ? 3 : (stage == 1 && gp.bm == 128 && gp.bn == 128) ? 2 : 4;
  } else if ((gp.bm == 256 && gp.bn == 128) || (gp.bm == 128 && gp.bn == 256)) {
    gp.ns = 3;
  } else {
    // Two stages where compiled (the two-plane 128 x 128 down tile has three).
    gp.ns = 2;
    while (gp.ns < 4 && !smlp::gemm_instantiated(stage, hilo, gp.bm, gp.bn, gp.wm, gp.wn, gp.ns)) ++gp.ns;
  }
  if (!smlp::gemm_instantiated(stage, hilo, gp.bm, gp.bn, gp.wm, gp.wn, gp.ns)) return false;
  gp.tiles_m = (int)((M + gp.bm - 1) / gp.bm);
  const int64_t tiles = tiles_for(gp.bm, gp.bn);
  gp.tiles = (int)tiles;
  int64_t ks = o.ksplit.load();
  if (!ks && stream_m && stage == 0 && gp.bm == 64) {
    ks = stream_ks(64, 64);
  } else if (!ks && stream_m && (gp.bm == 64 || (stage == 1 && K < 2048))) {
    ks = 1;
  } else if (!ks && stream_m && gp.bm == 128) {
    ks = gp.bn == 32 ? 1 : (stage == 1 && gp.bn == 128 && ksteps >= 48) ? 4 : stream_ks(gp.bn);
  } else if (!ks) {
    if (narrow_gu && gp.bn == 256) {
      ks = 224 / tiles;
      if (ks > 12) ks = 12;
    } else if (narrow_gu) {
      ks = (192 + tiles - 1) / tiles;
      if (ks > 6) ks = 6;
    } else if (short_dn) {
      ks = 1;
    } else if (gp.bm == 128 && gp.bn == 256) {
      ks = 3;
    } else if (gp.bm == 256 && gp.bn == 128) {
      ks = stage == 0 ? (3 * kCUs + tiles - 1) / tiles : 2;
      if (ks > 4) ks = 4;
    } else if (gp.bm == 256 && gp.bn == 256) {
      // up to one round of tiles: split K to fill it; gate_up between one and 1.5 rounds:
      // two slices; else none (a down stage from 7/8 of a round takes no K split either)
      ks = tiles <= kCUs ? kCUs / tiles : (stage == 0 && tiles < 384) ? 2 : 1;
      if (ks > 4) ks = 4;
    } else if (gp.bn == 32) {
      ks = 1;
    } else if (gp.bn == 64 && gp.bm == 128) {
      // Few weight tiles (medium M): split K until about 3 (gate_up) or 1.75 (down)
      // workgroups per compute unit stream weights; fp32 partials cost 2 M / K of the
      // weight traffic per slice, so short K (I of a TP shard) takes at most 3 slices.
      const int64_t target = stage == 0 ? 3 * kCUs : 7 * kCUs / 4;
      ks = (target + tiles - 1) / tiles;
      if (ks > 16) ks = 16;
      if (K < 2048 && ks > 3) ks = 3;
    } else {
      ks = tiles >= kCUs ? 1 : (kCUs + tiles - 1) / tiles;
    }
    const int64_t max_ks = ksteps / 2;  // at least two 64-element K steps per slice
    if (ks > max_ks) ks = max_ks;
    if (ks < 1) ks = 1;
  }
  if (ks > ksteps) ks = ksteps;
  const int64_t kslice = ((K + ks - 1) / ks + 63) / 64 * 64;
  gp.ksplit = (int)((K + kslice - 1) / kslice);
  gp.kslice = (int)kslice;
  // Non-temporal weight loads where every workgroup streams its weights exactly once and
  // all re-read the activations: one token tile, long K, wide weights (the replicated
  // layer at M <= 128; TP shards, with short K or few weight rows, were slower with it).
  gp.ntb = !hilo && gp.tiles_m == 1 && K >= 2048 && N * fpr >= 4096 &&
           smlp::gemm_nt_instantiated(hilo, gp.bm, gp.bn, gp.wm, gp.wn, gp.ns);
  *out = gp;
  return true;
}

// A 256 x 256 plan runs one workgroup per compute unit; when its tiles fill the chip a
// whole number of times plus a partial last round (M = 8192, H = 7168 down: 896 tiles =
// 3.5 rounds; M = 2048, I = 6144 gate_up: 384 tiles = 1.5 rounds), the output columns of
// the whole rounds keep that tile and the remaining
// columns (down rows or gate_up features) run as a second launch of 128 x 128 tiles
// (8 waves, two workgroups per compute unit), which fills the chip in one round instead
// of leaving part of it idle.  Not applied to a pinned tile.  N counts down rows or
// gate_up features; returns whether the plan was split.
bool split_columns(int stage, int64_t M, int64_t N, int64_t K, smlp::GemmPlan* g, smlp::GemmPlan* tail,
                   int64_t* split) {
  if (g_gtune[stage].bm.load() || g->bm != 256 || g->bn != 256 || g->ksplit != 1) return false;
  // Split only where at least 1/8 of the unsplit plan's round slots would sit idle
  // (gate_up at M = 6144, 4.5 rounds: 930.7 -> 948.8 us split, against 2048: 359.7 ->
  // 328.9 and 3072: 533.7 -> 488.2 us).
  const int64_t rounds = g->tiles / kCUs, slots = (g->tiles + kCUs - 1) / kCUs * kCUs;
  if (rounds < 1 || g->tiles % kCUs == 0 || (slots - g->tiles) * 8 < slots) return false;
  // Down: only where the last round is under 9/16 full; from there the tail's 128 x 128
  // tiles cost more than the idle slots (down at M = 4096 and 6144, last round 75% and
  // 62.5% full: 388.9 and 559.3 us split against 369.8 and 537.9 unsplit; at 3072, 5120,
  // 7168 and 8192, 31%, 19%, 6% and 50% full, the split saves 42, 59, 63 and 27 us).
  if (stage == 1 && (g->tiles % kCUs) * 16 >= 9 * kCUs) return false;
  const int64_t width = stage == 0 ? 128 : 256;  // output columns per 256 x 256 tile
  const int64_t cols = rounds * kCUs / g->tiles_m;  // column tiles in whole rounds
  if (cols < 1 || cols >= (N + width - 1) / width) return false;
  smlp::GemmPlan t{};
  t.bm = 128;
  t.bn = 128;
  t.wm = 4;
  t.wn = 2;
  t.ns = 2;
  if (!smlp::gemm_instantiated(stage, false, t.bm, t.bn, t.wm, t.wn, t.ns)) return false;
  const int64_t rest = N - cols * width, twidth = width / 2;
  t.tiles_m = (int)((M + 127) / 128);
  t.tiles = (int)(t.tiles_m * ((rest + twidth - 1) / twidth));
  t.ksplit = 1;
  t.kslice = (int)((K + 63) / 64 * 64);
  g->tiles = (int)(g->tiles_m * cols);
  *tail = t;
  *split = cols * width;
  return true;
}

int out_elem(int dtype, int partial_fp32) { return (dtype == SMLP_FP32 || partial_fp32) ? 4 : 2; }

// Shape/dtype validation and plan; no pointer checks.
int make_plan(int64_t M, int64_t H, int64_t I, int dtype, int partial_fp32, smlp::Plan* p) {
  if (dtype != SMLP_BF16 && dtype != SMLP_FP32)
    return fail(SMLP_ERR_DTYPE, "dtype %d is neither SMLP_BF16 (0) nor SMLP_FP32 (1)", dtype);
  if (M < 0) return fail(SMLP_ERR_SHAPE, "M = %lld < 0", (long long)M);
  if (H < 1 || I < 1)
    return fail(SMLP_ERR_SHAPE, "H = %lld and I = %lld must be >= 1", (long long)H, (long long)I);
  if (H >= kLimit || I >= kLimit || 2 * I * H >= kLimit || M * H >= kLimit || M * I >= kLimit)
    return fail(SMLP_ERR_SHAPE, "sizes too large: M*H, M*I and 2*I*H must be < 2^31 (M=%lld H=%lld I=%lld)",
                (long long)M, (long long)H, (long long)I);
  if (dtype == SMLP_BF16 && (H % 8 || I % 8))
    return fail(SMLP_ERR_SHAPE, "bf16 needs H %% 8 == 0 and I %% 8 == 0 (H=%lld I=%lld)",
                (long long)H, (long long)I);
  std::memset(p, 0, sizeof *p);
  p->M = M;
  p->H = H;
  p->I = I;
  p->dtype = dtype;
  p->partial_fp32 = partial_fp32 ? 1 : 0;
  if (M == 0) {
    p->path = SMLP_PATH_NONE;
    p->h_dtype = dtype == SMLP_FP32 ? SMLP_FP32 : SMLP_BF16;
    return ok();
  }
  if (dtype == SMLP_FP32) {
    p->path = SMLP_PATH_FP32;
    p->h_dtype = SMLP_FP32;
    p->h_bytes = round_up((size_t)(M * I) * 4, 256);
    p->kernels = g_fuse.load() != 2 && smlp::fp32_small_layer(M, H, I) ? 1 : 2;
  } else if (M < g_threshold.load() && M <= kSmallMaxM) {
    p->path = SMLP_PATH_SMALL_M;
    // h as one bf16 plane (rounded once, as the serving stack stores it) when the down
    // contraction is long enough (I >= 256) for that rounding to average out and M <= 32
    // (the projection kernel streams the down weights with a deeper LDS ring than the
    // two-plane kernel has room for: 48.0 vs 51.5 us per Kimi-K3 layer at M = 16);
    // otherwise two planes hi + lo, with which h is effectively not rounded.
    const int hp = g_h_planes.load();
    const bool one = hp == 1 || (hp == 0 && M <= 32 && I >= 256);
    p->h_dtype = one ? SMLP_BF16 : SMLP_BF16_HILO;
    p->h_bytes = round_up((size_t)(M * I) * (one ? 2 : 4), 256);
    if (one && M > 32)
      return fail(SMLP_ERR_ARG, "one plane of h on the small-M path needs M <= 32 (M = %lld)", (long long)M);
    if (!plan_skinny(0, M, I, H, &p->gu) || !plan_skinny(1, M, H, I, &p->dn, one ? 2 : 1))
      return fail(SMLP_ERR_ARG, "the pinned small-M tuning is not a compiled configuration for M = %lld",
                  (long long)M);
    size_t part = 0;
    if (p->gu.ksplit > 1) part = (size_t)p->gu.ksplit * M * 2 * I * 4;
    if (p->dn.ksplit > 1) {
      size_t d = (size_t)p->dn.ksplit * M * H * 4;
      if (d > part) part = d;
    }
    p->part_bytes = round_up(part, 256);
    // a K-split streaming stage reduces in its own launch (the last-arriving slice of a
    // column applies the epilogue) when there are at most 256 columns; else a finalize launch
    auto finalize_launch = [](const smlp::SkinnyPlan& sp) {
      const int cols = sp.blocks / (sp.ksplit * (sp.ttiles > 1 ? sp.ttiles : 1));
      return sp.ksplit > 1 && !(g_fuse.load() != 2 && sp.kind == smlp::SKINNY_STREAM16 && sp.red_ok && cols <= 256);
    };
    p->kernels = 2 + finalize_launch(p->gu) + finalize_launch(p->dn);
    // both stages in one launch (one bf16 plane of h, M <= 32): see shared_mlp_tune_layer_fusion
    if (g_fuse.load() != 2 && smlp::decode_layer_eligible(*p)) p->kernels = 1;
  } else {
    p->path = SMLP_PATH_LARGE_M;
    // h for a bf16 output: one fp16 plane (the down stage converts its bf16 weight
    // fragments to fp16 in registers, exactly, and multiplies with fp16 MFMAs), rounded
    // with 11 significant bits instead of bf16's 8: with one bf16 plane, h's rounding on
    // top of the output's own rounding took the whole-output error to 0.94-1.01 of the
    // bound at M = 8100...8192 and 0.93 on medium shapes.  For an fp32 output (a TP
    // rank's partial, no output rounding) one bf16 plane keeps the error near 0.7 of the
    // bound and spares the conversion (5-14% of the down GEMM).  Two bf16 planes (hi +
    // lo) when the down contraction is too short (I < 256) for the rounding of h to
    // average out.
    const int hf = g_h_format.load();
    p->h_dtype = hf == 1 ? SMLP_BF16 : hf == 2 ? SMLP_BF16_HILO : hf == 3 ? SMLP_FP16
               : I < 256 ? SMLP_BF16_HILO : partial_fp32 ? SMLP_BF16 : SMLP_FP16;
    p->h_bytes = round_up((size_t)(M * I) * (p->h_dtype == SMLP_BF16_HILO ? 4 : 2), 256);
    const bool hilo = p->h_dtype == SMLP_BF16_HILO;
    // Only the down stage reads h; its two-plane form has its own tile list.
    if (!plan_gemm(0, M, I, H, false, &p->ggu) || !plan_gemm(1, M, H, I, hilo, &p->gdn))
      return fail(SMLP_ERR_ARG, "the pinned large-M tile is not a compiled configuration");
    const int ts = g_tsplit.load();
    if (ts != 2 && M <= 256 && (ts == 1 || token_split_default(M, I)) && plan_token_split(M, I, H, &p->gu))
      p->gu_tsplit = 1;
    size_t part = 0;
    if (!p->gu_tsplit && p->ggu.ksplit > 1) part = (size_t)p->ggu.ksplit * M * 2 * I * 4;
    if (p->gdn.ksplit > 1) {
      const size_t d = (size_t)p->gdn.ksplit * M * H * 4;
      if (d > part) part = d;
    }
    p->part_bytes = round_up(part, 256);
    p->kernels = 2 + (!p->gu_tsplit && p->ggu.ksplit > 1) + (p->gdn.ksplit > 1);
    if (split_columns(1, M, H, I, &p->gdn, &p->gdn_tail, &p->dn_split)) p->kernels += 1;
    if (!hilo && !p->gu_tsplit && split_columns(0, M, I, H, &p->ggu, &p->ggu_tail, &p->gu_split)) p->kernels += 1;
    // With fp16 h and many tokens, converting each weight fragment in registers costs more
    // than one streaming pass over w_down (M = 2048: +72 us in registers against ~27 us for
    // the pass; M = 8192: +130 us): convert once into the workspace.
    if (p->h_dtype == SMLP_FP16 && M >= g_wd16_min_m.load()) {
      p->wd16_bytes = round_up((size_t)(H * I) * 2, 256);
      p->kernels += 1;
    }
  }
  p->h_offset = 0;
  p->part_offset = p->h_bytes;
  p->wd16_offset = p->h_bytes + p->part_bytes;
  p->workspace_bytes = p->h_bytes + p->part_bytes + p->wd16_bytes;
  p->up_off = I;
  p->ldwd = I;
  return ok();
}

// Plan of the plain projection y[M, N] = x[M, K] . w[N, K]^T.  M < min(threshold, 33):
// the streaming kernel, 4 waves with a 4-stage ring, one 16-row tile per workgroup, or
// two when N has at least 64 tiles (every workgroup re-reads the activations of its K
// slice, so wider workgroups halve that traffic), and K split over workgroups to about
// 200 workgroups, with at least 14 K steps per slice.  Measured on MI355X (M = 16,
// K = 7168): N = 2112 takes 2 tiles x 3 slices (10.9 us), N = 132 one tile x 8 slices
// (5.9 us), each within noise of the best pinned plan.  Otherwise the LDS-tiled kernel
// with the down stage's tile rules.
struct LinearPlan {
  int path;
  smlp::SkinnyPlan sk;
  smlp::GemmPlan gm;
  int ksplit, blocks;
  size_t part_bytes;
};

int make_linear_plan(int64_t M, int64_t K, int64_t N, int64_t ldy, LinearPlan* lp) {
  if (M < 0) return fail(SMLP_ERR_SHAPE, "M = %lld < 0", (long long)M);
  if (K < 8 || K % 8 || N < 4 || N % 4)
    return fail(SMLP_ERR_SHAPE, "projection needs K >= 8, K %% 8 == 0, N >= 4, N %% 4 == 0 (K=%lld N=%lld)",
                (long long)K, (long long)N);
  if (ldy < N || ldy % 4)
    return fail(SMLP_ERR_SHAPE, "ldy = %lld must be >= N = %lld and a multiple of 4", (long long)ldy,
                (long long)N);
  if (K >= kLimit || N >= kLimit || ldy >= kLimit || M * K >= kLimit || N * K >= kLimit ||
      M * ldy >= kLimit)
    return fail(SMLP_ERR_SHAPE, "sizes too large: M*K, N*K and M*ldy must be < 2^31");
  std::memset(lp, 0, sizeof *lp);
  if (M == 0) {
    lp->path = SMLP_PATH_NONE;
    return ok();
  }
  const int64_t thr = g_threshold.load() < 33 ? g_threshold.load() : 33;
  if (M < thr) {
    using namespace smlp;
    const SkinnyOverride& o = g_tune[2];
    SkinnyPlan& sp = lp->sk;
    if (o.kind.load() && o.kind.load() != SKINNY_STREAM16)
      return fail(SMLP_ERR_ARG, "the projection's small-M kernel is kind %d only", SKINNY_STREAM16);
    sp.kind = SKINNY_STREAM16;
    sp.mt = M <= 16 ? 1 : 2;
    const int64_t tiles16 = (N + 15) / 16;
    int64_t nt = o.nb.load() ? o.nb.load() : (tiles16 >= 64 ? 2 : 1);
    if (nt > 4) nt = 4;
    sp.nb = (int)nt;
    sp.fpw = (int)(16 * nt);
    const int64_t groups = (N + sp.fpw - 1) / sp.fpw;
    static const int kPref[][2] = {{4, 4}, {8, 3}, {4, 6}, {8, 2}};
    sp.waves = o.waves.load();
    sp.u = o.u.load();
    if (!sp.waves || !sp.u) {
      for (const auto& c : kPref) {
        const int w = sp.waves ? sp.waves : c[0], st = sp.u ? sp.u : c[1];
        if (skinny_instantiated(2, sp.kind, sp.mt, sp.nb, w, st)) {
          sp.waves = w;
          sp.u = st;
          break;
        }
      }
    }
    if (!sp.waves || !sp.u || !skinny_instantiated(2, sp.kind, sp.mt, sp.nb, sp.waves, sp.u))
      return fail(SMLP_ERR_ARG, "the pinned projection tuning is not a compiled configuration");
    const int64_t ksteps = (K + 63) / 64;
    int64_t ks = o.ksplit.load();
    if (!ks) {
      ks = (200 + groups / 2) / groups;
      const int64_t max_ks = ksteps / 14;
      if (ks > max_ks) ks = max_ks;
      if (ks < 1) ks = 1;
    }
    if (ks > ksteps) ks = ksteps;
    const int64_t kslice = ((K + ks - 1) / ks + 63) / 64 * 64;
    ks = (K + kslice - 1) / kslice;
    sp.ksplit = (int)ks;
    sp.kslice = (int)kslice;
    sp.blocks = (int)(groups * ks);
    sp.red_ok = !o.nb.load() && !o.waves.load() && !o.u.load();  // as for the layer stages
    lp->path = SMLP_PATH_SMALL_M;
    lp->ksplit = sp.ksplit;
    lp->blocks = sp.blocks;
  } else {
    if (!plan_gemm(1, M, N, K, false, &lp->gm, &g_gtune[2]))
      return fail(SMLP_ERR_ARG, "the pinned projection tile is not a compiled configuration");
    lp->path = SMLP_PATH_LARGE_M;
    lp->ksplit = lp->gm.ksplit;
    lp->blocks = lp->gm.tiles * lp->gm.ksplit;
  }
  lp->part_bytes = lp->ksplit > 1 ? round_up((size_t)lp->ksplit * M * N * 4, 256) : 0;
  return ok();
}

int check_ptr(const void* ptr, const char* name, size_t align) {
  if (!ptr) return fail(SMLP_ERR_NULL, "%s is NULL", name);
  if (!aligned(ptr, align))
    return fail(SMLP_ERR_ALIGN, "%s = %p is not %zu-byte aligned", name, ptr, align);
  return SMLP_OK;
}

int hip_status(int rc, const char* what) {
  if (rc == hipSuccess) return SMLP_OK;
  return fail(SMLP_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)rc));
}

enum Stage { kBoth, kGateUp, kDown };

int run(Stage stage, const void* x, const void* wgu, const void* wd, void* out, int64_t M,
        int64_t H, int64_t I, int dtype, int partial_fp32, void* ws, size_t ws_bytes,
        hipStream_t stream) {
  smlp::Plan p;
  int rc = make_plan(M, H, I, dtype, partial_fp32, &p);
  if (rc) return rc;
  if (M == 0) return ok();
  const size_t al = dtype == SMLP_BF16 ? 16 : 4;
  const size_t ie = dtype == SMLP_BF16 ? 2 : 4;
  const size_t oe = (size_t)out_elem(dtype, partial_fp32);
  const size_t x_n = (size_t)(M * H) * ie, wgu_n = (size_t)(2 * I * H) * ie,
               wd_n = (size_t)(H * I) * ie, out_n = (size_t)(M * H) * oe;
  if (stage != kDown) {
    if ((rc = check_ptr(x, "x", al)) || (rc = check_ptr(wgu, "w_gate_up", al))) return rc;
  }
  if (stage != kGateUp) {
    if ((rc = check_ptr(wd, "w_down", al)) || (rc = check_ptr(out, "out", al))) return rc;
  }
  if ((rc = check_ptr(ws, "workspace", 256))) return rc;
  if (ws_bytes < p.workspace_bytes)
    return fail(SMLP_ERR_WORKSPACE, "workspace_bytes = %zu < %zu needed", ws_bytes,
                p.workspace_bytes);
  if (stage != kDown) {
    if (overlap(ws, p.workspace_bytes, x, x_n) || overlap(ws, p.workspace_bytes, wgu, wgu_n))
      return fail(SMLP_ERR_ALIAS, "workspace overlaps x or w_gate_up");
  }
  if (stage != kGateUp) {
    if (overlap(ws, p.workspace_bytes, wd, wd_n))
      return fail(SMLP_ERR_ALIAS, "workspace overlaps w_down");
    if (overlap(out, out_n, wd, wd_n) || overlap(out, out_n, ws, p.workspace_bytes) ||
        (stage == kBoth && (overlap(out, out_n, x, x_n) || overlap(out, out_n, wgu, wgu_n))))
      return fail(SMLP_ERR_ALIAS, "out overlaps an input or the workspace");
  }

  (void)hipGetLastError();  // clear stale state so a failure below is attributed to us
  if (stage == kBoth && g_fuse.load() != 2 && smlp::decode_layer_eligible(p)) {
    const int slot = layer_sync_slot(stream);
    if (slot >= 0)
      return hip_status(smlp::launch_decode_layer(p, x, wgu, wd, out, ws, slot, g_fuse_limit.load(), stream),
                        "decode layer launch");
  }
  if (stage == kBoth && g_fuse.load() != 2 && p.path == SMLP_PATH_FP32 && smlp::fp32_small_layer(p.M, p.H, p.I))
    return hip_status(smlp::launch_fp32_layer(p, (const float*)x, (const float*)wgu, (const float*)wd,
                                              (float*)out, stream),
                      "fp32 layer launch");
  if (stage != kDown) {
    switch (p.path) {
      case SMLP_PATH_FP32:
        rc = smlp::launch_fp32_gate_up(p, (const float*)x, (const float*)wgu, ws, stream);
        break;
      case SMLP_PATH_SMALL_M: rc = smlp::launch_skinny_gate_up(p, x, wgu, ws, stream); break;
      default:
        rc = p.gu_tsplit ? smlp::launch_skinny_gate_up(p, x, wgu, ws, stream)
                         : smlp::launch_gemm_gate_up(p, x, wgu, ws, stream);
        break;
    }
    if ((rc = hip_status(rc, "gate_up launch"))) return rc;
  }
  if (stage != kGateUp) {
    switch (p.path) {
      case SMLP_PATH_FP32:
        rc = smlp::launch_fp32_down(p, (const float*)wd, (float*)out, ws, stream);
        break;
      case SMLP_PATH_SMALL_M: rc = smlp::launch_skinny_down(p, wd, out, ws, stream); break;
      default: rc = smlp::launch_gemm_down(p, wd, out, ws, stream); break;
    }
    if ((rc = hip_status(rc, "down launch"))) return rc;
  }
  return ok();
}

}  // namespace

namespace smlp {
// Counter slot of a stream (one-launch decode layer, in-launch K-split reductions):
// launches on one stream run one after another and share a slot; each stream gets its
// own, up to kLayerSyncSlots per device (-1 beyond that: those stages then run as
// separate launches).
int stream_slot(hipStream_t stream) {
  struct Key {
    int dev;
    hipStream_t s;
  };
  static std::mutex mu;
  static std::vector<Key> keys;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  int n = 0;
  for (const Key& k : keys) {
    if (k.dev != dev) continue;
    if (k.s == stream) return n;
    ++n;
  }
  if (n >= smlp::kLayerSyncSlots) return -1;
  keys.push_back({dev, stream});
  return n;
}

bool fusion_enabled() { return g_fuse.load() != 2; }

// Status setter shared with the other host-only translation units (layout.cpp).
int set_error(int status, const char* msg) {
  if (status == SMLP_OK) return ok();
  return fail(status, "%s", msg);
}
}  // namespace smlp

extern "C" {

const char* shared_mlp_status_string(int status) {
  switch (status) {
    case SMLP_OK: return "SMLP_OK";
    case SMLP_ERR_NULL: return "SMLP_ERR_NULL";
    case SMLP_ERR_SHAPE: return "SMLP_ERR_SHAPE";
    case SMLP_ERR_ALIGN: return "SMLP_ERR_ALIGN";
    case SMLP_ERR_ALIAS: return "SMLP_ERR_ALIAS";
    case SMLP_ERR_WORKSPACE: return "SMLP_ERR_WORKSPACE";
    case SMLP_ERR_DTYPE: return "SMLP_ERR_DTYPE";
    case SMLP_ERR_HIP: return "SMLP_ERR_HIP";
    case SMLP_ERR_ARG: return "SMLP_ERR_ARG";
    default: return "SMLP_ERR_UNKNOWN";
  }
}

const char* shared_mlp_last_error(void) { return g_last_error.c_str(); }

int shared_mlp_plan(int64_t M, int64_t H, int64_t I, int dtype, int partial_fp32,
                    smlp_plan* plan) {
  if (!plan) return fail(SMLP_ERR_NULL, "plan is NULL");
  smlp::Plan p;
  int rc = make_plan(M, H, I, dtype, partial_fp32, &p);
  if (rc) return rc;
  plan->path = p.path;
  plan->h_dtype = p.h_dtype;
  plan->h_offset = p.h_offset;
  plan->workspace_bytes = p.workspace_bytes;
  if (p.path == SMLP_PATH_SMALL_M) {
    plan->gate_up_ksplit = p.gu.ksplit;
    plan->down_ksplit = p.dn.ksplit;
    plan->gate_up_blocks = p.gu.blocks;
    plan->down_blocks = p.dn.blocks;
  } else if (p.path == SMLP_PATH_LARGE_M) {
    plan->gate_up_ksplit = p.gu_tsplit ? 1 : p.ggu.ksplit;
    plan->down_ksplit = p.gdn.ksplit;
    plan->gate_up_blocks = p.gu_tsplit ? p.gu.blocks : p.ggu.tiles * p.ggu.ksplit + (p.gu_split ? p.ggu_tail.tiles : 0);
    plan->down_blocks = p.gdn.tiles * p.gdn.ksplit + (p.dn_split ? p.gdn_tail.tiles : 0);
  } else {
    plan->gate_up_ksplit = plan->down_ksplit = 1;
    plan->gate_up_blocks = plan->down_blocks = 0;
  }
  plan->kernels = p.kernels;
  return ok();
}

int shared_mlp_workspace_bytes(int64_t M, int64_t H, int64_t I, int dtype, size_t* bytes) {
  if (!bytes) return fail(SMLP_ERR_NULL, "bytes is NULL");
  size_t worst = 0;
  for (int partial = 0; partial < 2; ++partial) {
    smlp::Plan p;
    int rc = make_plan(M, H, I, dtype, partial, &p);
    if (rc) return rc;
    if (p.workspace_bytes > worst) worst = p.workspace_bytes;
  }
  *bytes = worst;
  return ok();
}

int shared_mlp_forward(const void* x, const void* w_gate_up, const void* w_down, void* out,
                       int64_t M, int64_t H, int64_t I, int dtype, int partial_fp32,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(kBoth, x, w_gate_up, w_down, out, M, H, I, dtype, partial_fp32, workspace,
             workspace_bytes, stream);
}

int shared_mlp_forward_noalloc(const void* x, const void* w_gate_up, const void* w_down, void* out,
                               int64_t M, int64_t H, int64_t I, int dtype, int partial_fp32,
                               hipStream_t stream) {
  // Host-side checks first (no HIP call before them): the plan, the scratch limit and
  // the pointers; run() repeats the full validation against the scratch array.
  smlp::Plan p;
  int rc = make_plan(M, H, I, dtype, partial_fp32, &p);
  if (rc) return rc;
  if (M == 0) return ok();
  if (p.workspace_bytes > (size_t)SMLP_NOALLOC_SCRATCH_BYTES)
    return fail(SMLP_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch, more than the %zu bytes of the static scratch array "
                "(call shared_mlp_forward with a workspace instead)",
                p.workspace_bytes, (size_t)SMLP_NOALLOC_SCRATCH_BYTES);
  const size_t al = dtype == SMLP_BF16 ? 16 : 4;
  if ((rc = check_ptr(x, "x", al)) || (rc = check_ptr(w_gate_up, "w_gate_up", al)) ||
      (rc = check_ptr(w_down, "w_down", al)) || (rc = check_ptr(out, "out", al)))
    return rc;
  void* scratch = nullptr;
  if ((rc = hip_status(smlp::noalloc_scratch(&scratch), "static scratch lookup"))) return rc;
  return run(kBoth, x, w_gate_up, w_down, out, M, H, I, dtype, partial_fp32, scratch,
             (size_t)SMLP_NOALLOC_SCRATCH_BYTES, stream);
}

int shared_mlp_gate_up_act(const void* x, const void* w_gate_up, int64_t M, int64_t H,
                           int64_t I, int dtype, int partial_fp32, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return run(kGateUp, x, w_gate_up, nullptr, nullptr, M, H, I, dtype, partial_fp32, workspace,
             workspace_bytes, stream);
}

int shared_mlp_down(const void* w_down, void* out, int64_t M, int64_t H, int64_t I, int dtype,
                    int partial_fp32, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return run(kDown, nullptr, nullptr, w_down, out, M, H, I, dtype, partial_fp32, workspace,
             workspace_bytes, stream);
}

int shared_mlp_linear_plan(int64_t M, int64_t K, int64_t N, smlp_plan* plan) {
  if (!plan) return fail(SMLP_ERR_NULL, "plan is NULL");
  LinearPlan lp;
  int rc = make_linear_plan(M, K, N, N, &lp);
  if (rc) return rc;
  std::memset(plan, 0, sizeof *plan);
  plan->path = lp.path;
  plan->h_dtype = SMLP_BF16;
  plan->workspace_bytes = lp.part_bytes;
  plan->down_ksplit = lp.path == SMLP_PATH_NONE ? 1 : lp.ksplit;
  plan->down_blocks = lp.blocks;
  const bool red_here = lp.path == SMLP_PATH_SMALL_M && g_fuse.load() != 2 && lp.sk.red_ok &&
                        lp.sk.blocks / lp.sk.ksplit <= 256;
  plan->kernels = lp.path == SMLP_PATH_NONE ? 0 : 1 + (lp.ksplit > 1 && !red_here);
  return ok();
}

int shared_mlp_linear_workspace_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes) {
  if (!bytes) return fail(SMLP_ERR_NULL, "bytes is NULL");
  LinearPlan lp;
  int rc = make_linear_plan(M, K, N, N, &lp);
  if (rc) return rc;
  *bytes = lp.part_bytes;
  return ok();
}

int shared_mlp_linear(const void* x, const void* w, void* y, int64_t M, int64_t K, int64_t N,
                      int64_t ldy, int out_fp32, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (out_fp32 != 0 && out_fp32 != 1) return fail(SMLP_ERR_DTYPE, "out_fp32 = %d is neither 0 nor 1", out_fp32);
  LinearPlan lp;
  int rc = make_linear_plan(M, K, N, ldy, &lp);
  if (rc) return rc;
  if (M == 0) return ok();
  const size_t oe = out_fp32 ? 4 : 2;
  if ((rc = check_ptr(x, "x", 16)) || (rc = check_ptr(w, "w", 16)) || (rc = check_ptr(y, "y", 4 * oe)))
    return rc;
  if (lp.part_bytes) {
    if ((rc = check_ptr(workspace, "workspace", 256))) return rc;
    if (workspace_bytes < lp.part_bytes)
      return fail(SMLP_ERR_WORKSPACE, "workspace_bytes = %zu < %zu needed", workspace_bytes, lp.part_bytes);
  }
  const size_t x_n = (size_t)(M * K) * 2, w_n = (size_t)(N * K) * 2,
               y_n = ((size_t)(M - 1) * ldy + N) * oe;
  if (overlap(y, y_n, x, x_n) || overlap(y, y_n, w, w_n) || overlap(y, y_n, workspace, lp.part_bytes))
    return fail(SMLP_ERR_ALIAS, "y overlaps x, w or the workspace");
  if (overlap(workspace, lp.part_bytes, x, x_n) || overlap(workspace, lp.part_bytes, w, w_n))
    return fail(SMLP_ERR_ALIAS, "workspace overlaps x or w");
  (void)hipGetLastError();
  float* part = static_cast<float*>(workspace);
  if (lp.path == SMLP_PATH_SMALL_M)
    rc = smlp::launch_skinny_linear(lp.sk, x, w, y, (int)M, (int)K, (int)N, (int)ldy, out_fp32, part, stream);
  else
    rc = smlp::launch_gemm_linear(lp.gm, x, w, y, (int)M, (int)K, (int)N, (int)ldy, out_fp32, part, stream);
  if ((rc = hip_status(rc, "projection launch"))) return rc;
  return ok();
}

int shared_mlp_restore_logical(const void* gathered, void* out, int64_t M, int64_t n_gathered,
                               const int64_t* sizes, int nsizes, int tp, int elem_bytes,
                               hipStream_t stream) {
  if (!sizes) return fail(SMLP_ERR_NULL, "sizes is NULL");
  if (nsizes < 1 || nsizes > SMLP_MAX_RANGES)
    return fail(SMLP_ERR_ARG, "nsizes = %d outside [1, %d]", nsizes, SMLP_MAX_RANGES);
  if (elem_bytes != 2 && elem_bytes != 4)
    return fail(SMLP_ERR_ARG, "elem_bytes = %d is neither 2 nor 4", elem_bytes);
  if (tp < 1) return fail(SMLP_ERR_SHAPE, "tp = %d < 1", tp);
  int64_t total = 0;
  for (int t = 0; t < nsizes; ++t) {
    if (sizes[t] <= 0 || sizes[t] % tp)
      return fail(SMLP_ERR_SHAPE, "range %d has size %lld, not a positive multiple of tp = %d", t,
                  (long long)sizes[t], tp);
    if (sizes[t] >= kLimit) return fail(SMLP_ERR_SHAPE, "range %d is too large", t);
    total += sizes[t];
  }
  if (n_gathered != total)
    return fail(SMLP_ERR_SHAPE, "gathered width %lld does not match the ranges (sum %lld)",
                (long long)n_gathered, (long long)total);
  if (M < 0 || M * n_gathered >= kLimit)
    return fail(SMLP_ERR_SHAPE, "M = %lld out of range (M * n_gathered < 2^31)", (long long)M);
  if (M == 0) return ok();
  int rc;
  if ((rc = check_ptr(gathered, "gathered", elem_bytes)) || (rc = check_ptr(out, "out", elem_bytes))) return rc;
  const size_t n = (size_t)(M * n_gathered) * elem_bytes;
  if (overlap(gathered, n, out, n)) return fail(SMLP_ERR_ALIAS, "out overlaps gathered");
  (void)hipGetLastError();
  rc = smlp::launch_restore_logical(gathered, out, M, n_gathered, sizes, nsizes, tp, elem_bytes, stream);
  if ((rc = hip_status(rc, "restore launch"))) return rc;
  return ok();
}

int shared_mlp_forward_rank(const void* x, const void* w_gate_up, const void* w_down, void* out,
                            int64_t M, int64_t H, int64_t I, int tp, int rank, int dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (tp < 1 || rank < 0 || rank >= tp || I < 1 || I % tp)
    return fail(SMLP_ERR_ARG, "rank %d of tp %d does not slice I = %lld", rank, tp, (long long)I);
  const int64_t sl = I / tp;
  smlp::Plan p;
  int rc = make_plan(M, H, sl, dtype, 1, &p);
  if (rc) return rc;
  if (2 * I * H >= kLimit) return fail(SMLP_ERR_SHAPE, "2*I*H must be < 2^31");
  if (M == 0) return ok();
  const size_t al = dtype == SMLP_BF16 ? 16 : 4, e = dtype == SMLP_BF16 ? 2 : 4;
  if ((rc = check_ptr(x, "x", al)) || (rc = check_ptr(w_gate_up, "w_gate_up", al)) ||
      (rc = check_ptr(w_down, "w_down", al)) || (rc = check_ptr(out, "out", al)) ||
      (rc = check_ptr(workspace, "workspace", 256)))
    return rc;
  if (workspace_bytes < p.workspace_bytes)
    return fail(SMLP_ERR_WORKSPACE, "workspace_bytes = %zu < %zu needed", workspace_bytes, p.workspace_bytes);
  const size_t x_n = (size_t)(M * H) * e, wgu_n = (size_t)(2 * I * H) * e, wd_n = (size_t)(H * I) * e,
               out_n = (size_t)(M * H) * 4, ws_n = p.workspace_bytes;
  if (overlap(workspace, ws_n, x, x_n) || overlap(workspace, ws_n, w_gate_up, wgu_n) ||
      overlap(workspace, ws_n, w_down, wd_n) || overlap(out, out_n, x, x_n) ||
      overlap(out, out_n, w_gate_up, wgu_n) || overlap(out, out_n, w_down, wd_n) ||
      overlap(out, out_n, workspace, ws_n))
    return fail(SMLP_ERR_ALIAS, "out or the workspace overlaps an input (or each other)");
  // The rank's slice, read in place: gate rows [r s, (r+1) s) with their up rows I rows
  // further on, and the K range [r s, (r+1) s) of every w_down row (row stride I).
  p.up_off = I;
  p.ldwd = I;
  const char* gu = static_cast<const char*>(w_gate_up) + (size_t)rank * sl * H * e;
  const char* wd = static_cast<const char*>(w_down) + (size_t)rank * sl * e;
  (void)hipGetLastError();
  switch (p.path) {
    case SMLP_PATH_FP32: rc = smlp::launch_fp32_gate_up(p, (const float*)x, (const float*)gu, workspace, stream); break;
    case SMLP_PATH_SMALL_M: rc = smlp::launch_skinny_gate_up(p, x, gu, workspace, stream); break;
    default:
      rc = p.gu_tsplit ? smlp::launch_skinny_gate_up(p, x, gu, workspace, stream)
                       : smlp::launch_gemm_gate_up(p, x, gu, workspace, stream);
      break;
  }
  if ((rc = hip_status(rc, "gate_up launch"))) return rc;
  switch (p.path) {
    case SMLP_PATH_FP32: rc = smlp::launch_fp32_down(p, (const float*)wd, (float*)out, workspace, stream); break;
    case SMLP_PATH_SMALL_M: rc = smlp::launch_skinny_down(p, wd, out, workspace, stream); break;
    default: rc = smlp::launch_gemm_down(p, wd, out, workspace, stream); break;
  }
  if ((rc = hip_status(rc, "down launch"))) return rc;
  return ok();
}

int64_t shared_mlp_set_large_m_threshold(int64_t threshold) {
  if (threshold < 1 || threshold > kSmallMaxM + 1) {
    fail(SMLP_ERR_ARG, "threshold %lld outside [1, %lld]", (long long)threshold,
         (long long)(kSmallMaxM + 1));
    return -1;
  }
  ok();
  return g_threshold.exchange(threshold);
}

int shared_mlp_tune_skinny(int stage, int kind, int nb, int waves, int u, int ksplit) {
  if (stage < 0 || stage > 2 || kind < 0 || kind == 1 || kind > 3 || (stage == 2 && kind == 2) ||
      !(nb == 0 || nb == 1 || nb == 2 || nb == 3 || nb == 4) ||
      !(waves == 0 || waves == 4 || waves == 8) || u < 0 || u > 8 || ksplit < 0 || ksplit > 1024)
    return fail(SMLP_ERR_ARG, "bad small-M tuning (stage %d kind %d nb %d waves %d u %d ksplit %d)",
                stage, kind, nb, waves, u, ksplit);
  g_tune[stage].kind = kind;
  g_tune[stage].nb = nb;
  g_tune[stage].waves = waves;
  g_tune[stage].u = u;
  g_tune[stage].ksplit = ksplit;
  return ok();
}

int shared_mlp_tune_layer_fusion(int mode, int poll_limit) {
  if (mode < 0 || mode > 2) return fail(SMLP_ERR_ARG, "mode = %d outside {0, 1, 2}", mode);
  g_fuse = mode;
  g_fuse_limit = poll_limit > 0 ? poll_limit : poll_limit == 0 ? 1 << 18 : 0;
  return ok();
}

int shared_mlp_tune_h_planes(int planes) {
  if (planes < 0 || planes > 2) return fail(SMLP_ERR_ARG, "planes = %d outside {0, 1, 2}", planes);
  g_h_planes = planes;
  return ok();
}

int64_t shared_mlp_tune_weight_convert(int64_t min_m) {
  if (min_m < 1) {
    fail(SMLP_ERR_ARG, "min_m = %lld < 1", (long long)min_m);
    return -1;
  }
  ok();
  return g_wd16_min_m.exchange(min_m);
}

int shared_mlp_tune_token_split(int mode) {
  if (mode < 0 || mode > 2) return fail(SMLP_ERR_ARG, "mode = %d outside {0, 1, 2}", mode);
  g_tsplit = mode;
  return ok();
}

int shared_mlp_tune_h_format(int fmt) {
  if (fmt < 0 || fmt > 3) return fail(SMLP_ERR_ARG, "fmt = %d outside {0, 1, 2, 3}", fmt);
  g_h_format = fmt;
  return ok();
}

int shared_mlp_tune_gemm(int stage, int bm, int bn, int wm, int wn, int ns, int ksplit) {
  if (stage < 0 || stage > 2 || !(bm == 0 || bm == 64 || bm == 128 || bm == 256) ||
      !(bn == 0 || bn == 32 || bn == 64 || bn == 128 || bn == 256) || (bm == 0) != (bn == 0) ||
      !(wm == 0 || wm == 1 || wm == 2 || wm == 4) || !(wn == 0 || wn == 1 || wn == 2 || wn == 4) ||
      (wm == 0) != (wn == 0) || ns < 0 || ns > 8 || ksplit < 0 || ksplit > 1024)
    return fail(SMLP_ERR_ARG, "bad large-M tuning (stage %d bm %d bn %d wm %d wn %d ns %d ksplit %d)", stage,
                bm, bn, wm, wn, ns, ksplit);
  g_gtune[stage].bm = bm;
  g_gtune[stage].bn = bn;
  g_gtune[stage].wm = wm;
  g_gtune[stage].wn = wn;
  g_gtune[stage].ns = ns;
  g_gtune[stage].ksplit = ksplit;
  return ok();
}

int shared_mlp_shard_eligible(int flag_on, int use_sequence_parallel, int caller_eligible, int tp,
                              int64_t H, int64_t I) {
  return (flag_on && use_sequence_parallel && caller_eligible && tp > 1 && H % tp == 0 &&
          I % tp == 0)
             ? 1
             : 0;
}

int shared_mlp_slice_rank(const void* w_gate_up, const void* w_down, void* w_gate_up_r,
                          void* w_down_r, int64_t H, int64_t I, int tp, int rank, int dtype,
                          hipStream_t stream) {
  if (dtype != SMLP_BF16 && dtype != SMLP_FP32)
    return fail(SMLP_ERR_DTYPE, "dtype %d is neither SMLP_BF16 (0) nor SMLP_FP32 (1)", dtype);
  if (H < 1 || I < 1 || 2 * I * H >= kLimit)
    return fail(SMLP_ERR_SHAPE, "H = %lld, I = %lld out of range", (long long)H, (long long)I);
  if (dtype == SMLP_BF16 && (H % 8 || I % 8))
    return fail(SMLP_ERR_SHAPE, "bf16 needs H %% 8 == 0 and I %% 8 == 0");
  if (tp < 1 || I % tp || rank < 0 || rank >= tp)
    return fail(SMLP_ERR_ARG, "rank %d of tp %d does not slice I = %lld", rank, tp, (long long)I);
  const size_t al = dtype == SMLP_BF16 ? 16 : 4, e = dtype == SMLP_BF16 ? 2 : 4;
  int rc;
  if ((rc = check_ptr(w_gate_up, "w_gate_up", al)) || (rc = check_ptr(w_down, "w_down", al)) ||
      (rc = check_ptr(w_gate_up_r, "w_gate_up_r", al)) ||
      (rc = check_ptr(w_down_r, "w_down_r", al)))
    return rc;
  const int64_t s = I / tp;
  const size_t ngu = (size_t)(2 * I * H) * e, nwd = (size_t)(H * I) * e,
               ngu_r = (size_t)(2 * s * H) * e, nwd_r = (size_t)(H * s) * e;
  if (overlap(w_gate_up_r, ngu_r, w_gate_up, ngu) || overlap(w_gate_up_r, ngu_r, w_down, nwd) ||
      overlap(w_down_r, nwd_r, w_gate_up, ngu) || overlap(w_down_r, nwd_r, w_down, nwd) ||
      overlap(w_gate_up_r, ngu_r, w_down_r, nwd_r))
    return fail(SMLP_ERR_ALIAS, "slice destinations overlap the sources or each other");
  (void)hipGetLastError();
  rc = smlp::launch_slice_rank(w_gate_up, w_down, w_gate_up_r, w_down_r, H, I, tp, rank, (int)e,
                               stream);
  if ((rc = hip_status(rc, "slice launch"))) return rc;
  return ok();
}

int shared_mlp_rms_rescale(const float* in, void* out, int64_t M, int64_t H, hipStream_t stream) {
  if (M < 0 || H < 4 || H % 4 || M * H >= kLimit || M >= 0x7fffffff)
    return fail(SMLP_ERR_SHAPE, "rescale needs M >= 0, H >= 4, H %% 4 == 0 (M=%lld H=%lld)",
                (long long)M, (long long)H);
  if (M == 0) return ok();
  int rc;
  if ((rc = check_ptr(in, "in", 16)) || (rc = check_ptr(out, "out", 16))) return rc;
  if (overlap(in, (size_t)(M * H) * 4, out, (size_t)(M * H) * 2))
    return fail(SMLP_ERR_ALIAS, "out overlaps in");
  (void)hipGetLastError();
  rc = smlp::launch_rms_rescale(in, (uint16_t*)out, M, H, stream);
  if ((rc = hip_status(rc, "rescale launch"))) return rc;
  return ok();
}

}  // extern "C"
