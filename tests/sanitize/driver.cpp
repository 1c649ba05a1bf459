// Host-only driver of libsmlp's C ABI for the AddressSanitizer / UndefinedBehaviorSanitizer
// build: every validation path, the planners over a grid of shapes, the layout model on
// random curves, the tuning hooks and the error reporting.  No GPU is needed (the kernel
// launchers are stand-ins that report hipErrorNotReady).  Exits non-zero on a wrong status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "smlp.h"
#include "smlp_latent.h"
#include "smlp_layout.h"
#include "smlp_tuning.h"

static int g_fail = 0;
#define EXPECT(cond)                                                         \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, \
                   shared_mlp_last_error());                                 \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

// Fake device addresses: never dereferenced on the host; aligned as the ABI requires.
static void* fake(uintptr_t base) { return reinterpret_cast<void*>(base); }

static void plans() {
  const int64_t Ms[] = {0, 1, 5, 16, 17, 32, 33, 64, 100, 128, 129, 256, 300, 512, 1024, 2048, 8192};
  const int64_t Hs[] = {8, 16, 64, 1024, 4096, 7168, 8704, 16384};
  const int64_t Is[] = {8, 24, 64, 256, 384, 768, 1032, 1536, 4096, 6144, 8192};
  for (int64_t thr : {33, 129})
    for (int64_t M : Ms)
      for (int64_t H : Hs)
        for (int64_t I : Is)
          for (int part = 0; part < 2; ++part) {
            if (2 * I * H >= (int64_t(1) << 31) || M * H >= (int64_t(1) << 31)) continue;
            EXPECT(shared_mlp_set_large_m_threshold(thr) >= 1);
            smlp_plan p;
            EXPECT(shared_mlp_plan(M, H, I, SMLP_BF16, part, &p) == SMLP_OK);
            size_t ws = 0;
            EXPECT(shared_mlp_workspace_bytes(M, H, I, SMLP_BF16, &ws) == SMLP_OK);
            EXPECT(ws >= p.workspace_bytes);
            smlp_plan q;
            EXPECT(shared_mlp_linear_plan(M, H, I, &q) == SMLP_OK);
          }
  shared_mlp_set_large_m_threshold(33);
  smlp_plan p;
  EXPECT(shared_mlp_plan(12, 16, 12, SMLP_FP32, 0, &p) == SMLP_OK && p.path == SMLP_PATH_FP32);
  EXPECT(shared_mlp_plan(-1, 16, 12, SMLP_BF16, 0, &p) == SMLP_ERR_SHAPE);
  EXPECT(shared_mlp_plan(4, 12, 16, SMLP_BF16, 0, &p) == SMLP_ERR_SHAPE);
  EXPECT(shared_mlp_plan(4, 16, 16, 7, 0, &p) == SMLP_ERR_DTYPE);
  EXPECT(shared_mlp_plan(4, 16, 16, SMLP_BF16, 0, nullptr) == SMLP_ERR_NULL);
  EXPECT(shared_mlp_plan(int64_t(1) << 40, 16, 16, SMLP_BF16, 0, &p) == SMLP_ERR_SHAPE);
}

static void forward_validation() {
  const int64_t M = 16, H = 7168, I = 6144;
  size_t ws = 0;
  EXPECT(shared_mlp_workspace_bytes(M, H, I, SMLP_BF16, &ws) == SMLP_OK);
  // disjoint fake ranges, 1 GiB apart
  void *x = fake(1ull << 40), *wgu = fake(2ull << 40), *wd = fake(3ull << 40), *out = fake(4ull << 40),
       *w = fake(5ull << 40);
  EXPECT(shared_mlp_forward(nullptr, wgu, wd, out, M, H, I, SMLP_BF16, 0, w, ws, nullptr) == SMLP_ERR_NULL);
  EXPECT(shared_mlp_forward(fake((1ull << 40) + 2), wgu, wd, out, M, H, I, SMLP_BF16, 0, w, ws, nullptr) ==
         SMLP_ERR_ALIGN);
  EXPECT(shared_mlp_forward(x, wgu, wd, out, M, H, I, SMLP_BF16, 0, w, ws - 1, nullptr) == SMLP_ERR_WORKSPACE);
  EXPECT(shared_mlp_forward(x, wgu, wd, x, M, H, I, SMLP_BF16, 0, w, ws, nullptr) == SMLP_ERR_ALIAS);
  EXPECT(shared_mlp_forward(x, wgu, wd, out, M, H, I, SMLP_BF16, 0, wgu, ws, nullptr) == SMLP_ERR_ALIAS);
  EXPECT(shared_mlp_forward(x, wgu, wd, out, M, H, 12, SMLP_BF16, 0, w, ws, nullptr) == SMLP_ERR_SHAPE);
  EXPECT(shared_mlp_forward(x, wgu, wd, out, 0, H, I, SMLP_BF16, 0, w, ws, nullptr) == SMLP_OK);
  // valid arguments reach the (stand-in) launcher, which fails
  EXPECT(shared_mlp_forward(x, wgu, wd, out, M, H, I, SMLP_BF16, 0, w, ws, nullptr) == SMLP_ERR_HIP);
  EXPECT(std::strlen(shared_mlp_last_error()) > 0);
  EXPECT(shared_mlp_gate_up_act(x, wgu, M, H, I, SMLP_BF16, 0, w, ws, nullptr) == SMLP_ERR_HIP);
  EXPECT(shared_mlp_down(wd, out, M, H, I, SMLP_BF16, 0, nullptr, ws, nullptr) == SMLP_ERR_NULL);
  EXPECT(shared_mlp_forward_rank(x, wgu, wd, out, 128, H, I, 8, 8, SMLP_BF16, w, ws, nullptr) == SMLP_ERR_ARG);
  EXPECT(shared_mlp_forward_rank(x, wgu, wd, out, 128, H, I, 7, 0, SMLP_BF16, w, ws, nullptr) == SMLP_ERR_ARG);
  EXPECT(shared_mlp_slice_rank(wgu, wd, x, out, H, I, 8, 3, SMLP_BF16, nullptr) == SMLP_ERR_HIP);
  EXPECT(shared_mlp_slice_rank(wgu, wd, wgu, out, H, I, 8, 3, SMLP_BF16, nullptr) == SMLP_ERR_ALIAS);
  EXPECT(shared_mlp_rms_rescale((const float*)x, out, 128, 7168, nullptr) == SMLP_ERR_HIP);
  EXPECT(shared_mlp_rms_rescale((const float*)x, out, 128, 7166, nullptr) == SMLP_ERR_SHAPE);
  EXPECT(shared_mlp_shard_eligible(1, 1, 1, 8, H, I) == 1);
  EXPECT(shared_mlp_shard_eligible(1, 1, 1, 5, H, I) == 0);
  for (int s = -1; s <= 9; ++s) EXPECT(shared_mlp_status_string(s) != nullptr);
}

static void noalloc_validation() {
  void *x = fake(1ull << 40), *wgu = fake(2ull << 40), *wd = fake(3ull << 40), *out = fake(4ull << 40);
  // the M = 8192 prefill needs more than the static scratch: refused before any HIP call
  EXPECT(shared_mlp_forward_noalloc(x, wgu, wd, out, 8192, 7168, 6144, SMLP_BF16, 0, nullptr) == SMLP_ERR_WORKSPACE);
  EXPECT(shared_mlp_forward_noalloc(nullptr, wgu, wd, out, 16, 7168, 6144, SMLP_BF16, 0, nullptr) == SMLP_ERR_NULL);
  EXPECT(shared_mlp_forward_noalloc(x, wgu, wd, out, 16, 7168, 6143, SMLP_BF16, 0, nullptr) == SMLP_ERR_SHAPE);
  EXPECT(shared_mlp_forward_noalloc(x, wgu, wd, out, 0, 7168, 6144, SMLP_BF16, 0, nullptr) == SMLP_OK);
  // valid arguments reach the scratch lookup (a stand-in here, which fails)
  EXPECT(shared_mlp_forward_noalloc(x, wgu, wd, out, 16, 7168, 6144, SMLP_BF16, 0, nullptr) == SMLP_ERR_HIP);
}

static void latent_validation() {
  void *x = fake(1ull << 40), *w = fake(2ull << 40), *y = fake(3ull << 40), *ws = fake(4ull << 40);
  size_t need = 0;
  EXPECT(shared_mlp_linear_workspace_bytes(16, 7168, 2112, &need) == SMLP_OK);
  EXPECT(shared_mlp_linear(x, w, y, 16, 7168, 2112, 2112, 0, ws, need, nullptr) == SMLP_ERR_HIP);
  EXPECT(shared_mlp_linear(x, w, y, 16, 7168, 2112, 2000, 0, ws, need, nullptr) == SMLP_ERR_SHAPE);
  EXPECT(shared_mlp_linear(x, w, y, 16, 7168, 2112, 2112, 2, ws, need, nullptr) == SMLP_ERR_DTYPE);
  const int64_t sizes[] = {1536, 576};
  EXPECT(shared_mlp_restore_logical(x, y, 16, 2112, sizes, 2, 16, 2, nullptr) == SMLP_ERR_HIP);
  EXPECT(shared_mlp_restore_logical(x, y, 16, 2111, sizes, 2, 16, 2, nullptr) == SMLP_ERR_SHAPE);
  EXPECT(shared_mlp_restore_logical(x, y, 16, 2112, sizes, 2, 7, 2, nullptr) == SMLP_ERR_SHAPE);
  EXPECT(shared_mlp_restore_logical(x, y, 16, 2112, nullptr, 2, 16, 2, nullptr) == SMLP_ERR_NULL);
  EXPECT(shared_mlp_restore_logical(x, x, 16, 2112, sizes, 2, 16, 2, nullptr) == SMLP_ERR_ALIAS);
}

static void layout_models() {
  std::mt19937_64 rng(50656);
  std::uniform_real_distribution<double> U(0.0, 1.0);
  for (int n = 0; n < 300; ++n) {
    const int nr = 1 + (int)(U(rng) * 7), ns = 1 + (int)(U(rng) * 7);
    std::vector<double> rm(nr), rt(nr), sm(ns), st(ns);
    double a = 0, b = 0;
    for (int i = 0; i < nr; ++i) { a += 1 + (int)(U(rng) * 900); rm[i] = a; rt[i] = 1 + U(rng) * 500; }
    for (int i = 0; i < ns; ++i) { b += 1 + (int)(U(rng) * 900); sm[i] = b; st[i] = 1 + U(rng) * 500; }
    smlp_layout_model m{};
    m.tp = 2 << (int)(U(rng) * 3);
    m.hidden = 7168;
    m.partial_elem_bytes = U(rng) < 0.5 ? 2 : 4;
    m.alpha_us = U(rng) * 30;
    m.link_gbps = 20 + U(rng) * 300;
    m.links = 1 + (int)(U(rng) * 7);
    m.n_rep = nr; m.rep_m = rm.data(); m.rep_us = rt.data();
    m.n_shard = ns; m.shard_m = sm.data(); m.shard_us = st.data();
    double r = 0, s = 0;
    int choose = -1;
    int64_t cross = -1;
    EXPECT(shared_mlp_layout_times(&m, 1 + (int64_t)(U(rng) * 20000), &r, &s) == SMLP_OK);
    EXPECT(std::isfinite(r) && std::isfinite(s));
    EXPECT(shared_mlp_choose_layout(&m, 128, &choose) == SMLP_OK && (choose == 0 || choose == 1));
    EXPECT(shared_mlp_layout_crossover(&m, 4096, &cross) == SMLP_OK && cross >= 0 && cross <= 4096);
    m.n_rep = 0;
    EXPECT(shared_mlp_layout_times(&m, 16, &r, &s) != SMLP_OK);
  }
  EXPECT(shared_mlp_layout_times(nullptr, 16, nullptr, nullptr) != SMLP_OK);
}

static void tuning() {
  EXPECT(shared_mlp_tune_skinny(0, 3, 2, 4, 4, 3) == SMLP_OK);
  smlp_plan p;
  EXPECT(shared_mlp_plan(16, 7168, 6144, SMLP_BF16, 0, &p) == SMLP_OK && p.gate_up_ksplit == 3);
  EXPECT(shared_mlp_tune_skinny(0, 0, 0, 0, 0, 0) == SMLP_OK);
  EXPECT(shared_mlp_tune_skinny(5, 0, 0, 0, 0, 0) == SMLP_ERR_ARG);
  EXPECT(shared_mlp_tune_gemm(0, 128, 128, 4, 2, 2, 2) == SMLP_OK);
  EXPECT(shared_mlp_plan(512, 7168, 6144, SMLP_BF16, 0, &p) == SMLP_OK && p.gate_up_ksplit == 2);
  EXPECT(shared_mlp_tune_gemm(0, 0, 0, 0, 0, 0, 0) == SMLP_OK);
  EXPECT(shared_mlp_tune_gemm(0, 96, 128, 4, 2, 2, 0) == SMLP_ERR_ARG);
  EXPECT(shared_mlp_tune_h_planes(2) == SMLP_OK && shared_mlp_tune_h_planes(0) == SMLP_OK);
  EXPECT(shared_mlp_tune_h_format(3) == SMLP_OK && shared_mlp_tune_h_format(0) == SMLP_OK);
  EXPECT(shared_mlp_tune_h_format(9) == SMLP_ERR_ARG);
  EXPECT(shared_mlp_set_large_m_threshold(0) == -1);
}

static void threads() {
  // last-error strings are per thread
  std::thread t([] { smlp_plan p; shared_mlp_plan(4, 12, 16, SMLP_BF16, 0, &p); });
  smlp_plan p;
  EXPECT(shared_mlp_plan(4, 16, 16, SMLP_BF16, 0, &p) == SMLP_OK);
  t.join();
  EXPECT(std::strlen(shared_mlp_last_error()) == 0);
}

int main() {
  plans();
  forward_validation();
  noalloc_validation();
  latent_validation();
  layout_models();
  tuning();
  threads();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("sanitizer driver: all checks passed\n");
  return 0;
}
