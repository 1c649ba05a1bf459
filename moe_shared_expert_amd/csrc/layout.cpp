// Per-step replicated-vs-sharded choice (host only): measured kernel curves plus a
// latency-bandwidth model of the all-gather and reduce-scatter around the sharded MLP
// (vLLM PR 50656, "[Kimi-K3] Add option to shard the shared expert instead of
// replicating", sections Change, Trade-off and why it is opt-in, Evaluation).
#include <cmath>

#include "smlp.h"
#include "smlp_layout.h"

namespace smlp {
int set_error(int status, const char* msg);  // api.cpp
}

namespace {

bool curve_ok(int n, const double* m, const double* t) {
  if (n < 1 || !m || !t) return false;
  for (int i = 0; i < n; ++i) {
    if (!std::isfinite(m[i]) || !std::isfinite(t[i]) || t[i] < 0) return false;
    if (i > 0 && !(m[i] > m[i - 1])) return false;
  }
  return true;
}

int check(const smlp_layout_model* md) {
  if (!md) return smlp::set_error(SMLP_ERR_NULL, "model is NULL");
  if (md->tp < 2 || md->hidden < 1 || (md->partial_elem_bytes != 2 && md->partial_elem_bytes != 4) ||
      !(md->alpha_us >= 0) || !std::isfinite(md->alpha_us) || !(md->link_gbps > 0) ||
      !std::isfinite(md->link_gbps) || md->links < 1)
    return smlp::set_error(SMLP_ERR_ARG,
                           "layout model needs tp >= 2, hidden >= 1, partial_elem_bytes 2 or 4, "
                           "alpha_us >= 0, link_gbps > 0, links >= 1");
  if (!curve_ok(md->n_rep, md->rep_m, md->rep_us) || !curve_ok(md->n_shard, md->shard_m, md->shard_us))
    return smlp::set_error(SMLP_ERR_ARG,
                           "kernel curves need >= 1 finite point, strictly increasing M, times >= 0");
  return SMLP_OK;
}

// Piecewise-linear curve: first value below the first point, last segment extended
// above the last point, never below the last value.
double curve(int n, const double* m, const double* t, double x) {
  if (n == 1 || x <= m[0]) return t[0];
  for (int i = 0; i + 1 < n; ++i)
    if (x <= m[i + 1]) return t[i] + (t[i + 1] - t[i]) * ((x - m[i]) / (m[i + 1] - m[i]));
  const double slope = (t[n - 1] - t[n - 2]) / (m[n - 1] - m[n - 2]);
  const double v = t[n - 1] + slope * (x - m[n - 1]);
  return v > t[n - 1] ? v : t[n - 1];
}

// One all-gather or reduce-scatter of T token rows: a chunk of ceil(T / tp) rows to or
// from each of the tp - 1 peers, ceil((tp - 1) / links) chunks per link.
double collective(const smlp_layout_model* md, int64_t T, int elem) {
  const int64_t rows = (T + md->tp - 1) / md->tp;
  const int64_t rounds = (md->tp - 1 + md->links - 1) / md->links;
  const double chunk = (double)rows * (double)md->hidden * (double)elem;
  return md->alpha_us + (double)rounds * chunk / (md->link_gbps * 1e3);
}

void times(const smlp_layout_model* md, int64_t T, double* t_rep, double* t_shard) {
  const int64_t m_rep = (T + md->tp - 1) / md->tp;
  *t_rep = curve(md->n_rep, md->rep_m, md->rep_us, (double)m_rep);
  *t_shard = curve(md->n_shard, md->shard_m, md->shard_us, (double)T) + collective(md, T, 2) +
             collective(md, T, md->partial_elem_bytes);
}

}  // namespace

extern "C" {

int shared_mlp_layout_times(const smlp_layout_model* model, int64_t T, double* t_rep_us,
                            double* t_shard_us) {
  int rc = check(model);
  if (rc) return rc;
  if (!t_rep_us || !t_shard_us) return smlp::set_error(SMLP_ERR_NULL, "output pointer is NULL");
  if (T < 1 || T > ((int64_t)1 << 40)) return smlp::set_error(SMLP_ERR_ARG, "T outside [1, 2^40]");
  times(model, T, t_rep_us, t_shard_us);
  return smlp::set_error(SMLP_OK, "");
}

int shared_mlp_choose_layout(const smlp_layout_model* model, int64_t T, int* sharded) {
  if (!sharded) return smlp::set_error(SMLP_ERR_NULL, "sharded is NULL");
  double r, s;
  int rc = shared_mlp_layout_times(model, T, &r, &s);
  if (rc) return rc;
  *sharded = s < r ? 1 : 0;
  return SMLP_OK;
}

int shared_mlp_layout_crossover(const smlp_layout_model* model, int64_t T_max, int64_t* T_cross) {
  int rc = check(model);
  if (rc) return rc;
  if (!T_cross) return smlp::set_error(SMLP_ERR_NULL, "T_cross is NULL");
  if (T_max < 1 || T_max > ((int64_t)1 << 24)) return smlp::set_error(SMLP_ERR_ARG, "T_max outside [1, 2^24]");
  *T_cross = 0;
  for (int64_t T = 1; T <= T_max; ++T) {
    double r, s;
    times(model, T, &r, &s);
    if (!(s < r)) {
      *T_cross = T;
      break;
    }
  }
  return smlp::set_error(SMLP_OK, "");
}

}  // extern "C"
