// Adaptive block size (host code): pick K per step from running acceptance
// statistics.
//
// kongchang.com "D-Flash", "Ablations": a drafter trained on a large block
// works at smaller blocks, so the block size can be lowered with the load
// to control verification cost ("Limitations": not built there).  Google
// Developers Blog, "Scaling theory" and "Predictability": acceptance is a
// per-position probability a with positional decay, slow for math and
// code, fast for chat.
//
// Model: position i agrees with probability p_i = a gamma^i, so
//   E[tau | K] = 1 + sum_{m=1..K} prod_{i<m} a gamma^i.
// Statistics: per position, with exponential forgetting at every observed
// step, the weight of steps that reached it and of those that agreed there.
// Estimate: weighted least squares of log((agreed + 1/2) / (reached + 1))
// against the position, weights `reached`, over positions reached at least
// `min_count` times; (a, gamma) = exp of intercept and slope, clamped to
// [1e-6, 1]; the prior until two positions qualify.  Choice: the candidate
// with the largest E[tau | K] / cost(K), the smaller K on ties.
#include <math.h>

#include <vector>

#include "../../include/dflash.h"

// Records the message dflash_last_error returns (defined with the C ABI).
dflash_status dflash_set_error(dflash_status st, const char* msg);

struct dflash_adapt {
  int kmax = 0;
  double decay = 1.0, min_count = 4.0, a0 = 0.8, g0 = 0.95;
  std::vector<double> reached, agreed;
};

namespace {

double expected_tau(int K, double a, double g) {
  double e = 1.0, run = 1.0;
  for (int i = 0; i < K; ++i) {
    run *= a * pow(g, (double)i);
    e += run;
  }
  return e;
}

void estimate(const dflash_adapt* p, double* a, double* g) {
  double sw = 0, sx = 0, sy = 0, sxx = 0, sxy = 0;
  int n = 0;
  for (int i = 0; i < p->kmax; ++i) {
    const double w = p->reached[i];
    if (w < p->min_count) continue;
    const double y = log((p->agreed[i] + 0.5) / (w + 1.0));
    sw += w;
    sx += w * i;
    sy += w * y;
    sxx += w * (double)i * i;
    sxy += w * i * y;
    ++n;
  }
  if (n < 2) {
    *a = p->a0;
    *g = p->g0;
    return;
  }
  const double slope = (sw * sxy - sx * sy) / (sw * sxx - sx * sx);
  const double icpt = (sy - slope * sx) / sw;
  *a = fmin(1.0, fmax(1e-6, exp(icpt)));
  *g = fmin(1.0, fmax(1e-6, exp(slope)));
}

}  // namespace

extern "C" {

dflash_status dflash_adapt_create(int32_t kmax, double decay, double min_count, double a0, double gamma0,
                                  dflash_adapt** out) {
  if (!out) return dflash_set_error(DFLASH_E_ARG, "out is NULL");
  *out = nullptr;
  if (kmax < 1 || kmax > DFLASH_MAX_K || !(decay > 0.0 && decay <= 1.0) || !(min_count >= 0.0) ||
      !(a0 > 0.0 && a0 <= 1.0) || !(gamma0 > 0.0 && gamma0 <= 1.0))
    return dflash_set_error(DFLASH_E_ARG, "kmax in [1, DFLASH_MAX_K], decay in (0, 1], min_count >= 0 and "
                                          "a0, gamma0 in (0, 1] required");
  dflash_adapt* p = new dflash_adapt();
  p->kmax = kmax;
  p->decay = decay;
  p->min_count = min_count;
  p->a0 = a0;
  p->g0 = gamma0;
  p->reached.assign(kmax, 0.0);
  p->agreed.assign(kmax, 0.0);
  *out = p;
  return DFLASH_OK;
}

dflash_status dflash_adapt_destroy(dflash_adapt* p) {
  delete p;
  return DFLASH_OK;
}

dflash_status dflash_adapt_observe(dflash_adapt* p, int32_t K, int32_t tau) {
  if (!p) return dflash_set_error(DFLASH_E_ARG, "policy is NULL");
  if (K < 1 || K > p->kmax || tau < 1 || tau > K + 1)
    return dflash_set_error(DFLASH_E_ARG, "K must be in [1, kmax] and tau in [1, K + 1]");
  for (int i = 0; i < p->kmax; ++i) {
    p->reached[i] *= p->decay;
    p->agreed[i] *= p->decay;
  }
  const int last = tau - 1 < K - 1 ? tau - 1 : K - 1;   // last position reached
  for (int i = 0; i <= last; ++i) p->reached[i] += 1.0;
  for (int i = 0; i < tau - 1; ++i) p->agreed[i] += 1.0;
  return DFLASH_OK;
}

dflash_status dflash_adapt_choose(const dflash_adapt* p, const int32_t* Ks, const double* cost, int32_t n,
                                  int32_t* K, double* a, double* gamma, double* tokens_per_cost) {
  if (!p || n < 0 || (n > 0 && (!Ks || !cost))) return dflash_set_error(DFLASH_E_ARG, "NULL pointer or n < 0");
  for (int j = 0; j < n; ++j)
    if (Ks[j] < 1 || Ks[j] > DFLASH_MAX_K || (j > 0 && Ks[j] <= Ks[j - 1]) || !(cost[j] > 0.0) ||
        !isfinite(cost[j]))
      return dflash_set_error(DFLASH_E_ARG, "Ks must increase within [1, DFLASH_MAX_K] and costs be finite, > 0");
  double ea, eg;
  estimate(p, &ea, &eg);
  if (a) *a = ea;
  if (gamma) *gamma = eg;
  int best = n > 0 ? Ks[0] : 0;
  double best_v = -1.0;
  for (int j = 0; j < n; ++j) {
    const double v = expected_tau(Ks[j], ea, eg) / cost[j];
    if (v > best_v) {   // Ks increase: the smaller K keeps a tie
      best = Ks[j];
      best_v = v;
    }
  }
  if (K) *K = best;
  if (tokens_per_cost) *tokens_per_cost = n > 0 ? best_v : 0.0;
  return DFLASH_OK;
}

}  // extern "C"
