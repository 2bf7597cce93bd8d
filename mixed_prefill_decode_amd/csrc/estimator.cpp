// Fitting the iteration-latency estimator from profiles (host only).
//
// ConfluxServe §6.2 ("Estimator construction") and App. D: each base function
// is affine in its dominant workload metric -- f_GEMM(n) (Eq. 7) in the
// rank-local tokens, f_D(W) (Eq. 8) in the aggregate decode context, f_P(W)
// (Eq. 10) in the per-rank causal-attention workload of Eq. 9, f_comm(n)
// (Eq. 11) in the largest prefill shard -- with coefficients fitted from
// profiles of each part in isolation; the contention factors alpha and beta of
// Eq. 4 are then calibrated on heterogeneous iterations.
//
// Readings: the pages name no loss, and their accuracy figure is a mean
// absolute percentage error, so every fit minimizes squared relative error.
// alpha and beta come from a grid of step 1/64 (exhaustive, so the fit has no
// starting point to depend on).
#pragma clang fp contract(off)

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/xp.h"

namespace xp {
xp_status fail(xp_status code, const char* fmt, ...);
}
using xp::fail;

namespace {

xp_status check_samples(const xp_samples* s, const char* what) {
  if (!s || s->n < 0) return fail(XP_EINVAL, "%s samples: null or negative count", what);
  if (s->n > 0 && (!s->x || !s->t)) return fail(XP_EINVAL, "%s samples: null array", what);
  for (int i = 0; i < s->n; ++i)
    if (!(s->t[i] > 0.0) || !isfinite(s->t[i]) || !isfinite(s->x[i]))
      return fail(XP_EINVAL, "%s samples: t[%d] <= 0 or not finite", what, i);
  return XP_OK;
}

// min over (a, b) of sum_i (a u_i + b v_i - 1)^2 with u = x/t, v = 1/t.  The two
// columns are scaled to unit norm before the 2x2 normal equations are solved, so
// workload metrics of very different magnitudes stay well conditioned.
void affine(int n, const double* x, const double* t, double* slope, double* icpt) {
  *slope = 0.0;
  *icpt = 0.0;
  if (n == 0) return;
  bool same = true;
  for (int i = 1; i < n; ++i) same = same && x[i] == x[0];
  double svv = 0.0, sv = 0.0;
  for (int i = 0; i < n; ++i) {
    const double v = 1.0 / t[i];
    svv += v * v;
    sv += v;
  }
  if (same) {  // intercept only: b = sum v / sum v^2
    *icpt = sv / svv;
    return;
  }
  double suu = 0.0;
  for (int i = 0; i < n; ++i) {
    const double u = x[i] / t[i];
    suu += u * u;
  }
  const double nu = sqrt(suu), nv = sqrt(svv);
  double a11 = 0.0, a12 = 0.0, r1 = 0.0, r2 = 0.0;
  for (int i = 0; i < n; ++i) {
    const double u = x[i] / t[i] / nu, v = 1.0 / t[i] / nv;
    a11 += u * u;
    a12 += u * v;
    r1 += u;
    r2 += v;
  }
  const double a22 = 1.0;
  const double det = a11 * a22 - a12 * a12;
  if (!(det > 1e-15)) {  // numerically one column: intercept only
    *icpt = sv / svv;
    return;
  }
  const double p = (r1 * a22 - a12 * r2) / det, q = (a11 * r2 - a12 * r1) / det;
  *slope = p / nu;
  *icpt = q / nv;
}

}  // namespace

extern "C" {

xp_status xp_fit_affine(const xp_samples* s, double* slope, double* intercept) {
  xp_status st = check_samples(s, "xp_fit_affine");
  if (st) return st;
  if (!slope || !intercept) return fail(XP_EINVAL, "xp_fit_affine: null output");
  affine(s->n, s->x, s->t, slope, intercept);
  return XP_OK;
}

xp_status xp_fit_latency_model(const xp_samples* gemm, const xp_samples* decode, const xp_samples* prefill,
                               const xp_samples* comm, const xp_mixed_samples* mixed, int32_t n_layers,
                               double ab_max, xp_latency_model* out) {
  xp_status st;
  if ((st = check_samples(gemm, "gemm")) || (st = check_samples(decode, "decode")) ||
      (st = check_samples(prefill, "prefill")) || (st = check_samples(comm, "comm")))
    return st;
  if (!mixed || mixed->n < 0 || !out) return fail(XP_EINVAL, "xp_fit_latency_model: null mixed / out");
  if (mixed->n > 0 && (!mixed->gemm_x || !mixed->decode_x || !mixed->prefill_x || !mixed->comm_x || !mixed->t))
    return fail(XP_EINVAL, "xp_fit_latency_model: null mixed array");
  for (int j = 0; j < mixed->n; ++j)
    if (!(mixed->t[j] > 0.0) || !isfinite(mixed->t[j]))
      return fail(XP_EINVAL, "xp_fit_latency_model: mixed t[%d] <= 0", j);
  if (n_layers < 1 || !(ab_max >= 1.0 && ab_max <= 16.0))
    return fail(XP_EINVAL, "xp_fit_latency_model: n_layers %d / ab_max", n_layers);

  xp_latency_model m{};
  affine(gemm->n, gemm->x, gemm->t, &m.gamma, &m.gamma0);
  affine(decode->n, decode->x, decode->t, &m.a_d, &m.a_d0);
  affine(prefill->n, prefill->x, prefill->t, &m.a_p, &m.a_p0);
  affine(comm->n, comm->x, comm->t, &m.a_comm, &m.a_comm0);
  m.n_layers = n_layers;

  // per-iteration terms of Eq. 3, 5, 6 under the fitted base functions
  const int J = mixed->n;
  std::vector<double> tg(J), tp(J), td(J);
  for (int j = 0; j < J; ++j) {
    tg[j] = m.gamma * mixed->gemm_x[j] + m.gamma0;
    td[j] = mixed->decode_x[j] >= 0.0 ? m.a_d * mixed->decode_x[j] + m.a_d0 : 0.0;
    tp[j] = mixed->prefill_x[j] >= 0.0
                ? (m.a_comm * mixed->comm_x[j] + m.a_comm0) + (m.a_p * mixed->prefill_x[j] + m.a_p0)
                : 0.0;
  }
  const int K = int(floor((ab_max - 1.0) * 64.0 + 1e-9));
  double best = INFINITY;
  m.alpha = m.beta = 1.0;
  for (int ka = 0; ka <= K; ++ka) {
    const double alpha = 1.0 + ka / 64.0;
    for (int kb = 0; kb <= K; ++kb) {
      const double beta = 1.0 + kb / 64.0;
      double err = 0.0;
      for (int j = 0; j < J; ++j) {
        const double pred = double(n_layers) * (tg[j] + std::max(beta * tp[j], alpha * td[j]));
        const double e = pred / mixed->t[j] - 1.0;
        err += e * e;
      }
      if (err < best) {
        best = err;
        m.alpha = alpha;
        m.beta = beta;
      }
    }
  }
  *out = m;
  return XP_OK;
}

}  // extern "C"
