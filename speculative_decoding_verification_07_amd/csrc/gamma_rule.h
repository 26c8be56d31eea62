// The adaptive draft-length rule for one request (include/spec_adapt.h
// states it and its sources), shared by the controller kernel and the
// drafter that runs it in its last step.  All arithmetic is fp64 in the
// rule's order; the library is built with -ffp-contract=off, so every result
// is the IEEE value of these operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec_rule {

struct GammaParams {
  int gamma_max;
  double decay, prior_alpha, prior_weight, cost;
  int batch_off;
};

// Row b's update and choice.  n, g: the previous round's accepted count
// and draft length (g = 0 or n outside [0, g]: no observation); st: the
// row's {A, T}, updated in place; limit: the row's cap (negative = 0);
// off: speculation is off for the batch.  Returns gamma; *alpha_out gets the
// running acceptance.
__device__ inline int gamma_rule(const GammaParams& p, int n, int g, double* st, int limit,
                                 bool off, double* alpha_out) {
  double A = st[0], T = st[1];
  if (g >= 1 && n >= 0 && n <= g) {
    const int tested = n + 1 < g ? n + 1 : g;
    A = p.decay * A + (double)n;
    T = p.decay * T + (double)tested;
  } else {
    A = p.decay * A;
    T = p.decay * T;
  }
  st[0] = A;
  st[1] = T;
  const double den = T + p.prior_weight;
  const double alpha = den > 0.0 ? (A + p.prior_weight * p.prior_alpha) / den : p.prior_alpha;
  *alpha_out = alpha;
  if (off) return 0;
  int cap = p.gamma_max;
  if (limit < cap) cap = limit < 0 ? 0 : limit;
  // E(0) = 1, E(k) = E(k-1) + alpha^k; k beats the best j so far when
  // E(k) (1 + j c) > E(j) (1 + k c)
  double best_e = 1.0, pw = 1.0, e = 1.0;
  int best = 0;
  for (int k = 1; k <= cap; ++k) {
    pw = pw * alpha;
    e = e + pw;
    if (e * (1.0 + (double)best * p.cost) > best_e * (1.0 + (double)k * p.cost)) {
      best = k;
      best_e = e;
    }
  }
  return best;
}

// Host-side argument check shared by the entry points.
inline bool gamma_params_ok(double decay, double prior_alpha, double prior_weight, double cost,
                            int batch_off) {
  return decay >= 0.0 && decay <= 1.0 && prior_alpha >= 0.0 && prior_alpha <= 1.0 &&
         prior_weight >= 0.0 && prior_weight <= 1.7976931348623157e308 && cost >= 0.0 &&
         cost <= 1.7976931348623157e308 && batch_off >= 0;
}

}  // namespace spec_rule
