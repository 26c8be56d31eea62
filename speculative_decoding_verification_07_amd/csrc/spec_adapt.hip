// Adaptive draft length on gfx950: each request's next draft length from its
// running acceptance, speculation off at large batch.  The rule and its
// sources are in include/spec_adapt.h.
//
// The work is a few fp64 operations per row and at most gamma_max steps of
// the E(gamma) / (1 + gamma c) search, so one workgroup does the whole batch:
// it counts the active rows (the switch-off needs the batch's total), then
// every thread decides its rows.  The operations and their order are the
// rule's, in fp64 and built with -ffp-contract=off, so the results are
// bit-for-bit those of any IEEE double implementation of the same steps.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spec_adapt.h"

namespace {

constexpr int kThreads = 1024;

struct GArgs {
  const int32_t* n_acc;
  const int32_t* g_used;
  const int32_t* active;
  const int32_t* limit;
  double* state;
  int B, gamma_max;
  double decay, prior_alpha, prior_weight, cost;
  int batch_off;
  int32_t* out_gamma;
  double* out_alpha;
};

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(kThreads) void gamma_kernel(GArgs a) {
  __shared__ int part[kThreads / 64];
  const int tid = threadIdx.x;
  int cnt = 0;
  for (int b = tid; b < a.B; b += kThreads) cnt += !a.active || a.active[b] != 0;
  cnt = wave_sum(cnt);
  if ((tid & 63) == 0) part[tid >> 6] = cnt;
  __syncthreads();
  int n_active = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) n_active += part[i];
  const bool off = a.batch_off >= 1 && n_active >= a.batch_off;

  for (int b = tid; b < a.B; b += kThreads) {
    if (a.active && a.active[b] == 0) {
      a.out_gamma[b] = 0;
      if (a.out_alpha) a.out_alpha[b] = 0.0;
      continue;
    }
    double A = a.state[2 * b], T = a.state[2 * b + 1];
    const int g = a.g_used ? a.g_used[b] : 0;
    const int n = a.n_acc ? a.n_acc[b] : -1;
    if (g >= 1 && n >= 0 && n <= g) {
      const int tested = n + 1 < g ? n + 1 : g;
      A = a.decay * A + (double)n;
      T = a.decay * T + (double)tested;
    } else {
      A = a.decay * A;
      T = a.decay * T;
    }
    a.state[2 * b] = A;
    a.state[2 * b + 1] = T;
    const double den = T + a.prior_weight;
    const double alpha = den > 0.0 ? (A + a.prior_weight * a.prior_alpha) / den : a.prior_alpha;
    if (a.out_alpha) a.out_alpha[b] = alpha;
    int best = 0;
    if (!off) {
      int cap = a.gamma_max;
      if (a.limit && a.limit[b] < cap) cap = a.limit[b] < 0 ? 0 : a.limit[b];
      double best_e = 1.0, pw = 1.0, e = 1.0;
      for (int k = 1; k <= cap; ++k) {
        pw = pw * alpha;
        e = e + pw;
        if (e * (1.0 + (double)best * a.cost) > best_e * (1.0 + (double)k * a.cost)) {
          best = k;
          best_e = e;
        }
      }
    }
    a.out_gamma[b] = best;
  }
}

bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

}  // namespace

extern "C" int spec_gamma_control(const int32_t* n_accepted, const int32_t* gamma_used,
                                  const int32_t* active, const int32_t* gamma_limit, double* state,
                                  int B, int gamma_max, double decay, double prior_alpha,
                                  double prior_weight, double draft_cost, int batch_off,
                                  int32_t* out_gamma, double* out_alpha, void* stream) {
  if (B < 0 || gamma_max < 0 || gamma_max > SPEC_GAMMA_MAX_LIMIT) return SPEC_ERR_SHAPE;
  if (!(decay >= 0.0 && decay <= 1.0) || !(prior_alpha >= 0.0 && prior_alpha <= 1.0))
    return SPEC_ERR_ARG;
  if (!(prior_weight >= 0.0) || !isfinite(prior_weight) || !(draft_cost >= 0.0) ||
      !isfinite(draft_cost) || batch_off < 0)
    return SPEC_ERR_ARG;
  if (B == 0) return SPEC_OK;
  if (!state || !out_gamma || (n_accepted == nullptr) != (gamma_used == nullptr))
    return SPEC_ERR_NULL;
  for (const void* p : {(const void*)n_accepted, (const void*)gamma_used, (const void*)active,
                        (const void*)gamma_limit, (const void*)out_gamma})
    if (p && !aligned(p, 4)) return SPEC_ERR_ALIGN;
  if (!aligned(state, 8) || (out_alpha && !aligned(out_alpha, 8))) return SPEC_ERR_ALIGN;
  GArgs a{n_accepted, gamma_used, active, gamma_limit, state, B, gamma_max, decay, prior_alpha,
          prior_weight, draft_cost, batch_off, out_gamma, out_alpha};
  hipLaunchKernelGGL(gamma_kernel, dim3(1), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP - (int)e;
}
