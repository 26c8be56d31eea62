// Adaptive draft length on gfx950: each request's next draft length from its
// running acceptance, speculation off at large batch.  The rule and its
// sources are in include/spec_adapt.h.
//
// The work is a few fp64 operations per row and at most gamma_max steps of
// the E(gamma) / (1 + gamma c) search (gamma_rule.h), so one workgroup does
// the whole batch: it counts the active rows (the switch-off needs the
// batch's total), then every thread decides its rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gamma_rule.h"
#include "spec_adapt.h"

namespace {

constexpr int kThreads = 1024;

struct GArgs {
  const int32_t* n_acc;
  const int32_t* g_used;
  const int32_t* active;
  const int32_t* limit;
  double* state;
  int B;
  spec_rule::GammaParams p;
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
  const bool off = a.p.batch_off >= 1 && n_active >= a.p.batch_off;

  for (int b = tid; b < a.B; b += kThreads) {
    if (a.active && a.active[b] == 0) {
      a.out_gamma[b] = 0;
      if (a.out_alpha) a.out_alpha[b] = 0.0;
      continue;
    }
    double st[2] = {a.state[2 * b], a.state[2 * b + 1]};
    double alpha;
    const int g = spec_rule::gamma_rule(a.p, a.n_acc ? a.n_acc[b] : -1, a.g_used ? a.g_used[b] : 0,
                                        st, a.limit ? a.limit[b] : a.p.gamma_max, off, &alpha);
    a.state[2 * b] = st[0];
    a.state[2 * b + 1] = st[1];
    if (a.out_alpha) a.out_alpha[b] = alpha;
    a.out_gamma[b] = g;
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
  if (!spec_rule::gamma_params_ok(decay, prior_alpha, prior_weight, draft_cost, batch_off))
    return SPEC_ERR_ARG;
  if (B == 0) return SPEC_OK;
  if (!state || !out_gamma || (n_accepted == nullptr) != (gamma_used == nullptr))
    return SPEC_ERR_NULL;
  for (const void* p : {(const void*)n_accepted, (const void*)gamma_used, (const void*)active,
                        (const void*)gamma_limit, (const void*)out_gamma})
    if (p && !aligned(p, 4)) return SPEC_ERR_ALIGN;
  if (!aligned(state, 8) || (out_alpha && !aligned(out_alpha, 8))) return SPEC_ERR_ALIGN;
  GArgs a{n_accepted, gamma_used, active, gamma_limit, state, B,
          spec_rule::GammaParams{gamma_max, decay, prior_alpha, prior_weight, draft_cost, batch_off},
          out_gamma, out_alpha};
  hipLaunchKernelGGL(gamma_kernel, dim3(1), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP - (int)e;
}
