// Prompt-lookup (n-gram) drafting on gfx950.
//
// The drafter copies what followed the most recent earlier occurrence of the
// context's current suffix, trying the longest suffix first ("Speculative
// decoding", mhtirogla.ai, "Implementation notes"; "Speculative decoding",
// inference.tusharamrit.in, "Self-speculation").  The exact reading is in
// include/spec_ngram.h.
//
// One pass over the context finds every n at once.  For each token index t
// of a row (t <= L - 2, so a token follows), let m(t) be the number of
// tokens that agree walking back from c[t] against the suffix walking back
// from c[L-1], capped at n_max:  c[t-i] == c[L-1-i] for i < m(t).  The
// n-token suffix then ends an occurrence at t exactly when m(t) >= n, so the
// longest n with an occurrence is max_t m(t), and its most recent occurrence
// is the largest t reaching that maximum: both come out of one max over the
// key (m(t), t + 1).  The draft starts at t + 1.
//
// The work is integer compares over the context, read once: bound by HBM
// reads of 4 bytes per token.  A row is cut into chunks of kChunk tokens,
// one workgroup each; a workgroup reduces its keys in registers and LDS,
// folds its best key into the row's word with one agent-scope atomic max,
// and takes the row's arrival ticket; the last workgroup of the row reads
// the word, writes the draft and clears the row's workspace.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gamma_rule.h"
#include "spec_adapt.h"
#include "spec_ngram.h"

namespace {

// 256 threads of 8 tokens: 4 tokens or 128 / 512 threads measure the same,
// 16 or more tokens per thread leave too few waves to hide latency
constexpr int kThreads = 256;
constexpr int kTok = 8;                  // consecutive tokens per thread
constexpr int kChunk = kThreads * kTok;  // tokens per workgroup
constexpr int kHalo = SPEC_NGRAM_MAX_N;  // tokens before the chunk kept in LDS
constexpr int kRegN = 8;                 // n_max up to this: matches in registers
// Workspace words per row: {key, ticket}, padded so that rows' words lie
// 256 bytes apart; packed together, every row's atomics would queue at the
// same memory channel.
constexpr int kRowWords = 64;
// key = m << kPosBits | (t + 1): m <= 64 needs 7 bits above the position
constexpr int kPosBits = 25;
constexpr unsigned kPosMask = (1u << kPosBits) - 1;
static_assert(SPEC_NGRAM_MAX_STRIDE <= (1 << kPosBits), "position field too narrow");
static_assert(((uint64_t)SPEC_NGRAM_MAX_N << kPosBits) <= 0xffffffffull, "key overflows");
static_assert(kTok <= 32 && kTok % 4 == 0, "a thread's positions form one 32-bit mask");
static_assert(kThreads % 64 == 0 && kThreads >= kHalo, "whole waves; one thread per halo token");

struct NArgs {
  const int32_t* ctx;
  const int32_t* len;
  int B, stride, n_min, n_max, gamma, nch;
  int32_t* draft;
  int32_t* dlen;
  int32_t* dn;
  int32_t* dpos;
  unsigned* ws;  // per row: {key, ticket}
  // the draft-length rule run in the same last step (adapt != 0)
  int adapt;
  const int32_t* n_acc;
  const int32_t* g_used;
  const int32_t* active;
  double* state;
  spec_rule::GammaParams gp;
  int32_t* out_gamma;
  double* out_alpha;
};

// Batches up to this many rows run the draft-length rule inside the
// drafter: each row's last workgroup counts the batch's active rows itself.
constexpr int kFuseMaxB = 1024;

__device__ __forceinline__ unsigned wave_max(unsigned v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, o, 64));
  return v;
}

// The rule's per-row inputs, loaded by thread 0 of every workgroup when it
// starts, so that the row's last workgroup has them when it needs them.
struct RuleIn {
  int n, g, act;
  double A, T;
};

__device__ __forceinline__ RuleIn rule_inputs(const NArgs& a, int b) {
  RuleIn r{-1, 0, 1, 0.0, 0.0};
  if (!a.adapt || threadIdx.x != 0) return r;
  if (a.n_acc) r.n = a.n_acc[b], r.g = a.g_used[b];
  if (a.active) r.act = a.active[b];
  r.A = a.state[2 * b], r.T = a.state[2 * b + 1];
  return r;
}

// Writes row b's outputs from the row's best key `w` (all threads), then,
// when adapting, the row's draft length for the verify: the rule of
// spec_adapt.h capped by the draft's length.
__device__ void write_row(const NArgs& a, int b, int L, bool valid, unsigned w, int* part,
                          const RuleIn& ri) {
  const int32_t* c = a.ctx + (size_t)b * a.stride;
  const int m = (int)(w >> kPosBits);
  const int pos = (int)(w & kPosMask);
  const bool hit = valid && m >= a.n_min;
  const int len = hit ? min(a.gamma, L - pos) : 0;
  int32_t* d = a.draft + (size_t)b * a.gamma;
  for (int i = threadIdx.x; i < a.gamma; i += kThreads) d[i] = i < len ? c[pos + i] : -1;
  if (threadIdx.x == 0) {
    a.dlen[b] = len;
    if (a.dn) a.dn[b] = !valid ? -2 : hit ? m : -1;
    if (a.dpos) a.dpos[b] = hit ? pos : -1;
  }
  if (!a.adapt) return;
  int n_active = a.B;  // no mask: every row is active
  if (a.active && a.gp.batch_off >= 1) {
    int cnt = 0;
    for (int i = threadIdx.x; i < a.B; i += kThreads) cnt += a.active[i] != 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
    __syncthreads();
    n_active = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) n_active += part[i];
  }
  if (threadIdx.x == 0) {
    if (ri.act == 0) {
      a.out_gamma[b] = 0;
      if (a.out_alpha) a.out_alpha[b] = 0.0;
    } else {
      const bool off = a.gp.batch_off >= 1 && n_active >= a.gp.batch_off;
      double st[2] = {ri.A, ri.T};
      double alpha;
      const int g = spec_rule::gamma_rule(a.gp, ri.n, ri.g, st, len, off, &alpha);
      a.state[2 * b] = st[0];
      a.state[2 * b + 1] = st[1];
      if (a.out_alpha) a.out_alpha[b] = alpha;
      a.out_gamma[b] = g;
    }
  }
}

// AL: 16-byte vector loads (aligned rows).  REG: n_max <= kRegN, so every
// match length comes from a fixed set of compares over registers; otherwise
// a thread walks back through LDS where its token equals the last one.
// PRIO (the whole grid resident): staging runs at wave priority 3, the
// scan at 2 and the hand-off at 1, so that a CU's younger workgroups still
// loading their chunks get issue slots before older ones' scans.
template <bool AL, bool REG, bool PRIO>
__global__ __launch_bounds__(kThreads) void ngram_kernel(NArgs a) {
  __shared__ int sfx[SPEC_NGRAM_MAX_N];  // sfx[i] = c[L-1-i]
  __shared__ __align__(16) int tok[kHalo + kChunk];  // c[cbase - kHalo .. cbase + kChunk)
  __shared__ unsigned red[kThreads / 64];
  __shared__ int part[kThreads / 64];
  __shared__ unsigned win;
  __shared__ int last_wg;

  if (PRIO) __builtin_amdgcn_s_setprio(3);
  const int b = blockIdx.x % a.B;
  const int k = blockIdx.x / a.B;
  const int tid = threadIdx.x;
  const int32_t* c = a.ctx + (size_t)b * a.stride;
  const int cbase = k * kChunk;
  const int base = cbase + tid * kTok;
  const int L = a.len[b];
  const bool valid = L >= 0 && L <= a.stride;
  const RuleIn ri = rule_inputs(a, b);
  const int last = L - 2;  // largest t with a token after it
  const bool active = valid && cbase <= last;
  // The suffix and the chunk load side by side, both after the length.
  const int nsfx = valid ? min(a.n_max, L) : 0;
  if (tid < SPEC_NGRAM_MAX_N) sfx[tid] = tid < nsfx ? c[L - 1 - tid] : 0;
  // Stage the chunk's tokens up to L - 2 and the kHalo tokens before it.
  // Entries past L - 2 or before the row are never compared (the position
  // mask and the match cap exclude them).
  if (active) {
    int v[kTok];
    if (AL && base + kTok - 1 <= last) {
#pragma unroll
      for (int q = 0; q < kTok; q += 4) {
        const int4 x = *reinterpret_cast<const int4*>(c + base + q);
        v[q] = x.x; v[q + 1] = x.y; v[q + 2] = x.z; v[q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTok; ++i) v[i] = base + i <= last ? c[base + i] : 0;
    }
#pragma unroll
    for (int q = 0; q < kTok; q += 4)
      *reinterpret_cast<int4*>(&tok[kHalo + tid * kTok + q]) = make_int4(v[q], v[q + 1], v[q + 2], v[q + 3]);
    if (tid < kHalo) {
      const int g = cbase - kHalo + tid;
      tok[tid] = g >= 0 ? c[g] : 0;
    }
  }
  __syncthreads();
  if (PRIO) __builtin_amdgcn_s_setprio(2);

  unsigned best = 0;
  if (active && base <= last) {
    const int* w = &tok[kHalo + tid * kTok];  // w[i] = c[base + i], i >= -kHalo
    if (REG) {
      int x[kRegN + kTok];  // x[kRegN + i] = c[base + i]
#pragma unroll
      for (int q = 0; q < kRegN + kTok; q += 4) {
        const int4 y = *reinterpret_cast<const int4*>(w - kRegN + q);
        x[q] = y.x; x[q + 1] = y.y; x[q + 2] = y.z; x[q + 3] = y.w;
      }
      // Level j compares every position's token j back with the suffix's
      // token j back, as a bit mask over the thread's kTok positions; R keeps
      // the positions whose first j+1 tokens all agree.  The deepest level
      // with a position left gives m, its highest bit the latest t.  Lanes
      // leave as soon as R empties, which for most tokens is after level 0.
      const int nok = min(last - base + 1, kTok);  // positions t <= L - 2
      unsigned R = nok >= 32 ? ~0u : (1u << nok) - 1u;
      unsigned Rm = 0;
      int m = 0;
#pragma unroll
      for (int j = 0; j < kRegN; ++j) {
        if (j >= a.n_max) break;
        const int sj = sfx[j];
        unsigned M = 0;
#pragma unroll
        for (int i = 0; i < kTok; ++i) M |= x[kRegN + i - j] == sj ? 1u << i : 0u;
        // positions whose token j back lies before the row's start
        if (j > base) M &= ~0u << (j - base);
        R &= M;
        if (R == 0) break;
        Rm = R;
        m = j + 1;
      }
      if (m) best = ((unsigned)m << kPosBits) | (unsigned)(base + (31 - __clz(Rm)) + 1);
    } else {
      const int s0 = sfx[0];
      for (int i = 0; i < kTok; ++i) {
        const int t = base + i;
        if (t <= last && w[i] == s0) {
          const int cap = min(a.n_max, t + 1);
          int m = 1;
          while (m < cap && w[i - m] == sfx[m]) ++m;
          best = max(best, ((unsigned)m << kPosBits) | (unsigned)(t + 1));
        }
      }
    }
  }

  best = wave_max(best);
  if ((tid & 63) == 0) red[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    unsigned w = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) w = max(w, red[i]);
    int fin = 1;
    if (a.nch > 1) {
      unsigned* key = a.ws + kRowWords * b;
      unsigned* ticket = key + 1;
      // the max must be performed before this workgroup counts itself in:
      // waiting for its returned value orders the two atomics
      unsigned prev = 0;
      if (w) prev = __hip_atomic_fetch_max(key, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("" ::"v"(prev) : "memory");
      const unsigned arrived =
          __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("" ::"v"(arrived) : "memory");
      fin = arrived == (unsigned)(a.nch - 1);
      if (fin) {
        // every other workgroup's max was performed before its ticket
        w = __hip_atomic_load(key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::"v"(w) : "memory");
        __hip_atomic_store(key, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    win = w;
    last_wg = fin;
  }
  __syncthreads();
  if (last_wg) write_row(a, b, L, valid, win, part, ri);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Checks the drafting arguments and fills `a` (the rule's fields zero).
int ngram_args(const int32_t* context, const int32_t* ctx_len, int B, int stride, int n_min,
               int n_max, int gamma, int32_t* out_draft, int32_t* out_len, int32_t* out_n,
               int32_t* out_pos, void* workspace, size_t workspace_bytes, NArgs& a) {
  if (B < 0 || stride < 0 || stride > SPEC_NGRAM_MAX_STRIDE) return SPEC_ERR_SHAPE;
  if (n_min < 1 || n_max < n_min || n_max > SPEC_NGRAM_MAX_N) return SPEC_ERR_ARG;
  if (gamma < 0 || gamma > SPEC_NGRAM_MAX_GAMMA) return SPEC_ERR_ARG;
  if (B == 0) return SPEC_OK;
  if ((stride > 0 && !context) || !ctx_len || !out_len || (gamma > 0 && !out_draft))
    return SPEC_ERR_NULL;
  const int nch = stride > 0 ? (stride + kChunk - 1) / kChunk : 1;
  if ((int64_t)B * nch > 0x7fffffff) return SPEC_ERR_SHAPE;
  for (const void* p : {(const void*)context, (const void*)ctx_len, (const void*)out_draft,
                        (const void*)out_len, (const void*)out_n, (const void*)out_pos})
    if (p && !aligned(p, 4)) return SPEC_ERR_ALIGN;
  if (nch > 1) {
    if (!workspace || workspace_bytes < spec_ngram_workspace_bytes(B)) return SPEC_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SPEC_ERR_ALIGN;
  }
  a = NArgs{};
  a.ctx = context, a.len = ctx_len, a.B = B, a.stride = stride, a.n_min = n_min;
  a.n_max = n_max, a.gamma = gamma, a.nch = nch, a.draft = out_draft, a.dlen = out_len;
  a.dn = out_n, a.dpos = out_pos, a.ws = static_cast<unsigned*>(workspace);
  return SPEC_OK;
}

// Compute units of the calling thread's current device, asked once per
// device (0 if the runtime cannot tell).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64 && n > 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <bool PRIO>
void launch_variant(bool al, bool reg, dim3 grid, hipStream_t s, const NArgs& a) {
  if (al && reg)
    hipLaunchKernelGGL((ngram_kernel<true, true, PRIO>), grid, dim3(kThreads), 0, s, a);
  else if (al)
    hipLaunchKernelGGL((ngram_kernel<true, false, PRIO>), grid, dim3(kThreads), 0, s, a);
  else if (reg)
    hipLaunchKernelGGL((ngram_kernel<false, true, PRIO>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((ngram_kernel<false, false, PRIO>), grid, dim3(kThreads), 0, s, a);
}

int ngram_launch(const NArgs& a, void* stream) {
  const bool al = aligned(a.ctx, 16) && a.stride % 4 == 0;
  const dim3 grid((unsigned)(a.B * a.nch));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool reg = a.n_max <= kRegN;
  // wave priorities only when every workgroup is resident from the start
  const int cus = device_cus();
  if (cus > 0 && (int64_t)a.B * a.nch <= (int64_t)4 * cus)
    launch_variant<true>(al, reg, grid, s, a);
  else
    launch_variant<false>(al, reg, grid, s, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP - (int)e;
}

}  // namespace

extern "C" size_t spec_ngram_workspace_bytes(int B) {
  if (B < 1) return 0;
  return ((size_t)B * kRowWords * sizeof(unsigned) + 255) / 256 * 256;
}

extern "C" int spec_ngram_draft(const int32_t* context, const int32_t* ctx_len, int B, int stride,
                                int n_min, int n_max, int gamma, int32_t* out_draft,
                                int32_t* out_len, int32_t* out_n, int32_t* out_pos,
                                void* workspace, size_t workspace_bytes, void* stream) {
  NArgs a;
  const int rc = ngram_args(context, ctx_len, B, stride, n_min, n_max, gamma, out_draft, out_len,
                            out_n, out_pos, workspace, workspace_bytes, a);
  if (rc != SPEC_OK || B == 0) return rc;
  return ngram_launch(a, stream);
}

extern "C" int spec_ngram_draft_adaptive(
    const int32_t* context, const int32_t* ctx_len, int B, int stride, int n_min, int n_max,
    int gamma, const int32_t* n_accepted, const int32_t* gamma_used, const int32_t* active,
    double* state, double decay, double prior_alpha, double prior_weight, double draft_cost,
    int batch_off, int32_t* out_draft, int32_t* out_len, int32_t* out_n, int32_t* out_pos,
    int32_t* out_gamma, double* out_alpha, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (gamma > SPEC_GAMMA_MAX_LIMIT) return SPEC_ERR_ARG;
  if (!spec_rule::gamma_params_ok(decay, prior_alpha, prior_weight, draft_cost, batch_off))
    return SPEC_ERR_ARG;
  NArgs a;
  const int rc = ngram_args(context, ctx_len, B, stride, n_min, n_max, gamma, out_draft, out_len,
                            out_n, out_pos, workspace, workspace_bytes, a);
  if (rc != SPEC_OK || B == 0) return rc;
  if (!state || !out_gamma || (n_accepted == nullptr) != (gamma_used == nullptr))
    return SPEC_ERR_NULL;
  for (const void* p : {(const void*)n_accepted, (const void*)gamma_used, (const void*)active,
                        (const void*)out_gamma})
    if (p && !aligned(p, 4)) return SPEC_ERR_ALIGN;
  if (!aligned(state, 8) || (out_alpha && !aligned(out_alpha, 8))) return SPEC_ERR_ALIGN;
  if (B > kFuseMaxB) {
    // large batches: the drafter, then the controller over its lengths
    const int r1 = ngram_launch(a, stream);
    if (r1 != SPEC_OK) return r1;
    return spec_gamma_control(n_accepted, gamma_used, active, out_len, state, B, gamma, decay,
                              prior_alpha, prior_weight, draft_cost, batch_off, out_gamma,
                              out_alpha, stream);
  }
  a.adapt = 1;
  a.n_acc = n_accepted, a.g_used = gamma_used, a.active = active, a.state = state;
  a.gp = spec_rule::GammaParams{gamma, decay, prior_alpha, prior_weight, draft_cost, batch_off};
  a.out_gamma = out_gamma, a.out_alpha = out_alpha;
  return ngram_launch(a, stream);
}
