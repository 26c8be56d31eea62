// spec_verify.hip -- batched speculative-decoding verify step for MI355X (gfx950).
//
// One launch does the whole step.  Its workgroups are of two kinds, laid out
// in blockIdx order:
//
//   statistics items (b, r, c): chunk c of vocabulary row r of batch row b.
//     Streams the chunk from HBM with 16-byte loads and reduces it to the
//     online-softmax pair (m, S) = (max logit, sum 2^((l - m) log2e / T))
//     -- or, greedy, to (max, lowest argmax) -- then writes the pair to the
//     workspace and takes a ticket on the row.  The item that takes the
//     row's last ticket merges the row's pairs, gathers t[x_i] and d[x_i],
//     runs the acceptance test u * q < p for every position at once, finds
//     the first rejection with a wave ballot, writes the row's outputs and
//     publishes the row's decision.
//   draw items (b, s): slice s of the one or two vocabulary rows the row
//     draws from (the residual max(0, p_n - q_n) after a rejection at n, or
//     p_g for the bonus).  Each waits for its row's decision, sums its
//     slice's weights and takes a ticket; the last one prefix-sums the slice
//     totals, finds the slice holding tau = u * Z, re-reads that slice and
//     finds the token with a block prefix scan.
//
// Draw items of row k sit after the statistics items of row k + lag, so they
// rarely wait.  They wait only on items with smaller workgroup ids (the
// dispatcher issues ids in increasing order on each XCD), so every wait ends;
// a bounded spin backs that up.  Counters reset themselves, so the workspace
// is left zero after each call.
//
// Method: "Speculative decoding" (mhtirogla.ai), "How it works" steps 2-5
// and "Code"; blog.lo0.es, "The bare mechanism" step 3; tusharamrit, the
// loop and the modified rejection-sampling rule; tokentrails, steps 2 and 4.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;            // 16-byte loads in flight per thread
constexpr int kSub = kThreads;        // draw: elements per sub-slice
constexpr int kMaxSubs = 64;          // draw: sub-slices per slice
constexpr unsigned kFlagStats = 1u, kFlagNone = 2u;  // row flag values
constexpr unsigned kDiagSpin = 1u, kDiagZeroResid = 2u;
// Per-row counters (statistics ticket, draw ticket, row flag) each sit on
// their own 256-byte line.  The row blocks are laid out downwards from the
// end of the workspace, so a counter's address depends only on the workspace
// (pointer and size) and the row, never on the call's sizes: calls of any
// shape can share a workspace, and none finds another call's data where its
// counters belong.
constexpr int kCounterStride = 64;                   // unsigned words per counter line
constexpr int kRowBlock = 3 * kCounterStride;        // words per row block
constexpr size_t kRowBlockBytes = kRowBlock * sizeof(unsigned);
#define NEG_INF (-__builtin_inff())

struct Tuning {
  int chunk_bytes = 65536;
  int slice_elems = 8192;
  int lag_rows = 0;  // 0: derived from the plan
};
// Draw items of row k follow the statistics of row k + lag: about this many
// statistics workgroups run ahead of a row's draws (measured best on MI355X
// for 64-256 rows at V = 128K-152K).
constexpr int kLeadWorkgroups = 600;
Tuning g_tune;

// ------------------------------------------------------------------ plan
struct Plan {
  int B, G, V, dtype, mode;
  int NR;        // vocabulary rows per batch row
  int NC, CH;    // statistics chunks per vocabulary row, chunk length
  int ND, SL;    // draw slices per batch row, slice length
  int L;         // lag rows
  int NP;        // statistics slots per batch row = NR * NC
  int64_t total; // workgroups
  size_t off_part, off_sub, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int make_plan(int B, int G, int V, int dtype, int mode, Plan* p) {
  if (B < 1 || V < 1 || V > (1 << 30) || G < 0 || G > SPEC_GAMMA_MAX_LIMIT) return SPEC_ERR_SHAPE;
  if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return SPEC_ERR_ARG;
  if (mode != SPEC_MODE_SAMPLE && mode != SPEC_MODE_GREEDY) return SPEC_ERR_ARG;
  const int e = dtype == SPEC_DTYPE_F32 ? 4 : 2;
  const int vec = 16 / e;
  p->B = B, p->G = G, p->V = V, p->dtype = dtype, p->mode = mode;
  p->NR = mode == SPEC_MODE_SAMPLE ? 2 * G + 1 : G + 1;
  int target = g_tune.chunk_bytes / e;
  target = target < vec ? vec : target - target % vec;
  int nc = (V + target - 1) / target;
  int ch = (V + nc - 1) / nc;
  ch = (ch + vec - 1) / vec * vec;
  p->CH = ch;
  p->NC = (V + ch - 1) / ch;
  int sl = g_tune.slice_elems;
  if (sl > kSub * kMaxSubs) sl = kSub * kMaxSubs;
  sl = sl < kSub ? kSub : sl - sl % kSub;
  p->SL = sl;
  p->ND = mode == SPEC_MODE_SAMPLE ? (V + sl - 1) / sl : 0;
  p->NP = p->NR * p->NC;
  int lag = g_tune.lag_rows;
  if (lag <= 0) lag = (kLeadWorkgroups + p->NP / 2) / p->NP;
  if (lag < 1) lag = 1;
  p->L = lag < B ? lag : B;
  p->total = (int64_t)B * (p->NP + p->ND);
  if (p->total >= (int64_t)1 << 31) return SPEC_ERR_SHAPE;
  size_t off = 256;  // header: [0] unused, [1] diagnostic word
  p->off_part = off; off = align256(off + sizeof(float2) * (size_t)B * p->NP);
  p->off_sub = off; off = align256(off + sizeof(double) * (size_t)B * (p->ND ? p->ND : 1) * (sl / kSub));
  p->bytes = off + kRowBlockBytes * (size_t)B + 256;  // + counter blocks + end alignment
  return SPEC_OK;
}

// ------------------------------------------------------------------ kernel args
struct Args {
  const void* tgt;
  const void* dft;
  const int32_t* tok;
  const float* uni;
  const int32_t* gam;
  const int32_t* kv;
  int32_t* out_tok;
  int32_t* out_n;
  int32_t* out_len;
  float* pr_px;
  float* pr_qx;
  float* pr_z;
  float* pr_m;
  float* pr_s;
  unsigned* hdr;
  unsigned* ctr_end;  // 256-byte aligned end of the workspace; row blocks below it
  float2* part;
  double* sub;
  int B, G, V, NR, NC, CH, ND, SL, L, NP;
  float k2;  // log2(e) / T
  unsigned max_spin;
};

// ------------------------------------------------------------------ element access
template <int DT>
struct Elt;
template <>
struct Elt<SPEC_DTYPE_F32> {
  static constexpr int kBytes = 4, kVec = 4;
  __device__ static float one(const void* p, int64_t k) { return ((const float*)p)[k]; }
  __device__ static void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x), f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z), f[3] = __uint_as_float(v.w);
  }
};
template <>
struct Elt<SPEC_DTYPE_BF16> {
  static constexpr int kBytes = 2, kVec = 8;
  __device__ static float one(const void* p, int64_t k) {
    return __uint_as_float((uint32_t)((const uint16_t*)p)[k] << 16);
  }
  __device__ static void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16), f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16), f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16), f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16), f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Split [j0, j1) of a row into an unaligned head, a 16-byte aligned body of
// nv vectors starting at ja, and a tail starting at jb.
template <int DT>
struct Span {
  int j0, ja, jb, j1, nv, head;
  __device__ Span(const void* row, int lo, int hi) {
    using E = Elt<DT>;
    uintptr_t a = (uintptr_t)((const char*)row + (int64_t)lo * E::kBytes);
    int h = (int)(((16u - (unsigned)(a & 15u)) & 15u) / E::kBytes);
    if (h > hi - lo) h = hi - lo;
    j0 = lo, j1 = hi, head = h, ja = lo + h;
    nv = (hi - ja) / E::kVec;
    jb = ja + nv * E::kVec;
  }
};

// ------------------------------------------------------------------ reductions
// Softmax statistics are kept in the scaled domain z = l * k2 (k2 = log2(e)/T):
// a pair (m, S) has m = the largest raw logit and S = sum_j 2^(l_j k2 - R(m)),
// where R(m) = fl(m * k2) is the rounded reference.  Every weight is formed
// as 2^fma(l, k2, -R) against the same R that its sum used, so the rounding of
// R is a factor common to a weight and its normaliser and cancels in p.
__device__ __forceinline__ float ref_of(float m, float k2) { return m * k2; }

__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2, float k2) {
  const float M = fmaxf(m, m2);
  const float R = ref_of(M, k2);
  const float a = (m == NEG_INF) ? 0.f : s * ex2(ref_of(m, k2) - R);
  const float b = (m2 == NEG_INF) ? 0.f : s2 * ex2(ref_of(m2, k2) - R);
  m = M;
  s = a + b;
}

__device__ __forceinline__ void ms_fold(float& m, float& s, float v, float k2) {
  if (v > m) {
    s = (m == NEG_INF) ? 0.f : s * ex2(ref_of(m, k2) - ref_of(v, k2));
    m = v;
  }
  if (m != NEG_INF) s += ex2(fmaf(v, k2, -ref_of(m, k2)));
}

// argmax pair: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void am_merge(float& v, int& i, float v2, int i2) {
  bool take = (v2 > v) | ((v2 == v) & (i2 < i));
  v = take ? v2 : v;
  i = take ? i2 : i;
}

template <class T>
__device__ __forceinline__ T shfl_xor(T v, int lane_mask) {
  return __shfl_xor(v, lane_mask, 64);
}

// Block-wide reductions; results valid in thread 0.  `red` is LDS scratch of
// at least 2 * kWaves words.
__device__ void block_ms(float& m, float& s, float k2, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ms_merge(m, s, shfl_xor(m, o), shfl_xor(s, o), k2);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = m, red[kWaves + w] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = red[0], s = red[kWaves];
    for (int k = 1; k < kWaves; ++k) ms_merge(m, s, red[k], red[kWaves + k], k2);
  }
}

__device__ void block_am(float& v, int& i, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) am_merge(v, i, shfl_xor(v, o), shfl_xor(i, o));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v, red[kWaves + w] = __int_as_float(i);
  __syncthreads();
  if (threadIdx.x == 0) {
    v = red[0], i = __float_as_int(red[kWaves]);
    for (int k = 1; k < kWaves; ++k) am_merge(v, i, red[k], __float_as_int(red[kWaves + k]));
  }
}

__device__ void block_sum_d(double& a, double* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a += shfl_xor(a, o);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    a = red[0];
    for (int k = 1; k < kWaves; ++k) a += red[k];
  }
}

// ------------------------------------------------------------------ streaming loops
// Per-thread online (m, S) over [lo, hi) of one vocabulary row.
template <int DT>
__device__ void stats_range(const void* row, int lo, int hi, float k2, float& m, float& s) {
  using E = Elt<DT>;
  Span<DT> sp(row, lo, hi);
  const int t = threadIdx.x;
  if (t < sp.head) ms_fold(m, s, E::one(row, sp.j0 + t), k2);
  const uint4* vp = (const uint4*)((const char*)row + (int64_t)sp.ja * E::kBytes);
  for (int k0 = 0; k0 < sp.nv; k0 += kThreads * kUnroll) {
    uint4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int k = k0 + u * kThreads + t;
      if (k < sp.nv) raw[u] = vp[k];
    }
    float bm = NEG_INF;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int k = k0 + u * kThreads + t;
      if (k < sp.nv) {
        float f[E::kVec];
        E::unpack(raw[u], f);
#pragma unroll
        for (int e = 0; e < E::kVec; ++e) bm = fmaxf(bm, f[e]);
      }
    }
    if (bm > m) {
      s = (m == NEG_INF) ? 0.f : s * ex2(ref_of(m, k2) - ref_of(bm, k2));
      m = bm;
    }
    if (m != NEG_INF) {
      const float R = ref_of(m, k2);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        int k = k0 + u * kThreads + t;
        if (k < sp.nv) {
          float f[E::kVec];
          E::unpack(raw[u], f);
#pragma unroll
          for (int e = 0; e < E::kVec; ++e) s += ex2(fmaf(f[e], k2, -R));
        }
      }
    }
  }
  if (t < sp.j1 - sp.jb) ms_fold(m, s, E::one(row, sp.jb + t), k2);
}

// Per-thread (max, lowest argmax) over [lo, hi) of one vocabulary row.
template <int DT>
__device__ void argmax_range(const void* row, int lo, int hi, float& bv, int& bi) {
  using E = Elt<DT>;
  Span<DT> sp(row, lo, hi);
  const int t = threadIdx.x;
  if (t < sp.head) am_merge(bv, bi, E::one(row, sp.j0 + t), sp.j0 + t);
  const uint4* vp = (const uint4*)((const char*)row + (int64_t)sp.ja * E::kBytes);
  for (int k0 = 0; k0 < sp.nv; k0 += kThreads * kUnroll) {
    uint4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int k = k0 + u * kThreads + t;
      if (k < sp.nv) raw[u] = vp[k];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int k = k0 + u * kThreads + t;
      if (k < sp.nv) {
        float f[E::kVec];
        E::unpack(raw[u], f);
        const int jb = sp.ja + k * E::kVec;
#pragma unroll
        for (int e = 0; e < E::kVec; ++e) am_merge(bv, bi, f[e], jb + e);
      }
    }
  }
  if (t < sp.j1 - sp.jb) am_merge(bv, bi, E::one(row, sp.jb + t), sp.jb + t);
}

// Draw weights.  kind 1 (residual after a rejection at n):
// p_j = 2^((t_j - mt) k2) / St, q_j likewise, w_j = max(0, p_j - q_j).
// kind 0 (bonus): w_j = 2^((t_j - mt) k2), the bonus row's own sum being the
// normaliser.  kind 2 (a residual that rounding left without mass): w_j = p_j.
// Weights are fp32; their sums and prefix sums are accumulated in fp64 so
// that the CDF is as exact as the fp32 weights allow.
struct DrawParams {
  float rt, st_inv, rd, sd_inv, k2;  // references R(m) of target/draft row n, 1/S
  int kind;
};

__device__ __forceinline__ float draw_weight(const DrawParams& d, float t, float q_logit) {
  const float et = ex2(fmaf(t, d.k2, -d.rt));
  if (d.kind == 1) {
    const float p = et * d.st_inv;
    const float q = ex2(fmaf(q_logit, d.k2, -d.rd)) * d.sd_inv;
    return fmaxf(p - q, 0.f);
  }
  return d.kind == 2 ? et * d.st_inv : et;
}

// ------------------------------------------------------------------ hand-off
// Workgroups pass data to each other through the workspace without writing
// back the L2 (an agent-scope release fence does that, costs microseconds and
// serialises across the device; so does an acquire's L2 invalidate).  A
// writer stores the data with agent-scope
// atomic stores, which complete only once the data is visible to every XCD,
// waits for them to complete (publish), and only then takes its ticket or
// sets its flag.  A reader that observes the last ticket or the flag does an
// agent-scope atomic loads for the data, which are served coherently at the
// device level; so no cache write-back or invalidate is ever needed.
__device__ __forceinline__ void publish() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void put64(void* p, uint64_t v) {
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_f2(float2* p, float2 v) {
  put64(p, (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32));
}
__device__ __forceinline__ void put_d(double* p, double v) {
  put64(p, (uint64_t)__double_as_longlong(v));
}
__device__ __forceinline__ uint64_t get64(const void* p) {
  return __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 get_f2(const float2* p) {
  const uint64_t v = get64(p);
  return make_float2(__uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32)));
}
__device__ __forceinline__ double get_d(const double* p) {
  return __longlong_as_double((long long)get64(p));
}
__device__ __forceinline__ unsigned ticket(unsigned* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_u(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned get_u(unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ int64_t trow_off(const Args& a, int b, int i) {
  return ((int64_t)b * (a.G + 1) + i) * a.V;
}
__device__ __forceinline__ int64_t drow_off(const Args& a, int b, int i) {
  return ((int64_t)b * a.G + i) * a.V;
}
template <int DT>
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t off) {
  return (const char*)base + off * Elt<DT>::kBytes;
}
enum { kRowTicket = 0, kDrawTicket = 1, kRowFlag = 2 };
__device__ __forceinline__ unsigned* counter(const Args& a, int which, int b) {
  return a.ctr_end - (int64_t)(b + 1) * kRowBlock + which * kCounterStride;
}

// The row's decision, shared through LDS.
struct Decision {
  int n;        // accepted drafts
  int dead;     // 1: data error, the row holds the sentinel
  int resid;    // 1: draw from the residual at n, 0: bonus draw from p_g
  float ustar;  // uniform of the draw
  float mt, st, md, sd;  // (max, exp-sum) of target row n and draft row n
  int n_hit;    // final draw: broadcast slot for the index found
};

constexpr int kSubChunks = 4;  // final draw: sub-slice sums held per thread

struct Lds {
  double red_d[kWaves];
  double subs[kMaxSubs];
  double fin_base;
  float red[2 * kWaves];
  float m[2 * SPEC_GAMMA_MAX_LIMIT + 1];
  float s[2 * SPEC_GAMMA_MAX_LIMIT + 1];
  unsigned long long mask[kWaves];
  Decision dec;
  unsigned flag;
  int last;
};

// Draw-side inputs of one position, read before the row's statistics are
// complete (they are immutable inputs): lane i of wave 0 holds x_i, u_i and
// the target and draft logits at x_i.
struct Gathered {
  int x;
  float tv, dv, u;
};

template <int DT, int MODE>
__device__ Gathered gather_inputs(const Args& a, int b, int g) {
  Gathered r{-1, 0.f, 0.f, 0.f};
  const int lane = threadIdx.x;
  if (threadIdx.x >= 64) return r;
  if (lane < g) {
    r.x = a.tok[(int64_t)b * a.G + lane];
    if (MODE == SPEC_MODE_SAMPLE && (unsigned)r.x < (unsigned)a.V) {
      r.tv = Elt<DT>::one(a.tgt, trow_off(a, b, lane) + r.x);
      r.dv = Elt<DT>::one(a.dft, drow_off(a, b, lane) + r.x);
    }
  }
  if (MODE == SPEC_MODE_SAMPLE && lane <= g) r.u = a.uni[(int64_t)b * (a.G + 1) + lane];
  return r;
}

// ------------------------------------------------------------------ decision
// Merges the row's chunk statistics, runs every acceptance test at once and
// finds the first rejection with a wave ballot.  Must be called by the whole
// workgroup after an acquire; the result is in L.dec after the call.  With
// write_out the row's outputs (all but the drawn token when sampling) and
// probes are written.
template <int DT, int MODE>
__device__ void decide(const Args& a, Lds& L, int b, int g, const Gathered& in, bool write_out) {
  constexpr bool kSample = MODE == SPEC_MODE_SAMPLE;
  const int t = threadIdx.x, lane = t & 63;
  const int nrows = kSample ? 2 * g + 1 : g + 1;
  for (int r = t - 64; r >= 0 && r < nrows; r += kThreads - 64) {
    const int slot = (r <= g) ? r : (a.G + 1 + (r - g - 1));
    const float2* pp = a.part + ((int64_t)b * a.NR + slot) * a.NC;
    if (kSample) {
      float m = NEG_INF, s = 0.f;
      for (int c = 0; c < a.NC; ++c) {
        const float2 v = get_f2(&pp[c]);
        ms_merge(m, s, v.x, v.y, a.k2);
      }
      L.m[slot] = m, L.s[slot] = s;
    } else {
      float v = NEG_INF;
      int i = 0x7fffffff;
      for (int c = 0; c < a.NC; ++c) {
        const float2 q = get_f2(&pp[c]);
        am_merge(v, i, q.x, __float_as_int(q.y));
      }
      L.m[slot] = v, L.s[slot] = __int_as_float(i);
    }
  }
  __syncthreads();
  if (t < 64) {
    if (write_out && a.pr_m) {
      for (int r = lane; r < nrows; r += 64) {
        const int slot = (r <= g) ? r : (a.G + 1 + (r - g - 1));
        const float mm = L.m[slot];
        a.pr_m[(int64_t)b * (2 * a.G + 1) + slot] = mm;
        // sampling: S relative to the raw max, i.e. undo the rounding of R(m)
        const float sv = kSample && mm != NEG_INF
                             ? L.s[slot] * ex2(-fmaf(mm, a.k2, -ref_of(mm, a.k2)))
                             : L.s[slot];
        if (a.pr_s) a.pr_s[(int64_t)b * (2 * a.G + 1) + slot] = sv;
      }
    }
    const bool valid = (unsigned)in.x < (unsigned)a.V;
    bool fail = false;
    if (lane < g) {
      if (!valid) {
        fail = true;
      } else if (kSample) {
        const float p = ex2(fmaf(in.tv, a.k2, -ref_of(L.m[lane], a.k2))) / L.s[lane];
        const int ds = a.G + 1 + lane;
        const float q = ex2(fmaf(in.dv, a.k2, -ref_of(L.m[ds], a.k2))) / L.s[ds];
        if (write_out && a.pr_px) {
          a.pr_px[(int64_t)b * a.G + lane] = p;
          a.pr_qx[(int64_t)b * a.G + lane] = q;
        }
        fail = !(in.u * q < p);
      } else {
        fail = (in.x != __float_as_int(L.s[lane]));
      }
    }
    const unsigned long long mask = __ballot(fail);
    const int n = mask ? (__ffsll((long long)mask) - 1) : g;
    const bool bad_token = mask && (__shfl(valid ? 1 : 0, n, 64) == 0);
    // sampling: a row the walk uses must have a finite logit.  A dead p_i or
    // q_i makes the test at i fail (NaN), so only the stop position can hold
    // one; rows after the stop are never used.
    const bool dead_n = kSample && (L.m[n] == NEG_INF || (n < g && L.m[a.G + 1 + n] == NEG_INF));
    const bool sentinel = dead_n || bad_token;
    const float ustar = __shfl(in.u, n < g ? n + 1 : g, 64);
    if (write_out) {
      // gamma_max <= 63, so lane i owns output position i (and holds x_i)
      if (lane <= a.G && !(kSample && lane == n && !sentinel)) {
        int v = -1;
        if (!sentinel && lane < n)
          v = in.x;
        else if (!sentinel && lane == n)
          v = __float_as_int(L.s[n]);  // greedy: the target's argmax at n
        a.out_tok[(int64_t)b * (a.G + 1) + lane] = v;
      }
      if (lane == 0) {
        const int kv = a.kv ? a.kv[b] : 0;
        a.out_n[b] = sentinel ? -1 : n;
        a.out_len[b] = sentinel ? kv : kv + n;
      }
    }
    if (lane == 0) {
      Decision d;
      d.n = n, d.dead = sentinel, d.resid = n < g, d.ustar = ustar;
      d.mt = L.m[n], d.st = L.s[n];
      d.md = n < g ? L.m[a.G + 1 + n] : 0.f;
      d.sd = n < g ? L.s[a.G + 1 + n] : 1.f;
      L.dec = d;
    }
  }
  __syncthreads();
}

__device__ void write_sentinel(const Args& a, int b) {
  for (int i = threadIdx.x; i <= a.G; i += kThreads) a.out_tok[(int64_t)b * (a.G + 1) + i] = -1;
  if (threadIdx.x == 0) {
    a.out_n[b] = -1;
    a.out_len[b] = a.kv ? a.kv[b] : 0;
  }
}

// ------------------------------------------------------------------ draw
// A slice of SL elements is cut into sub-slices of kSub elements.  A draw
// item writes the fp64 weight sum of each of its sub-slices and of the whole
// slice.  The row's last draw item then descends slices -> sub-slices ->
// elements, at each level finding the first entry whose running sum exceeds
// tau = u * Z with a block-wide fp64 prefix scan.

template <int DT>
__device__ __forceinline__ float weight_at(const DrawParams& d, const void* trow,
                                           const void* drow, int j) {
  return draw_weight(d, Elt<DT>::one(trow, j), d.kind == 1 ? Elt<DT>::one(drow, j) : 0.f);
}

template <int DT>
__device__ void draw_slice(const Args& a, Lds& L, int b, int slot, const void* trow,
                           const void* drow, const DrawParams& d) {
  using E = Elt<DT>;
  constexpr int kGroup = kSub / E::kVec;  // threads sharing one sub-slice
  const int t = threadIdx.x;
  const int lo = slot * a.SL, hi = min(a.V, lo + a.SL), len = hi - lo;
  const int nsub = (len + kSub - 1) / kSub;
  const bool two = d.kind == 1;
  const bool vec = (((uintptr_t)((const char*)trow + (int64_t)lo * E::kBytes)) & 15u) == 0 &&
                   (!two || (((uintptr_t)((const char*)drow + (int64_t)lo * E::kBytes)) & 15u) == 0);
  if (vec) {
    const uint4* tv = (const uint4*)((const char*)trow + (int64_t)lo * E::kBytes);
    const uint4* dv = (const uint4*)((const char*)drow + (int64_t)lo * E::kBytes);
    const int nfull = len / E::kVec;                       // whole 16-byte vectors
    const int nround = (len + kThreads * E::kVec - 1) / (kThreads * E::kVec);
    for (int r0 = 0; r0 < nround; r0 += 4) {
      uint4 rt[4], rd[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = (r0 + u) * kThreads + t;
        if (r0 + u < nround && k < nfull) {
          rt[u] = tv[k];
          if (two) rd[u] = dv[k];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u;
        if (r >= nround) break;
        const int k = r * kThreads + t;
        double ws = 0.0;
        if (k < nfull) {
          float ft[E::kVec], fd[E::kVec];
          E::unpack(rt[u], ft);
          if (two) E::unpack(rd[u], fd);
#pragma unroll
          for (int e = 0; e < E::kVec; ++e) ws += (double)draw_weight(d, ft[e], two ? fd[e] : 0.f);
        } else {
          for (int j = lo + k * E::kVec; j < min(hi, lo + (k + 1) * E::kVec); ++j)
            ws += (double)weight_at<DT>(d, trow, drow, j);
        }
#pragma unroll
        for (int o = kGroup / 2; o >= 1; o >>= 1) ws += shfl_xor(ws, o);
        const int sidx = r * E::kVec + t / kGroup;
        if ((t % kGroup) == 0 && sidx < nsub) L.subs[sidx] = ws;
      }
    }
  } else {
    // rows not 16-byte aligned here: one element per thread per sub-slice
    for (int k = 0; k < nsub; ++k) {
      const int j = lo + k * kSub + t;
      double ws = j < hi ? (double)weight_at<DT>(d, trow, drow, j) : 0.0;
      block_sum_d(ws, L.red_d);
      if (t == 0) L.subs[k] = ws;
    }
  }
  __syncthreads();
  double* sub = a.sub + ((int64_t)b * a.ND + slot) * (a.SL / kSub);
  if (t < nsub) put_d(&sub[t], L.subs[t]);
}

// Inclusive and exclusive block prefix sums of one double per thread, in a
// fixed order (deterministic).  `total` is the sum over the block.
__device__ void block_scan_d(double v, double* red, double& incl, double& excl, double& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  double x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  double prev = __shfl_up(x, 1, 64);
  if (lane == 0) prev = 0.0;
  __syncthreads();
  if (lane == 63) red[w] = x;
  __syncthreads();
  double off = 0.0, tot = 0.0;
  for (int k = 0; k < kWaves; ++k) {
    if (k < w) off += red[k];
    tot += red[k];
  }
  incl = off + x;
  excl = off + prev;
  total = tot;
}

// Lowest (highest) thread index whose predicate holds, or -1: one wave
// ballot per wave, then a scan of kWaves masks.
__device__ int block_first(bool pred, Lds& L) {
  const unsigned long long m = __ballot(pred);
  if ((threadIdx.x & 63) == 0) L.mask[threadIdx.x >> 6] = m;
  __syncthreads();
  int r = -1;
  for (int k = 0; k < kWaves; ++k)
    if (L.mask[k]) {
      r = k * 64 + __ffsll((long long)L.mask[k]) - 1;
      break;
    }
  __syncthreads();
  return r;
}

__device__ int block_last(bool pred, Lds& L) {
  const unsigned long long m = __ballot(pred);
  if ((threadIdx.x & 63) == 0) L.mask[threadIdx.x >> 6] = m;
  __syncthreads();
  int r = -1;
  for (int k = kWaves - 1; k >= 0; --k)
    if (L.mask[k]) {
      r = k * 64 + 63 - __clzll((long long)L.mask[k]);
      break;
    }
  __syncthreads();
  return r;
}

// First index i in [0, count) with weight val(i) > 0 and tau < base + the
// inclusive prefix at i (one entry per thread per chunk of kThreads).  On
// success returns i and the exclusive prefix at i (base included) in
// base_out.  If rounding leaves no such index, returns -(1 + the last index
// with positive weight), or INT_MIN if there is none.
template <class F>
__device__ int block_find(int count, double base, double tau, F val, Lds& L, double& base_out) {
  const int t = threadIdx.x;
  double carry = base;
  int lastpos = -1;
  for (int c0 = 0; c0 < count; c0 += kThreads) {
    const int i = c0 + t;
    const double v = i < count ? val(i) : 0.0;
    double incl, excl, tot;
    block_scan_d(v, L.red_d, incl, excl, tot);
    const bool pos = i < count && v > 0.0;
    const int first = block_first(pos && tau < carry + incl, L);
    if (first >= 0) {
      if (t == first) L.fin_base = carry + excl;
      __syncthreads();
      base_out = L.fin_base;
      __syncthreads();
      return c0 + first;
    }
    const int last = block_last(pos, L);
    if (last >= 0) lastpos = c0 + last;
    carry += tot;
  }
  return lastpos >= 0 ? -(1 + lastpos) : (int)0x80000000;
}

__device__ __forceinline__ DrawParams draw_params(const Decision& dc, float k2) {
  return DrawParams{ref_of(dc.mt, k2), 1.f / dc.st, ref_of(dc.md, k2), 1.f / dc.sd, k2,
                    dc.resid ? 1 : 0};
}

// Number of sub-slices of slice s.
__device__ __forceinline__ int subs_in_slice(const Args& a, int s) {
  const int lo = s * a.SL;
  return (min(a.V, lo + a.SL) - lo + kSub - 1) / kSub;
}

// Sum Z of the row's sub-slice weights and the first sub-slice whose running
// sum exceeds tau = u * Z, over the flattened (slice, sub-slice) array with
// every entry prefetched at once (count <= kThreads * kSubChunks).  Returns
// the flat index, or -(1 + last positive entry) when rounding leaves no hit.
template <class F>
__device__ int find_sub_prefetched(int count, float u, F val, Lds& L, double& base_out,
                                   double& z_out) {
  const int t = threadIdx.x;
  // thread t owns entries [t * kSubChunks, (t + 1) * kSubChunks)
  double v[kSubChunks];
  double mine = 0.0;
#pragma unroll
  for (int e = 0; e < kSubChunks; ++e) {
    const int i = t * kSubChunks + e;
    v[e] = i < count ? val(i) : 0.0;
  }
#pragma unroll
  for (int e = 0; e < kSubChunks; ++e) mine += v[e];
  double incl, excl, z;
  block_scan_d(mine, L.red_d, incl, excl, z);
  z_out = z;
  const double tau = (double)u * z;
  // first entry, in order, whose running sum exceeds tau; last positive entry
  double c = excl;
  int hit = -1, lastpos = -1;
  double hit_base = 0.0;
#pragma unroll
  for (int e = 0; e < kSubChunks; ++e) {
    const double nxt = c + v[e];
    if (v[e] > 0.0) {
      lastpos = t * kSubChunks + e;
      if (hit < 0 && tau < nxt) hit = t * kSubChunks + e, hit_base = c;
    }
    c = nxt;
  }
  const int owner = block_first(hit >= 0, L);
  if (owner >= 0) {
    if (t == owner) L.fin_base = hit_base, L.dec.n_hit = hit;
    __syncthreads();
    base_out = L.fin_base;
    const int r = L.dec.n_hit;
    __syncthreads();
    return r;
  }
  const int lo = block_last(lastpos >= 0, L);
  if (lo >= 0) {
    if (t == lo) L.dec.n_hit = lastpos;
    __syncthreads();
    const int r = L.dec.n_hit;
    __syncthreads();
    return -(1 + r);
  }
  return (int)0x80000000;
}

// Run by the row's last draw item; its own L.dec holds the row's decision.
template <int DT>
__device__ void final_draw(const Args& a, Lds& L, int b) {
  const int t = threadIdx.x;
  const int n = L.dec.n;
  DrawParams d = draw_params(L.dec, a.k2);
  const void* trow = row_ptr<DT>(a.tgt, trow_off(a, b, n));
  const void* drow = L.dec.resid ? row_ptr<DT>(a.dft, drow_off(a, b, n)) : trow;
  const int nsub_max = a.SL / kSub;
  const double* sub = a.sub + (int64_t)b * a.ND * nsub_max;
  // flattened (slice, sub-slice) entries; the last slice may hold fewer
  auto sub_val = [&](int i) {
    const int s = i / nsub_max, k = i % nsub_max;
    return k < subs_in_slice(a, s) ? get_d(&sub[i]) : 0.0;
  };
  const int count = a.ND * nsub_max;
  const auto pick = [](int r) { return r >= 0 ? r : (r == (int)0x80000000 ? 0 : -(r + 1)); };
  double base = 0.0, z = 0.0, tau = 0.0;
  int fs = 0;
  bool fallback = false;
  for (int attempt = 0; attempt < 2; ++attempt) {
    if (count <= kThreads * kSubChunks) {
      fs = find_sub_prefetched(count, L.dec.ustar, sub_val, L, base, z);
      tau = (double)L.dec.ustar * z;
    } else {
      // long vocabularies: total first, then a chunked search
      z = 0.0;
      for (int c0 = 0; c0 < count; c0 += kThreads) {
        const int i = c0 + t;
        double incl, excl, tot;
        block_scan_d(i < count ? sub_val(i) : 0.0, L.red_d, incl, excl, tot);
        z += tot;
      }
      tau = (double)L.dec.ustar * z;
      fs = block_find(count, 0.0, tau, sub_val, L, base);
    }
    if (z > 0.0 || d.kind != 1) break;
    // rounding left the residual without mass: draw from p_n instead (slow
    // path, one sub-slice per thread; exact arithmetic never gets here)
    d.kind = 2;
    for (int f = t; f < count; f += kThreads) {
      const int s = f / nsub_max, k = f % nsub_max;
      double acc = 0.0;
      if (k < subs_in_slice(a, s)) {
        const int j0 = s * a.SL + k * kSub, j1 = min(a.V, j0 + kSub);
        for (int j = j0; j < j1; ++j) acc += (double)weight_at<DT>(d, trow, drow, j);
      }
      put_d(const_cast<double*>(&sub[f]), acc);
    }
    publish();
    __syncthreads();
    if (t == 0) atomicOr(&a.hdr[1], kDiagZeroResid);
  }
  if (a.pr_z && t == 0) a.pr_z[b] = (float)(d.kind == 0 ? z * (double)d.st_inv : z);
  fallback = fs < 0;
  fs = pick(fs);
  // elements of that sub-slice: one per thread
  const int s = fs / nsub_max, k = fs % nsub_max;
  const int j0 = s * a.SL + k * kSub;
  const int cnt = min(kSub, a.V - j0);
  const double never = __builtin_inf();
  int j = block_find(cnt, base, fallback ? never : tau,
                     [&](int i) { return (double)weight_at<DT>(d, trow, drow, j0 + i); }, L, base);
  j = pick(j);
  if (t == 0) a.out_tok[(int64_t)b * (a.G + 1) + n] = j0 + j;
}

// ------------------------------------------------------------------ kernel
template <int DT, int MODE>
__global__ __launch_bounds__(kThreads) void verify_kernel(Args a) {
  constexpr bool kSample = MODE == SPEC_MODE_SAMPLE;
  __shared__ Lds L;
  const int t = threadIdx.x;
  const int64_t id = blockIdx.x;

  // decode the workgroup id: rows 0..L-1 statistics, then [stats(L+k),
  // draws(k)] blocks, then the remaining draws.
  int b, slot;
  bool is_draw;
  {
    const int64_t head = (int64_t)a.L * a.NP;
    if (a.ND == 0 || id < head) {
      b = (int)(id / a.NP), slot = (int)(id % a.NP), is_draw = false;
    } else {
      const int64_t blk = a.NP + a.ND;
      const int64_t id2 = id - head;
      const int64_t k = id2 / blk;
      if (k < a.B - a.L) {
        const int off = (int)(id2 % blk);
        if (off < a.NP)
          b = (int)(a.L + k), slot = off, is_draw = false;
        else
          b = (int)k, slot = off - a.NP, is_draw = true;
      } else {
        const int64_t id3 = id2 - (int64_t)(a.B - a.L) * blk;
        b = (int)(a.B - a.L + id3 / a.ND), slot = (int)(id3 % a.ND), is_draw = true;
      }
    }
  }
  const int g = a.gam[b];
  const bool gvalid = (g >= 0) && (g <= a.G);

  if (!is_draw) {
    if (!gvalid) {
      if (slot == 0) {
        write_sentinel(a, b);
        if (kSample && t == 0) put_u(counter(a, kRowFlag, b), kFlagNone);
      }
      return;
    }
    const int nrows = kSample ? 2 * g + 1 : g + 1;
    const int r = slot / a.NC, c = slot % a.NC;
    if (r >= nrows) return;  // padding of a short row: no work, no ticket
    const bool is_target = r <= g;
    const int i = is_target ? r : r - g - 1;
    const int pslot = is_target ? i : a.G + 1 + i;
    const void* row = is_target ? row_ptr<DT>(a.tgt, trow_off(a, b, i))
                                : row_ptr<DT>(a.dft, drow_off(a, b, i));
    const int lo = c * a.CH, hi = min(a.V, lo + a.CH);
    float2 res;
    if (kSample) {
      float m = NEG_INF, s = 0.f;
      stats_range<DT>(row, lo, hi, a.k2, m, s);
      block_ms(m, s, a.k2, L.red);
      res = make_float2(m, s);
    } else {
      float v = NEG_INF;
      int ix = 0x7fffffff;
      argmax_range<DT>(row, lo, hi, v, ix);
      block_am(v, ix, L.red);
      res = make_float2(v, __int_as_float(ix));
    }
    if (t == 0) {
      put_f2(&a.part[((int64_t)b * a.NR + pslot) * a.NC + c], res);
      publish();
      const unsigned tk = ticket(counter(a, kRowTicket, b));
      L.last = (tk == (unsigned)(nrows * a.NC) - 1);
      if (L.last) {
        put_u(counter(a, kRowTicket, b), 0u);
        // sampling: the row's draw items take the decision from here on
        if (kSample) put_u(counter(a, kRowFlag, b), kFlagStats);
      }
    }
    __syncthreads();
    if (kSample || !L.last) return;
    const Gathered in = gather_inputs<DT, MODE>(a, b, g);
    decide<DT, MODE>(a, L, b, g, in, true);
    return;
  }

  // ---------------- draw item (b, slot): sampling only
  Gathered in{-1, 0.f, 0.f, 0.f};
  if (gvalid) in = gather_inputs<DT, MODE>(a, b, g);  // immutable inputs: read while waiting
  if (t == 0) {
    unsigned f = get_u(counter(a, kRowFlag, b));
    unsigned spins = 0;
    while (f == 0u) {
      __builtin_amdgcn_s_sleep(2);
      f = get_u(counter(a, kRowFlag, b));
      if (++spins > a.max_spin) {
        atomicOr(&a.hdr[1], kDiagSpin);
        f = kFlagNone;
        break;
      }
    }
    L.flag = f;
  }
  __syncthreads();
  bool work = false;
  if (L.flag == kFlagStats) {
    decide<DT, MODE>(a, L, b, g, in, slot == 0);
    work = !L.dec.dead;
  }
  if (work) {
    const int n = L.dec.n;
    const DrawParams d = draw_params(L.dec, a.k2);
    const void* trow = row_ptr<DT>(a.tgt, trow_off(a, b, n));
    const void* drow = L.dec.resid ? row_ptr<DT>(a.dft, drow_off(a, b, n)) : trow;
    draw_slice<DT>(a, L, b, slot, trow, drow, d);
  }
  if (t == 0) {
    publish();
    const unsigned tk = ticket(counter(a, kDrawTicket, b));
    L.last = (tk == (unsigned)a.ND - 1);
  }
  __syncthreads();
  if (!L.last) return;
  if (work) {
    final_draw<DT>(a, L, b);
  }
  if (t == 0) {
    put_u(counter(a, kDrawTicket, b), 0u);
    put_u(counter(a, kRowFlag, b), 0u);
  }
}

// ------------------------------------------------------------------ probes
__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint4* p, size_t n16, unsigned char* tail,
                                                             int ntail) {
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

constexpr int kProbeBytesPerBlock = kThreads * 16 * 16;  // 64 KiB

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const uint4* src, size_t n16, float* out) {
  const size_t base = (size_t)blockIdx.x * (kProbeBytesPerBlock / 16);
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    size_t k = base + (size_t)u * kThreads + threadIdx.x;
    if (k < n16) {
      uint4 v = src[k];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t r[kWaves];
  if ((threadIdx.x & 63) == 0) r[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = __uint_as_float(r[0] ^ r[1] ^ r[2] ^ r[3]);
}

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const uint4* src, uint4* dst, size_t n16) {
  const size_t base = (size_t)blockIdx.x * (kProbeBytesPerBlock / 16);
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    size_t k = base + (size_t)u * kThreads + threadIdx.x;
    if (k < n16) dst[k] = src[k];
  }
}

int hip_status(hipError_t e) { return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP - (int)e; }

bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

int run(const void* tgt, const void* dft, const int32_t* tok, const float* uni, const int32_t* gam,
        const int32_t* kv, int B, int G, int V, int dtype, float T, int mode, int32_t* out_tok,
        int32_t* out_n, int32_t* out_len, void* ws, size_t ws_bytes, void* stream, float* px,
        float* qx, float* pz, float* pm, float* ps) {
  Plan p;
  int st = make_plan(B, G, V, dtype, mode, &p);
  if (st != SPEC_OK) return st;
  const bool sample = mode == SPEC_MODE_SAMPLE;
  if (!tgt || !gam || !out_tok || !out_n || !out_len) return SPEC_ERR_NULL;
  if (G > 0 && !tok) return SPEC_ERR_NULL;
  if (sample && ((G > 0 && !dft) || !uni)) return SPEC_ERR_NULL;
  if (sample && !(T > 0.f && isfinite(T))) return SPEC_ERR_ARG;
  if (!ws || ws_bytes < p.bytes) return SPEC_ERR_WORKSPACE;
  const size_t e = dtype == SPEC_DTYPE_F32 ? 4 : 2;
  if (!aligned(tgt, e) || (dft && !aligned(dft, e))) return SPEC_ERR_ALIGN;
  const void* four[] = {tok, uni, gam, kv, out_tok, out_n, out_len, px, qx, pz, pm, ps};
  for (const void* q : four)
    if (q && !aligned(q, 4)) return SPEC_ERR_ALIGN;
  if (!aligned(ws, 256)) return SPEC_ERR_ALIGN;

  Args a;
  a.tgt = tgt, a.dft = dft ? dft : tgt, a.tok = tok, a.uni = uni, a.gam = gam, a.kv = kv;
  a.out_tok = out_tok, a.out_n = out_n, a.out_len = out_len;
  a.pr_px = px, a.pr_qx = qx, a.pr_z = pz, a.pr_m = pm, a.pr_s = ps;
  char* w = (char*)ws;
  a.hdr = (unsigned*)w;
  a.ctr_end = (unsigned*)(((uintptr_t)w + ws_bytes) & ~(uintptr_t)255);
  a.part = (float2*)(w + p.off_part);
  a.sub = (double*)(w + p.off_sub);
  a.B = B, a.G = G, a.V = V, a.NR = p.NR, a.NC = p.NC, a.CH = p.CH, a.ND = p.ND, a.SL = p.SL;
  a.L = p.L, a.NP = p.NP;
  a.k2 = sample ? (float)(1.4426950408889634 / (double)T) : 1.f;
  a.max_spin = 1u << 24;
  hipStream_t s = (hipStream_t)stream;
  dim3 grid((unsigned)p.total), block(kThreads);
  if (dtype == SPEC_DTYPE_BF16) {
    if (sample)
      hipLaunchKernelGGL((verify_kernel<SPEC_DTYPE_BF16, SPEC_MODE_SAMPLE>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((verify_kernel<SPEC_DTYPE_BF16, SPEC_MODE_GREEDY>), grid, block, 0, s, a);
  } else {
    if (sample)
      hipLaunchKernelGGL((verify_kernel<SPEC_DTYPE_F32, SPEC_MODE_SAMPLE>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((verify_kernel<SPEC_DTYPE_F32, SPEC_MODE_GREEDY>), grid, block, 0, s, a);
  }
  return hip_status(hipGetLastError());
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

size_t spec_verify_workspace_bytes(int B, int gamma_max, int V, int dtype, int mode) {
  Plan p;
  if (make_plan(B, gamma_max, V, dtype, mode, &p) != SPEC_OK) return 0;
  return p.bytes;
}

int spec_verify_workspace_reset(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return SPEC_ERR_NULL;
  if (!aligned(workspace, 16)) return SPEC_ERR_ALIGN;
  if (bytes == 0) return SPEC_OK;
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes % 16);
  size_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint4*)workspace, n16,
                     (unsigned char*)workspace + n16 * 16, ntail);
  return hip_status(hipGetLastError());
}

int spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                const float* uniforms, const int32_t* gamma_per_row, const int32_t* kv_len_in,
                int B, int gamma_max, int V, int dtype, float temperature, int mode,
                int32_t* out_tokens, int32_t* out_n_accepted, int32_t* out_new_len,
                void* workspace, size_t workspace_bytes, void* stream) {
  return run(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row, kv_len_in, B,
             gamma_max, V, dtype, temperature, mode, out_tokens, out_n_accepted, out_new_len,
             workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, nullptr, nullptr);
}

int spec_verify_probe(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms,
                      const int32_t* gamma_per_row, const int32_t* kv_len_in, int B,
                      int gamma_max, int V, int dtype, float temperature, int mode,
                      int32_t* out_tokens, int32_t* out_n_accepted, int32_t* out_new_len,
                      void* workspace, size_t workspace_bytes, void* stream, float* out_px,
                      float* out_qx, float* out_z, float* out_m, float* out_s) {
  if ((out_px == nullptr) != (out_qx == nullptr)) return SPEC_ERR_NULL;
  return run(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row, kv_len_in, B,
             gamma_max, V, dtype, temperature, mode, out_tokens, out_n_accepted, out_new_len,
             workspace, workspace_bytes, stream, out_px, out_qx, out_z, out_m, out_s);
}

int spec_verify_plan(int B, int gamma_max, int V, int dtype, int mode, int64_t* out) {
  if (!out) return SPEC_ERR_NULL;
  Plan p;
  int st = make_plan(B, gamma_max, V, dtype, mode, &p);
  if (st != SPEC_OK) return st;
  out[0] = p.total, out[1] = p.NC, out[2] = p.CH, out[3] = p.ND;
  out[4] = p.SL, out[5] = p.L, out[6] = p.NR, out[7] = kThreads;
  return SPEC_OK;
}

int spec_verify_tune(int chunk_bytes, int slice_elems, int lag_rows) {
  if (chunk_bytes < 0 || slice_elems < 0 || lag_rows < 0) return SPEC_ERR_ARG;
  Tuning t;
  if (chunk_bytes) t.chunk_bytes = chunk_bytes;
  if (slice_elems) t.slice_elems = slice_elems;
  t.lag_rows = lag_rows;
  g_tune = t;
  return SPEC_OK;
}

int spec_verify_diagnostics(const void* workspace, uint32_t* out_flags, void* stream) {
  if (!workspace || !out_flags) return SPEC_ERR_NULL;
  hipError_t e = hipMemcpyAsync(out_flags, (const char*)workspace + 4, sizeof(uint32_t),
                                hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  return hip_status(e);
}

const char* spec_verify_strerror(int status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_NULL: return "a required pointer is NULL";
    case SPEC_ERR_SHAPE: return "invalid shape (B, V or gamma_max out of range)";
    case SPEC_ERR_ARG: return "invalid argument (mode, dtype or temperature)";
    case SPEC_ERR_WORKSPACE: return "workspace missing or too small";
    case SPEC_ERR_ALIGN: return "misaligned pointer";
    default: break;
  }
  if (status <= SPEC_ERR_HIP) return hipGetErrorString((hipError_t)(SPEC_ERR_HIP - status));
  return "unknown status";
}

int spec_verify_version(void) { return 100; }

int spec_probe_read_blocks(size_t bytes) {
  return (int)((bytes + kProbeBytesPerBlock - 1) / kProbeBytesPerBlock);
}

int spec_probe_read(const void* src, size_t bytes, float* out, void* stream) {
  if (!src || !out) return SPEC_ERR_NULL;
  if (bytes == 0 || bytes % 16 || !aligned(src, 16)) return SPEC_ERR_ALIGN;
  const size_t blocks = (bytes + kProbeBytesPerBlock - 1) / kProbeBytesPerBlock;
  if (blocks >= ((size_t)1 << 31)) return SPEC_ERR_SHAPE;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (const uint4*)src, bytes / 16, out);
  return hip_status(hipGetLastError());
}

int spec_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return SPEC_ERR_NULL;
  if (bytes == 0 || bytes % 16 || !aligned(src, 16) || !aligned(dst, 16)) return SPEC_ERR_ALIGN;
  const size_t blocks = (bytes + kProbeBytesPerBlock - 1) / kProbeBytesPerBlock;
  if (blocks >= ((size_t)1 << 31)) return SPEC_ERR_SHAPE;
  hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (const uint4*)src, (uint4*)dst, bytes / 16);
  return hip_status(hipGetLastError());
}

}  // extern "C"
