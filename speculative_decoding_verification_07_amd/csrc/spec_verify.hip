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
constexpr unsigned kFlagDraw = 1u, kFlagNone = 2u;
constexpr unsigned kDiagSpin = 1u, kDiagZeroResid = 2u;
#define NEG_INF (-__builtin_inff())

struct Tuning {
  int chunk_bytes = 32768;
  int slice_elems = 8192;
  int lag_rows = 0;  // 0: derived from the plan
};
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
  size_t off_rowt, off_drawt, off_flag, off_rec, off_part, off_ssum, off_sub, bytes;
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
  if (lag <= 0) lag = (4096 + p->NP - 1) / p->NP + 1;
  p->L = lag < B ? lag : B;
  p->total = (int64_t)B * (p->NP + p->ND);
  if (p->total >= (int64_t)1 << 31) return SPEC_ERR_SHAPE;
  size_t off = 256;  // header: [0] unused, [1] diagnostic word
  p->off_rowt = off; off = align256(off + sizeof(unsigned) * B);
  p->off_drawt = off; off = align256(off + sizeof(unsigned) * B);
  p->off_flag = off; off = align256(off + sizeof(unsigned) * B);
  p->off_rec = off; off = align256(off + sizeof(float) * 8 * B);
  p->off_part = off; off = align256(off + sizeof(float2) * (size_t)B * p->NP);
  p->off_ssum = off; off = align256(off + sizeof(double) * (size_t)B * (p->ND ? p->ND : 1));
  p->off_sub = off; off = align256(off + sizeof(double) * (size_t)B * (p->ND ? p->ND : 1) * (sl / kSub));
  p->bytes = off;
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
  unsigned* rowt;
  unsigned* drawt;
  unsigned* flag;
  float* rec;
  float2* part;
  double* ssum;
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
// (m, S) with S relative to m in units of 2^((l - m) k2); m = -inf means empty.
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2, float k2) {
  float M = fmaxf(m, m2);
  float a = (m == NEG_INF) ? 0.f : s * ex2((m - M) * k2);
  float b = (m2 == NEG_INF) ? 0.f : s2 * ex2((m2 - M) * k2);
  m = M;
  s = a + b;
}

__device__ __forceinline__ void ms_fold(float& m, float& s, float v, float k2) {
  if (v > m) {
    s = (m == NEG_INF) ? 0.f : s * ex2((m - v) * k2);
    m = v;
  }
  if (m != NEG_INF) s += ex2((v - m) * k2);
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
      s = (m == NEG_INF) ? 0.f : s * ex2((m - bm) * k2);
      m = bm;
    }
    if (m != NEG_INF) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        int k = k0 + u * kThreads + t;
        if (k < sp.nv) {
          float f[E::kVec];
          E::unpack(raw[u], f);
#pragma unroll
          for (int e = 0; e < E::kVec; ++e) s += ex2((f[e] - m) * k2);
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
  float mt, st_inv, md, sd_inv, k2;
  int kind;
};

__device__ __forceinline__ float draw_weight(const DrawParams& d, float t, float q_logit) {
  const float et = ex2((t - d.mt) * d.k2);
  if (d.kind == 1) {
    const float p = et * d.st_inv;
    const float q = ex2((q_logit - d.md) * d.k2) * d.sd_inv;
    return fmaxf(p - q, 0.f);
  }
  return d.kind == 2 ? et * d.st_inv : et;
}

// ------------------------------------------------------------------ fences
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ unsigned ticket(unsigned* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_rel(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load_rlx(unsigned* p) {
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

struct LdsDecide {
  float m[2 * SPEC_GAMMA_MAX_LIMIT + 1];
  float s[2 * SPEC_GAMMA_MAX_LIMIT + 1];
};

struct Lds {
  double red_d[kWaves];
  double subs[kMaxSubs];
  double fin_base;
  float red[2 * kWaves];
  unsigned flag;
  int last;
  int cand, lastpos;
  LdsDecide dec;
};

__device__ void write_sentinel(const Args& a, int b) {
  for (int i = threadIdx.x; i <= a.G; i += kThreads) a.out_tok[(int64_t)b * (a.G + 1) + i] = -1;
  if (threadIdx.x == 0) {
    a.out_n[b] = -1;
    a.out_len[b] = a.kv ? a.kv[b] : 0;
  }
}

// ------------------------------------------------------------------ decision
// Run by the workgroup holding the row's last statistics ticket.
template <int DT, int MODE>
__device__ void decide_row(const Args& a, Lds& L, int b, int g) {
  constexpr bool kSample = MODE == SPEC_MODE_SAMPLE;
  const int t = threadIdx.x, lane = t & 63;
  const int nrows = kSample ? 2 * g + 1 : g + 1;
  // wave 0: per-position gathers; lanes 0..G also hold the uniforms
  int x = -1;
  float tv = 0.f, dv = 0.f, u = 0.f;
  if (t < 64) {
    if (lane < g) {
      x = a.tok[(int64_t)b * a.G + lane];
      if ((unsigned)x < (unsigned)a.V && kSample) {
        tv = Elt<DT>::one(a.tgt, trow_off(a, b, lane) + x);
        dv = Elt<DT>::one(a.dft, drow_off(a, b, lane) + x);
      }
    }
    if (kSample && lane <= g) u = a.uni[(int64_t)b * (a.G + 1) + lane];
  }
  // waves 1..: merge the chunk pairs of every needed vocabulary row
  for (int r = t - 64; r >= 0 && r < nrows; r += kThreads - 64) {
    const int slot = (r <= g) ? r : (a.G + 1 + (r - g - 1));
    const float2* pp = a.part + ((int64_t)b * a.NR + slot) * a.NC;
    if (kSample) {
      float m = NEG_INF, s = 0.f;
      for (int c = 0; c < a.NC; ++c) {
        float2 v = pp[c];
        ms_merge(m, s, v.x, v.y, a.k2);
      }
      L.dec.m[slot] = m, L.dec.s[slot] = s;
    } else {
      float v = NEG_INF;
      int i = 0x7fffffff;
      for (int c = 0; c < a.NC; ++c) {
        float2 q = pp[c];
        am_merge(v, i, q.x, __float_as_int(q.y));
      }
      L.dec.m[slot] = v, L.dec.s[slot] = __int_as_float(i);
    }
  }
  __syncthreads();
  if (t >= 64) return;

  // probes of the merged statistics
  if (a.pr_m) {
    for (int r = lane; r < nrows; r += 64) {
      const int slot = (r <= g) ? r : (a.G + 1 + (r - g - 1));
      a.pr_m[(int64_t)b * (2 * a.G + 1) + slot] = L.dec.m[slot];
      if (a.pr_s) a.pr_s[(int64_t)b * (2 * a.G + 1) + slot] = L.dec.s[slot];
    }
  }
  // sampling needs every row to have a finite logit
  bool dead = false;
  if (kSample) {
    for (int r = lane; r < nrows; r += 64) {
      const int slot = (r <= g) ? r : (a.G + 1 + (r - g - 1));
      dead |= (L.dec.m[slot] == NEG_INF);
    }
  }
  const bool any_dead = __ballot(dead) != 0;

  const bool valid = (unsigned)x < (unsigned)a.V;
  bool fail = false;
  if (lane < g) {
    if (!valid) {
      fail = true;
    } else if (kSample) {
      float p = ex2((tv - L.dec.m[lane]) * a.k2) / L.dec.s[lane];
      const int ds = a.G + 1 + lane;
      float q = ex2((dv - L.dec.m[ds]) * a.k2) / L.dec.s[ds];
      if (a.pr_px) {
        a.pr_px[(int64_t)b * a.G + lane] = p;
        a.pr_qx[(int64_t)b * a.G + lane] = q;
      }
      fail = !(u * q < p);
    } else {
      fail = (x != __float_as_int(L.dec.s[lane]));
    }
  }
  const unsigned long long mask = __ballot(fail);
  const int n = mask ? (__ffsll((long long)mask) - 1) : g;
  const bool bad_token = mask && (__shfl(valid ? 1 : 0, n, 64) == 0);
  if (any_dead || bad_token) {
    for (int i = lane; i <= a.G; i += 64) a.out_tok[(int64_t)b * (a.G + 1) + i] = -1;
    if (lane == 0) {
      a.out_n[b] = -1;
      a.out_len[b] = a.kv ? a.kv[b] : 0;
      if (kSample) {
        fence_release();
        store_rel(&a.flag[b], kFlagNone);
      }
    }
    return;
  }
  const float ustar = __shfl(u, n < g ? n + 1 : g, 64);
  // gamma_max <= 63, so lane i owns output position i (and holds x_i)
  if (lane <= a.G && !(kSample && lane == n)) {
    int v = -1;
    if (lane < n)
      v = x;
    else if (lane == n)
      v = __float_as_int(L.dec.s[n]);  // greedy: the target's argmax at n
    a.out_tok[(int64_t)b * (a.G + 1) + lane] = v;
  }
  if (lane == 0) {
    a.out_n[b] = n;
    a.out_len[b] = (a.kv ? a.kv[b] : 0) + n;
    if (kSample) {
      float* rc = a.rec + (int64_t)b * 8;
      const int ts = n;                    // target slot n (or g: bonus)
      const int ds = a.G + 1 + n;          // draft slot n (residual only)
      rc[0] = __int_as_float(n);
      rc[1] = __int_as_float(n < g ? 1 : 0);  // 1: residual, 0: bonus
      rc[2] = ustar;
      rc[3] = L.dec.m[ts];
      rc[4] = L.dec.s[ts];
      rc[5] = n < g ? L.dec.m[ds] : 0.f;
      rc[6] = n < g ? L.dec.s[ds] : 1.f;
      fence_release();
      store_rel(&a.flag[b], kFlagDraw);
    }
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
  if (t < nsub) sub[t] = L.subs[t];
  if (t == 0) {
    double tot = 0.0;
    for (int k = 0; k < nsub; ++k) tot += L.subs[k];
    a.ssum[(int64_t)b * a.ND + slot] = tot;
  }
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

// First index i in [0, count) with weight val(i) > 0 and tau < base + the
// inclusive prefix at i.  On success returns i and the exclusive prefix at i
// (base included) in base_out.  If rounding leaves no such index, returns
// -(1 + the last index with positive weight), or INT_MIN if there is none.
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
    if (t == 0) L.cand = 0x7fffffff, L.lastpos = -1;
    __syncthreads();
    const bool pos = i < count && v > 0.0;
    if (pos && tau < carry + incl) atomicMin(&L.cand, i);
    if (pos) atomicMax(&L.lastpos, i);
    __syncthreads();
    const int first = L.cand;
    if (L.lastpos >= 0) lastpos = L.lastpos;
    if (first != 0x7fffffff) {
      if (i == first) L.fin_base = carry + excl;
      __syncthreads();
      base_out = L.fin_base;
      __syncthreads();
      return first;
    }
    carry += tot;
    __syncthreads();
  }
  return lastpos >= 0 ? -(1 + lastpos) : (int)0x80000000;
}

// Run by the row's last draw item.
template <int DT>
__device__ void final_draw(const Args& a, Lds& L, int b) {
  const int t = threadIdx.x;
  const float* rc = a.rec + (int64_t)b * 8;
  const int n = __float_as_int(rc[0]);
  const bool resid = __float_as_int(rc[1]) != 0;
  const float ustar = rc[2];
  DrawParams d{rc[3], 1.f / rc[4], rc[5], 1.f / rc[6], a.k2, resid ? 1 : 0};
  const void* trow = row_ptr<DT>(a.tgt, trow_off(a, b, n));
  const void* drow = resid ? row_ptr<DT>(a.dft, drow_off(a, b, n)) : trow;
  const double* ss = a.ssum + (int64_t)b * a.ND;
  const int nsub_max = a.SL / kSub;

  // Z = sum of the slice totals (scanned in the same order as the search)
  double z = 0.0;
  for (int c0 = 0; c0 < a.ND; c0 += kThreads) {
    const int i = c0 + t;
    double incl, excl, tot;
    block_scan_d(i < a.ND ? ss[i] : 0.0, L.red_d, incl, excl, tot);
    z += tot;
  }
  if (!(z > 0.0)) {
    // rounding left the residual without mass: draw from p_n (slow path)
    d.kind = 2;
    for (int s = 0; s < a.ND; ++s) draw_slice<DT>(a, L, b, s, trow, drow, d);
    __syncthreads();
    if (t == 0) atomicOr(&a.hdr[1], kDiagZeroResid);
    z = 0.0;
    for (int c0 = 0; c0 < a.ND; c0 += kThreads) {
      const int i = c0 + t;
      double incl, excl, tot;
      block_scan_d(i < a.ND ? ss[i] : 0.0, L.red_d, incl, excl, tot);
      z += tot;
    }
  }
  const double tau = (double)ustar * z;
  if (a.pr_z && t == 0) a.pr_z[b] = (float)(d.kind == 0 ? z * (double)d.st_inv : z);

  // slices -> sub-slices -> elements.  Once rounding leaves no entry whose
  // running sum exceeds tau, the rest of the descent takes the last entry
  // with positive weight (tau = +inf finds nothing and reports it).
  auto pick = [](int r) { return r >= 0 ? r : (r == (int)0x80000000 ? 0 : -(r + 1)); };
  const double never = __builtin_inf();
  double base = 0.0;
  int s = block_find(a.ND, 0.0, tau, [&](int i) { return ss[i]; }, L, base);
  bool fallback = s < 0;
  s = pick(s);
  const int lo = s * a.SL;
  const int len = min(a.V, lo + a.SL) - lo;
  const int nsub = (len + kSub - 1) / kSub;
  const double* sub = a.sub + ((int64_t)b * a.ND + s) * nsub_max;
  int k = block_find(nsub, base, fallback ? never : tau, [&](int i) { return sub[i]; }, L, base);
  fallback = fallback || k < 0;
  k = pick(k);
  const int j0 = lo + k * kSub;
  const int cnt = min(kSub, lo + len - j0);
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
    const int nrows = gvalid ? (kSample ? 2 * g + 1 : g + 1) : 0;
    if (!gvalid) {
      if (slot == 0) {
        write_sentinel(a, b);
        if (kSample && t == 0) {
          fence_release();
          store_rel(&a.flag[b], kFlagNone);
        }
      }
      return;
    }
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
      a.part[((int64_t)b * a.NR + pslot) * a.NC + c] = res;
      fence_release();
      const unsigned total = (unsigned)(nrows * a.NC);
      const unsigned tk = ticket(&a.rowt[b]);
      L.last = (tk == total - 1);
      if (L.last) store_rel(&a.rowt[b], 0u);
    }
    __syncthreads();
    if (!L.last) return;
    fence_acquire();
    decide_row<DT, MODE>(a, L, b, g);
    return;
  }

  // ---------------- draw item (b, slot)
  if (t == 0) {
    unsigned f = load_rlx(&a.flag[b]);
    unsigned spins = 0;
    while (f == 0u) {
      __builtin_amdgcn_s_sleep(2);
      f = load_rlx(&a.flag[b]);
      if (++spins > a.max_spin) {
        atomicOr(&a.hdr[1], kDiagSpin);
        f = kFlagNone;
        break;
      }
    }
    L.flag = f;
  }
  __syncthreads();
  fence_acquire();
  const unsigned f = L.flag;
  if (f == kFlagDraw) {
    const float* rc = a.rec + (int64_t)b * 8;
    const int n = __float_as_int(rc[0]);
    const bool resid = __float_as_int(rc[1]) != 0;
    DrawParams d{rc[3], 1.f / rc[4], rc[5], 1.f / rc[6], a.k2, resid ? 1 : 0};
    const void* trow = row_ptr<DT>(a.tgt, trow_off(a, b, n));
    const void* drow = resid ? row_ptr<DT>(a.dft, drow_off(a, b, n)) : trow;
    draw_slice<DT>(a, L, b, slot, trow, drow, d);
  }
  if (t == 0) {
    fence_release();
    const unsigned tk = ticket(&a.drawt[b]);
    L.last = (tk == (unsigned)a.ND - 1);
  }
  __syncthreads();
  if (!L.last) return;
  fence_acquire();
  if (f == kFlagDraw) final_draw<DT>(a, L, b);
  if (t == 0) {
    store_rel(&a.drawt[b], 0u);
    store_rel(&a.flag[b], 0u);
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
  a.rowt = (unsigned*)(w + p.off_rowt);
  a.drawt = (unsigned*)(w + p.off_drawt);
  a.flag = (unsigned*)(w + p.off_flag);
  a.rec = (float*)(w + p.off_rec);
  a.part = (float2*)(w + p.off_part);
  a.ssum = (double*)(w + p.off_ssum);
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
