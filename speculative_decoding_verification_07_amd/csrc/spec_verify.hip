// spec_verify.hip -- batched speculative-decoding verify step for MI355X (gfx950).
//
// One launch does the whole step.  Batch row b is served by a group of NC
// workgroups with consecutive ids; workgroup c of the group owns the slice
// [c*CL, (c+1)*CL) of every vocabulary row of b: target rows 0..g and, when
// sampling, draft rows 0..g-1 (g = gamma_per_row[b]).
//
//   1. Each workgroup reads its slice of a row with 16-byte loads and reduces
//      it to the softmax pair (m, S) = (largest logit, sum 2^((l - m)
//      log2e / T)); greedy: (largest logit, lowest index).  It publishes its
//      pairs to the workspace, waits for its group's pairs of the same rows
//      and merges them in a fixed order, so that every workgroup of the group
//      holds bit-identical statistics.
//   2. The acceptance tests (u_i q_i(x_i) < p_i(x_i); greedy: x_i equal to
//      the argmax) run in a wave, and a ballot finds the first rejection n.
//      By default (verify_rows_kernel) the rows are read a group of positions
//      at a time and the walk reads on only after an acceptance, so no row
//      after the stop's group is read; verify_kernel streams every row in one
//      pass and runs all tests at once (SPEC_TUNE_ONE_PASS).
//   3. Sampling and point mode: every workgroup sums its slice of the
//      distribution the token is drawn from -- the residual max(0, p_n - q_n)
//      after a rejection at n, p_g for the bonus -- in fp64 from the slices
//      it holds in registers, publishes the sums and waits for the group's.
//      The workgroup whose slice holds tau = u * Z finds the token with block
//      prefix scans over its slice.  Greedy writes the argmax at n.
//   4. The last workgroup of a row to leave clears the row's workspace
//      entries, so a completed call leaves the workspace all zero.
//
// Waits are only on workgroups of the waiter's own group.  A group's ids are
// consecutive and each XCD dispatches its ids in increasing order, so the
// lowest unfinished group always has every member running or next in line:
// every wait ends.  A bounded spin backs that up.
//
// Method: "Speculative decoding" (mhtirogla.ai), "How it works" steps 2-5
// and "Code"; blog.lo0.es, "The bare mechanism" step 3; tusharamrit, the
// loop and the modified rejection-sampling rule; tokentrails, steps 2 and 4.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <type_traits>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxSlices = kThreads;  // the draw scans one slice sum per thread
constexpr int kMaxRows = 2 * SPEC_GAMMA_MAX_LIMIT + 1;
constexpr int kStage = 1024;          // LDS entries for staging a group's pairs
constexpr int kMaxVocab = 1 << 20;
constexpr int kDefaultTargetWorkgroups = 1024;
constexpr unsigned kDiagSpin = 1u, kDiagZeroResid = 2u;
constexpr int kWsWords = 5;  // draw words per slice (residual: W0, D, S_t, S_d; exact W)
// Per-row exit counter, on its own 128-byte line.
constexpr int kLine = 32;
enum { kExit = 0 };
constexpr int kRowWords = kLine;
#define NEG_INF (-__builtin_inff())

struct Tuning {
  int vectors = 0;  // 16-byte vectors per thread and row; 0: chosen from the sizes
  int target_workgroups = kDefaultTargetWorkgroups;
  int flags = 0;    // SPEC_TUNE_ONE_PASS: sampling streams every row in one pass
};
Tuning g_tune;

// ------------------------------------------------------------------ plan
struct Plan {
  int B, G, V, dtype, mode;
  int R;       // 16-byte vectors per thread per vocabulary row
  int CL, NC;  // slice length (elements), slices per vocabulary row
  int NR;      // vocabulary rows per batch row at gamma_max
  int64_t total;
  size_t off_ctr, off_part, off_wsum, off_thr, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int make_plan(int B, int G, int V, int dtype, int mode, Plan* p) {
  if (B < 1 || V < 1 || V > kMaxVocab || G < 0 || G > SPEC_GAMMA_MAX_LIMIT) return SPEC_ERR_SHAPE;
  if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return SPEC_ERR_ARG;
  if (mode != SPEC_MODE_SAMPLE && mode != SPEC_MODE_GREEDY && mode != SPEC_MODE_POINT)
    return SPEC_ERR_ARG;
  const bool draws = mode != SPEC_MODE_GREEDY;  // a token is drawn (sample, point)
  const int vec = dtype == SPEC_DTYPE_F32 ? 4 : 8;
  p->B = B, p->G = G, p->V = V, p->dtype = dtype, p->mode = mode;
  p->NR = mode == SPEC_MODE_SAMPLE ? 2 * G + 1 : G + 1;
  // a ring of rows in flight plus (sampling) the drawn rows' slices held in
  // registers: at most 4 vectors per thread and row
  const int rmax = 4;
  auto slices = [&](int r) { return (V + r * kThreads * vec - 1) / (r * kThreads * vec); };
  int R = 0;
  if (g_tune.vectors) {
    R = g_tune.vectors < rmax ? g_tune.vectors : rmax;
    if (slices(R) > kMaxSlices) return SPEC_ERR_SHAPE;
  } else {
    // the largest slices that still give target_workgroups workgroups, else
    // the smallest slices allowed
    for (int r = rmax; r >= 1; r /= 2) {
      if (slices(r) > kMaxSlices) break;
      R = r;
      if ((int64_t)B * slices(r) >= g_tune.target_workgroups) break;
    }
    if (R == 0) return SPEC_ERR_SHAPE;
  }
  p->R = R;
  const int nc = slices(R);
  int cl = (V + nc - 1) / nc;
  cl = (cl + vec - 1) / vec * vec;
  p->CL = cl;
  p->NC = (V + cl - 1) / cl;
  p->total = (int64_t)B * p->NC;
  if (p->total >= (int64_t)1 << 31) return SPEC_ERR_SHAPE;
  size_t off = 256;  // header: [1] diagnostic word
  p->off_ctr = off; off = align256(off + sizeof(unsigned) * kRowWords * (size_t)B);
  p->off_part = off; off = align256(off + sizeof(uint64_t) * (size_t)B * p->NC * p->NR);
  p->off_wsum = off;
  if (draws) off = align256(off + sizeof(uint64_t) * kWsWords * (size_t)B * p->NC);
  p->off_thr = off;  // filter thresholds, written by the filtered calls only
  if (draws) off = align256(off + sizeof(float) * (size_t)B * (2 * G + 1));
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
  float* pr_flo;
  float* pr_fhi;
  unsigned* hdr;
  unsigned* ctr;   // [B][kRowWords]
  uint64_t* part;  // [B][NC][NR] pairs of each slice: (m, S) or (max, argmax + 1)
  uint64_t* wsum;  // [B][5][NC] draw sums of each slice (see the draw)
  const float* thr;  // [B][2G+1] filter thresholds (entries below are cut), or null
  int B, G, V, NC, CL, NR;
  float k2;        // log2(e) / T
  double k2d;      // log2(e) / T in double precision (the draw)
  unsigned max_spin;
};

// ------------------------------------------------------------------ element access
template <int DT>
struct Elt;
template <>
struct Elt<SPEC_DTYPE_F32> {
  static constexpr int kBytes = 4, kVec = 4;
  static constexpr uint32_t kNegInfWord = 0xff800000u;
  __device__ static float one(const char* p, int k) { return ((const float*)p)[k]; }
  __device__ static void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x), f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z), f[3] = __uint_as_float(v.w);
  }
  // elements [k, k + 4) packed as one vector, read element by element
  __device__ static uint4 gather(const char* p, int k) {
    const uint32_t* w = (const uint32_t*)p + k;
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Elt<SPEC_DTYPE_BF16> {
  static constexpr int kBytes = 2, kVec = 8;
  static constexpr uint32_t kNegInfWord = 0xff80ff80u;
  __device__ static float one(const char* p, int k) {
    return __uint_as_float((uint32_t)((const uint16_t*)p)[k] << 16);
  }
  __device__ static void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16), f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16), f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16), f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16), f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static uint4 gather(const char* p, int k) {
    const uint16_t* h = (const uint16_t*)p + k;
    return make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16,
                      h[4] | (uint32_t)h[5] << 16, h[6] | (uint32_t)h[7] << 16);
  }
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ slices in registers
// A slice [lo, lo + len) of one row splits into an unaligned head of `head`
// elements, nv 16-byte vectors and a tail of len - jb elements.  Thread t
// holds head element t, body vectors k * kThreads + t for k < R, and tail
// element t; whatever is absent reads as -inf.  In index order: the head (in
// thread order), then round 0 of the body (thread order, each vector in
// element order), ..., round R-1, then the tail.
struct Geom {
  int head, nv, jb, len;
};

// AL: every row of the call is 16-byte aligned and V is a whole number of
// vectors, so no slice has a head or a tail (decided on the host).
template <int DT, bool AL>
__device__ __forceinline__ Geom geom_of(const char* p, int len) {
  using E = Elt<DT>;
  Geom g;
  if (AL) {
    g.head = 0, g.nv = len / E::kVec, g.jb = len, g.len = len;
    return g;
  }
  int h = (int)(((16u - ((unsigned)(uintptr_t)p & 15u)) & 15u) / E::kBytes);
  if (h > len) h = len;
  g.head = h;
  g.nv = (len - h) / E::kVec;
  g.jb = h + g.nv * E::kVec;
  g.len = len;
  return g;
}

template <int DT, int R>
struct Slice {
  uint4 v[R];
  float hd, tl;
};

// Makes a slice's registers opaque to the optimiser, so that values computed
// from them (unpacked logits, weights) are recomputed after this point
// instead of being kept live across waits.
template <int DT, int R>
__device__ __forceinline__ void opaque(Slice<DT, R>& s) {
#pragma unroll
  for (int k = 0; k < R; ++k)
    asm volatile("" : "+v"(s.v[k].x), "+v"(s.v[k].y), "+v"(s.v[k].z), "+v"(s.v[k].w));
  asm volatile("" : "+v"(s.hd), "+v"(s.tl));
}

template <int DT, int R, bool AL>
__device__ __forceinline__ void load_slice(const char* p, const Geom& g, Slice<DT, R>& s) {
  using E = Elt<DT>;
  const int t = threadIdx.x;
  const uint4* vp = (const uint4*)(p + g.head * E::kBytes);
  const uint4 ninf = make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
  if (AL) {
    // straight-line code: unconditional loads (clamped index; an aligned
    // slice holds at least one vector).  Absent vectors hold a copy of the
    // last one: readers mask them with vget, after the wait for the load.
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int q = k * kThreads + t;
      s.v[k] = vp[q < g.nv ? q : g.nv - 1];
    }
    s.hd = NEG_INF;
    s.tl = NEG_INF;
    return;
  }
  if (g.nv > 0) {  // uniform
    // unconditional loads (clamped index), then -inf for what is absent
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int q = k * kThreads + t;
      const uint4 raw = vp[q < g.nv ? q : g.nv - 1];
      s.v[k] = q < g.nv ? raw : ninf;
    }
  } else {
#pragma unroll
    for (int k = 0; k < R; ++k) s.v[k] = ninf;
  }
  s.hd = NEG_INF;
  s.tl = NEG_INF;
  if (g.head > 0 || g.jb < g.len) {  // uniform: only rows that are not 16-byte aligned
    if (t < g.head) s.hd = E::one(p, t);
    if (t < g.len - g.jb) s.tl = E::one(p, g.jb + t);
  }
}

// Vector k of this thread's share, -inf where the slice has none.
template <int DT, int R>
__device__ __forceinline__ uint4 vget(const Slice<DT, R>& s, int k, const Geom& g) {
  using E = Elt<DT>;
  const uint4 ninf = make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
  return k * kThreads + (int)threadIdx.x < g.nv ? s.v[k] : ninf;
}

// Loads a slice of another row into the register layout `g` of the slice
// [lo, lo + len) of a row with a different 16-byte alignment, element by
// element (the draft row of the draw, when it is aligned unlike the target
// row; only rows that are not 16-byte aligned get here).
template <int DT, int R>
__device__ void load_slice_as(const char* p, const Geom& g, Slice<DT, R>& s) {
  using E = Elt<DT>;
  const int t = threadIdx.x;
  const uint4 ninf = make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int q = k * kThreads + t;
    s.v[k] = q < g.nv ? E::gather(p, g.head + q * E::kVec) : ninf;
  }
  s.hd = t < g.head ? E::one(p, t) : NEG_INF;
  s.tl = t < g.len - g.jb ? E::one(p, g.jb + t) : NEG_INF;
}

// Sets element `rel` of the slice (index relative to its start) to -inf in
// the registers of the thread that holds it; nothing if rel is outside the
// slice.  Weights recomputed from the slice then give that element 0.
template <int DT, int R>
__device__ __forceinline__ void knock_out(Slice<DT, R>& s, const Geom& g, int rel) {
  using E = Elt<DT>;
  const int t = threadIdx.x;
  if (rel < 0 || rel >= g.len) return;
  if (rel < g.head) {
    if (t == rel) s.hd = NEG_INF;
    return;
  }
  if (rel >= g.jb) {
    if (t == rel - g.jb) s.tl = NEG_INF;
    return;
  }
  const int q = (rel - g.head) / E::kVec, e = (rel - g.head) % E::kVec;
  if (q % kThreads != t) return;
  const int k = q / kThreads;
  // the element's 32-bit word in the vector, and the bits it occupies there
  // (bf16: element 2i is the low half of word i)
  const int wi = DT == SPEC_DTYPE_F32 ? e : e >> 1;
  const int sh = DT == SPEC_DTYPE_F32 ? 0 : (e & 1) * 16;
  const uint32_t keep = DT == SPEC_DTYPE_F32 ? 0u : ~(0xffffu << sh);
  const uint32_t ninf = DT == SPEC_DTYPE_F32 ? 0xff800000u : 0xff80u << sh;
#pragma unroll
  for (int kk = 0; kk < R; ++kk) {
    if (kk != k) continue;
    uint4& v = s.v[kk];
    v.x = wi == 0 ? (v.x & keep) | ninf : v.x;
    v.y = wi == 1 ? (v.y & keep) | ninf : v.y;
    v.z = wi == 2 ? (v.z & keep) | ninf : v.z;
    v.w = wi == 3 ? (v.w & keep) | ninf : v.w;
  }
}

// Sets every element of the slice below tau to -inf (the filter's cut), in
// registers.
template <int DT, int R>
__device__ __forceinline__ void mask_slice(Slice<DT, R>& s, float tau) {
  auto cut = [&](float x) { return x >= tau ? x : NEG_INF; };
  s.hd = cut(s.hd);
  s.tl = cut(s.tl);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    uint32_t* wd = &s.v[k].x;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = (&s.v[k].x)[q];
      uint32_t o;
      if (DT == SPEC_DTYPE_F32) {
        o = __float_as_uint(cut(__uint_as_float(w)));
      } else {
        const uint32_t lo = __float_as_uint(cut(__uint_as_float(w << 16))) >> 16;
        const uint32_t hi = __float_as_uint(cut(__uint_as_float(w & 0xffff0000u))) & 0xffff0000u;
        o = hi | lo;
      }
      wd[q] = o;
    }
  }
}

// ------------------------------------------------------------------ reductions
// Softmax statistics are kept in the scaled domain z = l * k2 (k2 = log2(e)/T):
// a pair (m, S) has m = the largest raw logit and S = sum_j 2^(l_j k2 - R(m)),
// where R(m) = fl(m * k2) is the rounded reference.  Every weight is formed
// as 2^fma(l, k2, -R) against the same R that its sum used, so the rounding of
// R is a factor common to a weight and its normaliser and cancels in p.
__device__ __forceinline__ float ref_of(float m, float k2) { return m * k2; }

// Merge of two pairs; symmetric in its operands (max and + commute), so a
// butterfly leaves every lane with the same bits.  (-inf, 0) is the identity.
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2, float k2) {
  const float M = fmaxf(m, m2);
  const float R = ref_of(M, k2);
  const float a = (m == NEG_INF) ? 0.f : s * ex2(ref_of(m, k2) - R);
  const float b = (m2 == NEG_INF) ? 0.f : s2 * ex2(ref_of(m2, k2) - R);
  m = M;
  s = a + b;
}

// argmax pair: larger value wins, equal values go to the lower index
// (symmetric; (-inf, INT_MAX) is the identity).
__device__ __forceinline__ void am_merge(float& v, int& i, float v2, int i2) {
  const bool take = (v2 > v) | ((v2 == v) & (i2 < i));
  v = take ? v2 : v;
  i = take ? i2 : i;
}

// Wave-wide reductions on the DPP path (no LDS round trips): a butterfly
// inside each row of 16 lanes, then row broadcasts that leave the total in
// lane 63, which is read back as a wave-uniform value.  The order of the
// operations is fixed, so the result is deterministic.
#define SPEC_DPP(v, ident, ctrl, rows) __builtin_amdgcn_update_dpp((ident), (v), (ctrl), (rows), 0xf, false)
#define SPEC_WAVE_REDUCE(T, TO_I, FROM_I, OP, IDENT)                                     \
  {                                                                                     \
    const int id_ = TO_I(IDENT);                                                        \
    v = OP(v, FROM_I(SPEC_DPP(TO_I(v), id_, 0xB1, 0xf)));  /* quad_perm [1,0,3,2] */    \
    v = OP(v, FROM_I(SPEC_DPP(TO_I(v), id_, 0x4E, 0xf)));  /* quad_perm [2,3,0,1] */    \
    v = OP(v, FROM_I(SPEC_DPP(TO_I(v), id_, 0x141, 0xf))); /* row_half_mirror */       \
    v = OP(v, FROM_I(SPEC_DPP(TO_I(v), id_, 0x140, 0xf))); /* row_mirror */            \
    v = OP(v, FROM_I(SPEC_DPP(TO_I(v), id_, 0x142, 0xa))); /* row_bcast:15 */          \
    v = OP(v, FROM_I(SPEC_DPP(TO_I(v), id_, 0x143, 0xc))); /* row_bcast:31 */          \
    return FROM_I(__builtin_amdgcn_readlane(TO_I(v), 63));                              \
  }
__device__ __forceinline__ int as_i(float x) { return __float_as_int(x); }
__device__ __forceinline__ float as_f(int x) { return __int_as_float(x); }
__device__ __forceinline__ int id_i(int x) { return x; }
__device__ __forceinline__ float add_f(float x, float y) { return x + y; }
__device__ __forceinline__ int min_i(int x, int y) { return x < y ? x : y; }
__device__ __forceinline__ float wave_sum(float v) SPEC_WAVE_REDUCE(float, as_i, as_f, add_f, 0.f)
__device__ __forceinline__ int max_i(int x, int y) { return x > y ? x : y; }
__device__ __forceinline__ int wave_max_i(int v) SPEC_WAVE_REDUCE(int, id_i, id_i, max_i, (int)0x80000000)
// Floats ordered as signed integers: the bits, with the magnitude bits
// flipped when negative (-inf lowest, -0 just below +0).  A wave max over
// these keys is one integer max per step (no NaN canonicalisation).
__device__ __forceinline__ int fkey_i(float f) {
  const int i = __float_as_int(f);
  return i ^ ((i >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float fkey_f(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }
__device__ __forceinline__ float wave_max(float v) { return fkey_f(wave_max_i(fkey_i(v))); }
__device__ __forceinline__ int wave_min(int v) SPEC_WAVE_REDUCE(int, id_i, id_i, min_i, 0x7fffffff)

// (m, S) pairs of the lanes merged over the wave (result in every lane): the
// wave's largest m, then each lane's S rescaled to it, then the sum.
__device__ __forceinline__ void wave_ms_dpp(float& m, float& s, float k2) {
  const float M = wave_max(m);
  const float sc = (m == NEG_INF) ? 0.f : s * ex2(ref_of(m, k2) - ref_of(M, k2));
  s = wave_sum(sc);
  m = M;
}

// (max, lowest index) over the wave (result in every lane).
__device__ __forceinline__ void wave_am_dpp(float& v, int& i) {
  const float M = wave_max(v);
  i = wave_min(v == M ? i : 0x7fffffff);
  v = M;
}

// The same merges inside aligned groups of LPR lanes (LPR = 1, 2, 4, 8 or
// 16): the butterfly steps of SPEC_WAVE_REDUCE that stay inside a group, so
// every lane of a group ends with the group's result (same bits in each, the
// merges being symmetric).
template <int CTRL, class T>
__device__ __forceinline__ T dpp_mv(T x) {
  return __builtin_bit_cast(
      T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

template <int LPR, class T, class OP>
__device__ __forceinline__ T group_reduce(T v, OP op) {
  if constexpr (LPR >= 2) v = op(v, dpp_mv<0xB1>(v));   // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) v = op(v, dpp_mv<0x4E>(v));   // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) v = op(v, dpp_mv<0x141>(v));  // row_half_mirror
  if constexpr (LPR >= 16) v = op(v, dpp_mv<0x140>(v)); // row_mirror
  return v;
}

template <int LPR>
__device__ __forceinline__ void group_ms(float& m, float& s, float k2) {
  const float M = group_reduce<LPR>(m, [](float x, float y) { return fmaxf(x, y); });
  const float sc = (m == NEG_INF) ? 0.f : s * ex2(ref_of(m, k2) - ref_of(M, k2));
  s = group_reduce<LPR>(sc, [](float x, float y) { return x + y; });
  m = M;
}

template <int LPR>
__device__ __forceinline__ void group_am(float& v, int& i) {
  const float M = group_reduce<LPR>(v, [](float x, float y) { return fmaxf(x, y); });
  i = group_reduce<LPR>(v == M ? i : 0x7fffffff, [](int x, int y) { return x < y ? x : y; });
  v = M;
}

// Doubles on the DPP path: each half moves with its own DPP move, and lanes
// without a source read 0 (the identity of +).  Shuffles of doubles through
// the LDS crossbar (ds_bpermute) cost a round trip per step, which added up
// to microseconds in the draw's reductions.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROWS, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

__device__ __forceinline__ double readlane_d(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Wave total of a double in every lane (the butterfly and row broadcasts of
// SPEC_WAVE_REDUCE; fixed order, so deterministic).
__device__ __forceinline__ double wave_sum_d(double x) {
  x += dpp_d<0xB1, 0xf>(x);   // quad_perm [1,0,3,2]
  x += dpp_d<0x4E, 0xf>(x);   // quad_perm [2,3,0,1]
  x += dpp_d<0x141, 0xf>(x);  // row_half_mirror
  x += dpp_d<0x140, 0xf>(x);  // row_mirror
  x += dpp_d<0x142, 0xa>(x);  // row_bcast:15
  x += dpp_d<0x143, 0xc>(x);  // row_bcast:31
  return readlane_d(x, 63);
}

// Inclusive prefix sum over the wave: shifts by 1, 2, 4 and 8 inside each row
// of 16 lanes, then the row broadcasts carry each row's total into the rows
// above it.  `excl` is the inclusive sum of the lane below (0 in lane 0).
__device__ __forceinline__ double wave_scan_d(double x, double& excl) {
  x += dpp_d<0x111, 0xf>(x);  // row_shr:1
  x += dpp_d<0x112, 0xf>(x);  // row_shr:2
  x += dpp_d<0x114, 0xf>(x);  // row_shr:4
  x += dpp_d<0x118, 0xf>(x);  // row_shr:8
  x += dpp_d<0x142, 0xa>(x);  // row_bcast:15
  x += dpp_d<0x143, 0xc>(x);  // row_bcast:31
  excl = dpp_d<0x138, 0xf>(x);  // wave_shr:1
  return x;
}

// The same prefix scan on unsigned 64-bit integers (exact, so the order of
// the additions does not matter).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t x, uint64_t& excl) {
  x += dpp_u64<0x111, 0xf>(x);  // row_shr:1
  x += dpp_u64<0x112, 0xf>(x);  // row_shr:2
  x += dpp_u64<0x114, 0xf>(x);  // row_shr:4
  x += dpp_u64<0x118, 0xf>(x);  // row_shr:8
  x += dpp_u64<0x142, 0xa>(x);  // row_bcast:15
  x += dpp_u64<0x143, 0xc>(x);  // row_bcast:31
  excl = dpp_u64<0x138, 0xf>(x);  // wave_shr:1
  return x;
}

// (max, lowest index of the max) of this thread's share; lo = the slice's
// first index.  Only present elements count, so a slice of -inf yields its
// lowest present index.
template <int DT, int R>
__device__ __forceinline__ void slice_am(const Slice<DT, R>& s, const Geom& g, int lo, float& v,
                                         int& idx) {
  using E = Elt<DT>;
  const int t = threadIdx.x;
  float mx = fmaxf(s.hd, s.tl);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    float f[E::kVec];
    E::unpack(vget(s, k, g), f);
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) mx = fmaxf(mx, f[e]);
  }
  // walk the thread's elements from the highest index down
  int j = 0x7fffffff;
  if (t < g.len - g.jb && s.tl == mx) j = lo + g.jb + t;
#pragma unroll
  for (int k = R - 1; k >= 0; --k) {
    const int q = k * kThreads + t;
    if (q < g.nv) {
      float f[E::kVec];
      E::unpack(s.v[k], f);
#pragma unroll
      for (int e = E::kVec - 1; e >= 0; --e)
        if (f[e] == mx) j = lo + g.head + q * E::kVec + e;
    }
  }
  if (t < g.head && s.hd == mx) j = lo + t;
  v = mx;
  idx = j;
}

// ------------------------------------------------------------------ hand-off
// Workgroups pass data to each other through the workspace without writing
// back or invalidating the L2 (an agent-scope release fence writes back an
// XCD's whole L2, an acquire invalidates it; both cost microseconds).  A
// writer stores its data with agent-scope atomic stores, which are performed
// at the device's coherence point.  Every stored word is non-zero, so a
// reader needs no separate count: it polls the data words themselves with
// agent-scope atomic loads, served at the same coherence point, until each
// reads non-zero.
__device__ __forceinline__ void put64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get64(const uint64_t* p) {
  return __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack2(float x, float y) {
  return (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((unsigned)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((unsigned)(v >> 32)); }
__device__ __forceinline__ unsigned fetch_add(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_u(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Orders what follows after an atomic whose result `v` is: the result has
// returned, so the atomic has been performed, before any later access issues.
__device__ __forceinline__ void after(unsigned v) { asm volatile("" ::"v"(v) : "memory"); }

// Waits (in the calling thread) for a published word: every published word
// is non-zero and a completed call leaves the workspace zero, so the load
// that returns non-zero returns the data.  Gives up after max_spin polls:
// flags the diagnostic word and *gave_up (the workgroup's flag in LDS, from
// which the workgroup writes its row's sentinel instead of using the word).
__device__ uint64_t poll64(const Args& a, const uint64_t* p, int* gave_up) {
  uint64_t v = get64(p);
  for (unsigned n = 0; v == 0; ++n) {
    if (n > a.max_spin) {
      atomicOr(&a.hdr[1], kDiagSpin);
      *gave_up = 1;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    v = get64(p);
  }
  return v;
}

// The same for N words p[0], p[stride], ..., all loads in flight at once: one
// round trip per attempt instead of one per word.
template <int N>
__device__ void poll_n(const Args& a, const uint64_t* p, int stride, uint64_t (&v)[N],
                       int* gave_up) {
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = get64(p + (int64_t)k * stride);
  for (unsigned n = 0;; ++n) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < N; ++k) all = all && v[k] != 0;
    if (all) return;
    if (n > a.max_spin) {
      atomicOr(&a.hdr[1], kDiagSpin);
      *gave_up = 1;
      return;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (v[k] == 0) v[k] = get64(p + (int64_t)k * stride);
  }
}

// ------------------------------------------------------------------ LDS
struct Decision {
  int n;        // accepted drafts
  int dead;     // 1: data error, the row holds the sentinel
  int resid;    // 1: draw from the residual at n, 0: bonus draw from p_g
  int xn;       // x_n (point-mass drafts: the token the residual excludes)
  float ustar;  // uniform of the draw
  float tx;     // target logit at x_n (point-mass drafts: the excluded token)
  float mt, st, md, sd;  // (max, exp-sum) of target row n and draft row n
};

// Result of the search over a row's published slice sums, in every thread.
struct Owner {
  int r;         // slice holding tau (-1: no slice has weight)
  int fallback;  // rounding left no slice whose running sum exceeds tau
  int zero;      // residual without mass: drawn from p_n instead
  int retry;     // residual (nearly) without mass: search again with the exact rho
  double base;   // sum of the slices before r
  double z;      // Z in units of e (residual: S_t Z)
  double drho;   // rho - rho0 (residual)
  double st;     // S_t (residual)
  double rho;    // S_t / S_d (residual)
};

constexpr int kMaxSeg = 6;  // draw segments of a thread: head, up to 4 body rounds, tail

struct Lds {
  union {
    struct {                       // streaming and merging
      float wm[kMaxRows][kWaves];  // per-row wave partials: m (greedy: max)
      float ws[kMaxRows][kWaves];  // S (greedy: argmax bits)
      uint64_t stage[kStage];      // a group's published pairs
    } sm;
    struct {                       // the draw: each thread's segment sums
      double w[kMaxSeg][kThreads];
      double dd[kMaxSeg][kThreads];
    } dr;
  };
  float tau[kMaxRows];         // filter threshold of each vocabulary row (filtered calls)
  float M[kMaxRows];           // merged row statistics, row r = target i (r = i)
  float S[kMaxRows];           //   or draft i (r = g + 1 + i); greedy: argmax bits
  double red_d[8 * kWaves];
  unsigned long long mask[kWaves];
  Decision dec;
  Owner own;
  int pick, last;
  int bad;  // a poll of this workgroup gave up waiting
};

// ------------------------------------------------------------------ block helpers
// Block totals of N doubles per thread at once; every thread gets them.
template <int N>
__device__ void block_sums_n(const double (&v)[N], double (&tot)[N], Lds& L) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double x[N];
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] = wave_sum_d(v[n]);
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int n = 0; n < N; ++n) L.red_d[n * kWaves + w] = x[n];
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    double s = L.red_d[n * kWaves];
    for (int k = 1; k < kWaves; ++k) s += L.red_d[n * kWaves + k];
    tot[n] = s;
  }
  __syncthreads();
}

// Inclusive and exclusive block prefix sums of one double per thread, in a
// fixed order (deterministic); `total` is the sum over the block.
__device__ void block_scan_d(double v, Lds& L, double& incl, double& excl, double& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  double prev;
  const double x = wave_scan_d(v, prev);
  __syncthreads();
  if (lane == 63) L.red_d[w] = x;
  __syncthreads();
  double off = 0.0, tot = 0.0;
  for (int k = 0; k < kWaves; ++k) {
    if (k < w) off += L.red_d[k];
    tot += L.red_d[k];
  }
  incl = off + x;
  excl = off + prev;
  total = tot;
  __syncthreads();
}

// Lowest (highest) thread index whose predicate holds, or -1.
// (kW waves per workgroup; mask: kW words of LDS.)
template <int kW>
__device__ int block_first_m(bool pred, unsigned long long* mask) {
  const unsigned long long m = __ballot(pred);
  if ((threadIdx.x & 63) == 0) mask[threadIdx.x >> 6] = m;
  __syncthreads();
  int r = -1;
  for (int k = 0; k < kW; ++k)
    if (mask[k]) {
      r = k * 64 + __ffsll((long long)mask[k]) - 1;
      break;
    }
  __syncthreads();
  return r;
}

__device__ int block_first(bool pred, Lds& L) { return block_first_m<kWaves>(pred, L.mask); }

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

// ------------------------------------------------------------------ row access
template <int DT>
__device__ __forceinline__ const char* row_of(const Args& a, int b, int g, int r) {
  const int64_t off = r <= g ? ((int64_t)b * (a.G + 1) + r) * a.V
                             : ((int64_t)b * a.G + (r - g - 1)) * a.V;
  return (const char*)(r <= g ? a.tgt : a.dft) + off * Elt<DT>::kBytes;
}

// Probe slot of row r: target rows 0..gamma_max, then draft rows.
__device__ __forceinline__ int probe_slot(const Args& a, int g, int r) {
  return r <= g ? r : a.G + 1 + (r - g - 1);
}

// ------------------------------------------------------------------ step 1
// (m, S) of a wave's share of a slice, in every lane: the wave's largest
// logit first, then one sum against it (no rescaling), four partial sums for
// instruction-level parallelism, then the wave sum.
// FILT: entries below tau are cut (they weigh 0; the raw maximum, which a
// filter always keeps, is unchanged).
template <int DT, int R, bool AL, bool FILT>
__device__ __forceinline__ void wave_slice_ms(const Slice<DT, R>& s, const Geom& g, float k2,
                                              float tau, float& m, float& S) {
  using E = Elt<DT>;
  // (aligned rows have no head or tail element)
  float mx = AL ? NEG_INF : fmaxf(s.hd, s.tl);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    float f[E::kVec];
    E::unpack(vget(s, k, g), f);
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) mx = fmaxf(mx, f[e]);
  }
  mx = wave_max(mx);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (mx != NEG_INF) {  // uniform across the wave
    const float Rf = ref_of(mx, k2);
    auto cut = [&](float x) { return FILT && !(x >= tau) ? NEG_INF : x; };
    if (!AL) {
      acc[0] = ex2(fmaf(cut(s.hd), k2, -Rf));
      acc[1] = ex2(fmaf(cut(s.tl), k2, -Rf));
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float f[E::kVec];
      E::unpack(vget(s, k, g), f);
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) acc[e & 3] += ex2(fmaf(cut(f[e]), k2, -Rf));
    }
  }
  m = mx;
  S = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
}

// 16-byte vectors per thread kept in flight while streaming: rows of the
// ring = kRingVectors / R.
constexpr int kRingVectors = 12;

// Streaming order: the rows a draw is most likely to read again come last, so
// that they are still in the L2 when it does (a rejection at position i is
// about as likely as the walk reaching i, so early positions are the likely
// stops): t_g first, then (t_i, d_i) for i = g-1 down to 0 when sampling,
// t_g down to t_0 with point-mass drafts.  Greedy draws nothing and streams
// in index order.
template <int MODE>
__device__ __forceinline__ int stream_row(int k, int g) {
  if (MODE == SPEC_MODE_GREEDY) return k;
  if (MODE == SPEC_MODE_POINT) return g - k;
  if (k == 0) return g;
  const int j = (k - 1) >> 1;  // the pair of position g-1-j
  return (k & 1) ? g - 1 - j : 2 * g - j;
}

// The rows in flight while streaming: slot k % NB holds stream row k (the
// row loaded k-th, see stream_row).  When the stream is done the slots hold
// its last NB rows, which the draw uses instead of reading them again.
template <int DT, int R>
struct Ring {
  static constexpr int NB = kRingVectors / R > 2 ? kRingVectors / R : 2;
  Slice<DT, R> buf[NB];
  Geom geo[NB];
};

// Streams this workgroup's slice of rows 0..nrows-1 and leaves each row's
// slice pair in L.M / L.S (sampling: (m, S); greedy: (max, argmax bits)).
// The loads of the next NB-1 rows are in flight while a row is reduced; the
// ring is indexed at compile time (the row loop is unrolled by NB) and the
// loads are unconditional -- past the last row they re-read it -- so the
// waits stay counted exactly.
template <int DT, int MODE, int R, bool AL, bool FILT>
__device__ __forceinline__ void stream_rows(const Args& a, Lds& L, int b, int g, int nrows, int lo, int len,
                            Ring<DT, R>& ring) {
  constexpr bool kSample = MODE != SPEC_MODE_GREEDY;  // softmax statistics
  constexpr int NB = Ring<DT, R>::NB;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  if (FILT) {
    for (int r = t; r < nrows; r += kThreads)
      L.tau[r] = a.thr[(int64_t)b * (2 * a.G + 1) + probe_slot(a, g, r)];
    __syncthreads();
  }
  Slice<DT, R> buf[NB];
  Geom geo[NB];
  // past the end, when sampling, a slot loads the row it already holds
  // (stream row k with k = r mod NB among the last NB rows), so the last NB
  // rows stay in the ring for the draw.  Otherwise it re-reads the last row,
  // the one most surely still cached: greedy draws nothing, and with
  // point-mass drafts the rows kept (t_2..t_0) are read again from memory by
  // those reloads more often than the draw needs them.
  auto issue = [&](int r, Slice<DT, R>& sl, Geom& gg) {
    int k = r < nrows ? r : nrows - NB + (r - nrows) % NB;
    k = k < 0 ? nrows - 1 : k;  // a slot no row of this call maps to
    if (MODE != SPEC_MODE_SAMPLE) k = r < nrows ? r : nrows - 1;
    const int rr = stream_row<MODE>(k, g);
    const char* p = row_of<DT>(a, b, g, rr) + (int64_t)lo * Elt<DT>::kBytes;
    gg = geom_of<DT, AL>(p, len);
    load_slice<DT, R, AL>(p, gg, sl);
  };
#pragma unroll
  for (int j = 0; j < NB - 1; ++j) issue(j, buf[j], geo[j]);
  // whole groups of NB rows: no exit inside the unrolled body, whose rows
  // past the end reduce a reloaded row and store nothing
  for (int r0 = 0; r0 < nrows; r0 += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = r0 + j;
      issue(r + NB - 1, buf[(j + NB - 1) % NB], geo[(j + NB - 1) % NB]);
      if (kSample) {
        float m, sm;
        const float tau = FILT ? L.tau[stream_row<MODE>(r < nrows ? r : nrows - 1, g)] : NEG_INF;
        wave_slice_ms<DT, R, AL, FILT>(buf[j], geo[j], a.k2, tau, m, sm);
        if (lane == 0 && r < nrows) {
          const int rr = stream_row<MODE>(r, g);
          L.sm.wm[rr][w] = m, L.sm.ws[rr][w] = sm;
        }
      } else {
        float v;
        int ix;
        slice_am<DT, R>(buf[j], geo[j], lo, v, ix);
        wave_am_dpp(v, ix);
        if (lane == 0 && r < nrows) L.sm.wm[r][w] = v, L.sm.ws[r][w] = __int_as_float(ix);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) ring.buf[j] = buf[j], ring.geo[j] = geo[j];
  __syncthreads();
  for (int r = t; r < nrows; r += kThreads) {
    float m = L.sm.wm[r][0], s = L.sm.ws[r][0];
    for (int k = 1; k < kWaves; ++k) {
      if (kSample) {
        ms_merge(m, s, L.sm.wm[r][k], L.sm.ws[r][k], a.k2);
      } else {
        int i = __float_as_int(s);
        am_merge(m, i, L.sm.wm[r][k], __float_as_int(L.sm.ws[r][k]));
        s = __int_as_float(i);
      }
    }
    // filtered: a slice whose entries are all cut publishes the identity
    // (-inf, 0), whatever its raw maximum (which could be +0, whose pair
    // would be an all-zero word that readers take for "not yet published")
    if (FILT && kSample && s == 0.f) m = NEG_INF;
    L.M[r] = m, L.S[r] = s;
  }
  __syncthreads();
}

// Publishes this slice's pairs (entry r of the slice's record).  No written
// word is zero: S >= 1 whenever m is finite (a slice whose filter cut every
// entry publishes m = -inf), m = -inf has non-zero bits, and the argmax is
// stored plus one.  Nothing waits for the stores: readers poll
// the words themselves.
template <bool kSample>
__device__ void publish_pairs(const Args& a, Lds& L, int b, int c, int nrows) {
  uint64_t* rec = a.part + ((int64_t)b * a.NC + c) * a.NR;
  for (int r = threadIdx.x; r < nrows; r += kThreads) {
    const float s = kSample ? L.S[r] : __int_as_float(__float_as_int(L.S[r]) + 1);
    put64(&rec[r], pack2(L.M[r], s));
  }
}

// Merges the staged pairs of rows [r0, r1) (slice c of row r at
// stage[(r - r0) * nc + c]) when a row has at most LPR slices: a wave takes
// 64 / LPR rows at once, LPR lanes each.
template <bool kSample, int LPR>
__device__ void merge_rows_grouped(const Args& a, Lds& L, int r0, int r1, int nc) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int kRowsPerWave = 64 / LPR;
  const int sub = lane / LPR, c = lane % LPR;
  for (int rb = r0 + w * kRowsPerWave; rb < r1; rb += kWaves * kRowsPerWave) {
    const int r = rb + sub;
    const bool have = r < r1 && c < nc;
    const uint64_t st = have ? L.sm.stage[(r - r0) * nc + c] : 0;
    if (kSample) {
      float m = have ? lo_f(st) : NEG_INF, s = have ? hi_f(st) : 0.f;
      group_ms<LPR>(m, s, a.k2);
      if (c == 0 && r < r1) L.M[r] = m, L.S[r] = s;
    } else {
      float v = have ? lo_f(st) : NEG_INF;
      int i = have ? (int)__float_as_uint(hi_f(st)) - 1 : 0x7fffffff;
      group_am<LPR>(v, i);
      if (c == 0 && r < r1) L.M[r] = v, L.S[r] = __int_as_float(i);
    }
  }
}

// The same with more than 16 slices per row: lane l takes slices l, l + 64,
// ... of a row in turn, then a reduction across the wave; rows go to waves
// round-robin.
template <bool kSample>
__device__ void merge_rows_wide(const Args& a, Lds& L, int r0, int r1, int nc) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int r = r0 + w; r < r1; r += kWaves) {
    const uint64_t* st = &L.sm.stage[(r - r0) * nc];
    if (kSample) {
      float m = NEG_INF, s = 0.f;
      for (int c = lane; c < nc; c += 64) ms_merge(m, s, lo_f(st[c]), hi_f(st[c]), a.k2);
      wave_ms_dpp(m, s, a.k2);
      if (lane == 0) L.M[r] = m, L.S[r] = s;
    } else {
      float v = NEG_INF;
      int i = 0x7fffffff;
      for (int c = lane; c < nc; c += 64)
        am_merge(v, i, lo_f(st[c]), (int)__float_as_uint(hi_f(st[c])) - 1);
      wave_am_dpp(v, i);
      if (lane == 0) L.M[r] = v, L.S[r] = __int_as_float(i);
    }
  }
}

// Waits for the group's published pairs and merges them into L.M / L.S, in
// the same fixed order in every workgroup, staged through LDS in batches.
template <bool kSample>
__device__ void merge_group(const Args& a, Lds& L, int b, int nrows) {
  const int t = threadIdx.x;
  const int nc = a.NC;
  const uint64_t* base = a.part + (int64_t)b * nc * a.NR;
  const int per = kStage / nc > 0 ? kStage / nc : 1;
  for (int r0 = 0; r0 < nrows; r0 += per) {
    const int r1 = min(nrows, r0 + per);
    const int cnt = (r1 - r0) * nc;
    for (int k = t; k < cnt; k += kThreads) {
      const int r = r0 + k / nc, c = k % nc;
      L.sm.stage[k] = poll64(a, &base[(int64_t)c * a.NR + r], &L.bad);
    }
    __syncthreads();
    if (nc <= 4)
      merge_rows_grouped<kSample, 4>(a, L, r0, r1, nc);
    else if (nc <= 8)
      merge_rows_grouped<kSample, 8>(a, L, r0, r1, nc);
    else if (nc <= 16)
      merge_rows_grouped<kSample, 16>(a, L, r0, r1, nc);
    else
      merge_rows_wide<kSample>(a, L, r0, r1, nc);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ decision
// Immutable per-position inputs, read at the start: lane i of wave 0 holds
// x_i, u_i and the target and draft logits at x_i.
struct Gathered {
  int x;
  float tv, dv, u;
};

// x_i and u_i: read at the start, before the row loads.
template <int MODE>
__device__ Gathered gather_small(const Args& a, int b, int g) {
  Gathered r{-1, 0.f, 0.f, 0.f};
  const int lane = threadIdx.x;
  if (threadIdx.x >= 64) return r;
  if (lane < g) r.x = a.tok[(int64_t)b * a.G + lane];
  if (MODE != SPEC_MODE_GREEDY && lane <= g) r.u = a.uni[(int64_t)b * (a.G + 1) + lane];
  return r;
}

// t[x_i] and (sampling) d[x_i]: issued once the row loads are done (they
// depend on x_i, and waiting for them earlier would hold up the streaming).
template <int DT, int MODE, bool FILT>
__device__ void gather_logits(const Args& a, int b, int g, Gathered& r) {
  const int lane = threadIdx.x;
  if (threadIdx.x < 64 && lane < g && (unsigned)r.x < (unsigned)a.V) {
    r.tv = Elt<DT>::one(row_of<DT>(a, b, g, lane), r.x);
    if (MODE == SPEC_MODE_SAMPLE) r.dv = Elt<DT>::one(row_of<DT>(a, b, g, g + 1 + lane), r.x);
    if (FILT) {  // a token the filter cuts has probability 0
      const float* th = a.thr + (int64_t)b * (2 * a.G + 1);
      if (!(r.tv >= th[lane])) r.tv = NEG_INF;
      if (MODE == SPEC_MODE_SAMPLE && !(r.dv >= th[a.G + 1 + lane])) r.dv = NEG_INF;
    }
  }
}

// Runs every acceptance test at once from the merged statistics in L.M/L.S
// and finds the first rejection with a wave ballot; the result is in L.dec.
// With write_out the row's outputs (sampling: all but the drawn token) and
// probes are written.
template <int DT, int MODE>
__device__ void decide(const Args& a, Lds& L, int b, int g, const Gathered& in, bool write_out) {
  constexpr bool kSample = MODE != SPEC_MODE_GREEDY;  // a drawn token (sample, point)
  constexpr bool kPoint = MODE == SPEC_MODE_POINT;
  const int t = threadIdx.x, lane = t & 63;
  const int nrows = MODE == SPEC_MODE_SAMPLE ? 2 * g + 1 : g + 1;
  if (t < 64) {
    if (write_out && a.pr_m) {
      for (int r = lane; r < nrows; r += 64) {
        const int slot = probe_slot(a, g, r);
        const float mm = L.M[r];
        a.pr_m[(int64_t)b * (2 * a.G + 1) + slot] = mm;
        // sampling: S relative to the raw max, i.e. undo the rounding of R(m)
        const float sv = kSample && mm != NEG_INF
                             ? L.S[r] * ex2(-fmaf(mm, a.k2, -ref_of(mm, a.k2)))
                             : (kSample ? L.S[r] : (float)__float_as_int(L.S[r]));
        if (a.pr_s) a.pr_s[(int64_t)b * (2 * a.G + 1) + slot] = sv;
      }
    }
    const bool valid = (unsigned)in.x < (unsigned)a.V;
    bool fail = false;
    if (lane < g) {
      if (!valid) {
        fail = true;
      } else if (kSample) {
        const float p = ex2(fmaf(in.tv, a.k2, -ref_of(L.M[lane], a.k2))) / L.S[lane];
        // point-mass drafts: q_i is the indicator of x_i, so q_i(x_i) = 1
        const int dr = g + 1 + lane;
        const float q = kPoint ? 1.f : ex2(fmaf(in.dv, a.k2, -ref_of(L.M[dr], a.k2))) / L.S[dr];
        if (write_out && a.pr_px) {
          a.pr_px[(int64_t)b * a.G + lane] = p;
          a.pr_qx[(int64_t)b * a.G + lane] = q;
        }
        fail = !(in.u * q < p);
      } else {
        fail = (in.x != __float_as_int(L.S[lane]));
      }
    }
    const unsigned long long mask = __ballot(fail);
    const int n = mask ? (__ffsll((long long)mask) - 1) : g;
    const bool bad_token = mask && (__builtin_amdgcn_readlane(valid ? 1 : 0, n) == 0);
    // sampling: a row the walk uses must have a finite logit.  A dead p_i or
    // q_i makes the test at i fail (NaN), so only the stop position can hold
    // one; rows after the stop are never used.
    const bool dead_n =
        kSample && (L.M[n] == NEG_INF || (!kPoint && n < g && L.M[g + 1 + n] == NEG_INF));
    const bool sentinel = dead_n || bad_token;
    // n is uniform (from the ballot): lane reads, not shuffles
    const float ustar = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(in.u), n < g ? n + 1 : g));
    const int xn = __builtin_amdgcn_readlane(in.x, n < g ? n : 0);
    const float tx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(in.tv), n < g ? n : 0));
    if (write_out) {
      // gamma_max <= 63, so lane i owns output position i (and holds x_i)
      if (lane <= a.G && !(kSample && lane == n && !sentinel)) {
        int v = -1;
        if (!sentinel && lane < n)
          v = in.x;
        else if (!sentinel && lane == n)
          v = __float_as_int(L.S[n]);  // greedy: the target's argmax at n
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
      d.n = n, d.dead = sentinel, d.resid = n < g, d.xn = xn, d.ustar = ustar, d.tx = tx;
      d.mt = L.M[n], d.st = L.S[n];
      d.md = !kPoint && n < g ? L.M[g + 1 + n] : 0.f;
      d.sd = !kPoint && n < g ? L.S[g + 1 + n] : 1.f;
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
// The drawn distribution is formed in double precision from the logits of
// the row(s) it is drawn from.  An fp32 weight carries ~1e-7 relative
// rounding (more through the rounding of its exponent), and at V ~ 10^5 the
// CDF steps are ~1e-5 apart, so fp32 weights move enough boundaries past u
// to change a few draws in 10^4; in fp64 the boundaries sit within ~1e-10
// of the exact ones.
//
// Weights, in units of e(l) = 2^(l k2 - R), k2 = log2(e)/T and R = m k2 in
// fp64 for the row's largest logit m:
//   bonus draw (all drafts accepted):        w_j = e_t(j)  (its sum is Z)
//   point-mass draft rejected at n:          w_j = e_t(j), x_n set to -inf
//   residual after a rejection at n:         w_j = max(0, e_t(j) - rho e_d(j))
// with rho = S_t / S_d, the ratio of the two rows' sums of e, so that
// w_j = S_t max(0, p_n(j) - q_n(j)).  S_t and S_d are known only once every
// slice has summed its share, so each slice forms its weights against the
// provisional ratio rho0 of the fp32 statistics and publishes, besides its
// sums of e_t and e_d, W0 = sum_j max(0, e_t - rho0 e_d) and D = the sum of
// e_d over the entries with positive weight.  Then
//   W(rho) = W0 - (rho - rho0) D,
// exact but for entries whose ratio e_t/e_d lies between rho0 and rho
// (|rho - rho0| ~ 1e-6 rho), each off by at most |rho - rho0| e_d(j).  A
// residual whose corrected mass is below 2^-30 S_t (zero, or nearly, in
// exact arithmetic) is formed again against the exact rho.
//
// The code of this step runs once per row and vocabulary slice, so it is
// kept compact (one copy of each loop body, flags at run time): the whole
// kernel must stay small enough for the instruction cache that the four
// workgroups of a compute unit, each in a different phase, share.
//
// Sources: "Speculative decoding" (mhtirogla.ai), "How it works" steps 3-4
// and the `sample` routine of "Code"; tusharamrit, the modified
// rejection-sampling rule (the residual norm(max(0, p - q))).
struct DrawParams {
  double k2;    // log2(e) / T
  double rt;    // R of target row n (bonus: row g)
  double rd;    // R of draft row n (residual)
  double rho0;  // ratio the residual weights are formed against
  int resid;    // 1: residual of two rows; 0: the weights e_t of one row
};

// Minimax polynomial (relative error) for 2^r on [-1/2, 1/2], degree 7, from
// the Remez exchange (csrc/exp2_poly.py derives them): largest relative error
// 4.0e-11, coefficients of r^0 .. r^7.
constexpr double kExp2Poly[8] = {
    0.999999999961682,
    0.6931471807284468,
    0.24022651198157982,
    0.05550410353449052,
    0.009618027253625058,
    0.0013333922562610663,
    0.00015469291153107813,
    1.5201921815236906e-05,
};

// 2^x in double precision: x = n + r with n the nearest integer, so
// |r| <= 1/2 and r is exact; 2^r from the polynomial in Horner form, then the
// exact scaling by 2^n.  Arguments below -1100, and -inf, give 0 (the exact
// value is below the smallest subnormal).  Here x <= 0 always (logits never
// exceed their row's maximum).
__device__ __forceinline__ double exp2_f64(double x) {
  x = fmax(x, -1100.0);
  const double n = __builtin_rint(x);
  const double r = x - n;
  double p = kExp2Poly[7];
#pragma unroll
  for (int k = 6; k >= 0; --k) p = fma(p, r, kExp2Poly[k]);
  return __builtin_ldexp(p, (int)n);
}

__device__ __forceinline__ double e_of(float l, double k2, double ref) {
  return exp2_f64(fma((double)l, k2, -ref));
}

// One element pair of the residual against rho0: adds to the running sums.
__device__ __forceinline__ void add_pair(const DrawParams& d, float t, float q, double& w,
                                         double& dd, double& st, double& sd) {
  const double et = e_of(t, d.k2, d.rt), ed = e_of(q, d.k2, d.rd);
  st += et;
  sd += ed;
  const double x = fma(-d.rho0, ed, et);
  const bool pos = x > 0.0;
  w += pos ? x : 0.0;
  dd += pos ? ed : 0.0;
}

// Vector k of a slice selected at run time (register by register), -inf
// where the slice has none.
template <int DT, int R>
__device__ __forceinline__ uint4 vsel(const Slice<DT, R>& s, int k, const Geom& g) {
  uint4 v = s.v[0];
#pragma unroll
  for (int j = 1; j < R; ++j) {
    const bool take = k == j;
    v.x = take ? s.v[j].x : v.x, v.y = take ? s.v[j].y : v.y;
    v.z = take ? s.v[j].z : v.z, v.w = take ? s.v[j].w : v.w;
  }
  using E = Elt<DT>;
  const uint4 ninf = make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
  return k * kThreads + (int)threadIdx.x < g.nv ? v : ninf;
}

// This thread's sums of one slice, by segment in index order: [0] the head,
// [1 + k] body round k (one 16-byte vector), [R + 1] the tail.  The segment
// values go to LDS (L.dr.w: the weights against rho0 -- plain draws: the e_t;
// L.dr.dd: residual, the e_d where that weight is positive) for the owner's
// search; the thread's totals {W0, D, S_t, S_d} are returned.
template <int DT, int R, bool AL>
__device__ void slice_sums(const DrawParams& d, const Slice<DT, R>& st, const Slice<DT, R>& sd,
                           const Geom& g, Lds& L, double (&tot)[4]) {
  using E = Elt<DT>;
  const int t = threadIdx.x;
  double W = 0.0, D = 0.0, ST = 0.0, SD = 0.0;
  // head and tail: one element each (rows that are not 16-byte aligned)
  double hw = 0.0, hd = 0.0, tw = 0.0, td = 0.0;
  if (!AL) {
    if (d.resid) {
      add_pair(d, st.hd, sd.hd, hw, hd, ST, SD);
      add_pair(d, st.tl, sd.tl, tw, td, ST, SD);
    } else {
      hw = e_of(st.hd, d.k2, d.rt);
      tw = e_of(st.tl, d.k2, d.rt);
    }
  }
  L.dr.w[0][t] = hw, L.dr.dd[0][t] = hd;
  L.dr.w[R + 1][t] = tw, L.dr.dd[R + 1][t] = td;
  W = hw + tw, D = hd + td;
#pragma unroll 1
  for (int k = 0; k < R; ++k) {
    float ft[E::kVec], fd[E::kVec];
    E::unpack(vsel(st, k, g), ft);
    double w = 0.0, dd = 0.0;
    if (d.resid) {
      E::unpack(vsel(sd, k, g), fd);
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) add_pair(d, ft[e], fd[e], w, dd, ST, SD);
    } else {
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) w += e_of(ft[e], d.k2, d.rt);
    }
    L.dr.w[1 + k][t] = w, L.dr.dd[1 + k][t] = dd;
    W += w, D += dd;
  }
  if (!d.resid) ST = W;
  tot[0] = W, tot[1] = D, tot[2] = ST, tot[3] = SD;
}

// The published words of slice c, word k at ws[k * NC + c]:
//   plain draws:  [0] W = sum of e_t
//   residual:     [0] W0, [1] D, [2] S_t, [3] S_d (against rho0), and, when a
//                 second pass against the exact rho is needed, [4] W.
// Each is a non-negative double stored as the complement of its bits (sign
// bit set, so never zero).
constexpr int kWs = kWsWords;
__device__ __forceinline__ uint64_t enc_d(double x) { return ~(uint64_t)__double_as_longlong(x); }
__device__ __forceinline__ double dec_d(uint64_t v) { return __longlong_as_double((long long)~v); }

// Kinds of search over the published words.
enum { kPlain = 0, kLinear = 1, kExact = 2 };

// Waits for the group's published slice words and finds the slice holding
// tau = u Z, the same way in every workgroup (fixed-order sums).  Slices run
// one per lane of wave 0 (NC <= 64) or one per thread (NC <= 256).
//   kPlain:  the weights of word 0.
//   kLinear: the residual against rho0, corrected to the exact rho.  When the
//            corrected Z is below 2^-30 S_t (a residual that is zero, or
//            nearly, in exact arithmetic, where the rounding of the
//            correction is no longer small against Z) the search is not
//            done and `retry` asks for the exact pass.
//   kExact:  the residual of word 4, formed against the exact rho; if it has
//            no mass at all, p_n (its weights e_t are word 2) instead.
__device__ Owner find_owner(const Args& a, const uint64_t* ws, int kind, double rho0, float u,
                            Lds& L) {
  const int t = threadIdx.x, nc = a.NC;
  const bool one_wave = nc <= 64;
  if (one_wave && t >= 64) {
    __syncthreads();
    const Owner o = L.own;
    __syncthreads();
    return o;
  }
  const bool mine = t < nc;
  auto total = [&](double x) -> double {
    if (one_wave) return wave_sum_d(x);
    double tot[1];
    const double v[1] = {x};
    block_sums_n<1>(v, tot, L);
    return tot[0];
  };
  auto scan = [&](double x, double& excl, double& z) -> double {
    if (one_wave) {
      const double incl = wave_scan_d(x, excl);
      z = readlane_d(incl, 63);
      return incl;
    }
    double incl;
    block_scan_d(x, L, incl, excl, z);
    return incl;
  };
  Owner o{-1, 0, 0, 0, 0.0, 0.0, 0.0, 0.0, 0.0};
  // one round trip for all the words of the slice: words 0..3 (linear),
  // words 2 and 4 (exact: S_t, W), word 0 (plain)
  uint64_t v[4] = {0, 0, 0, 0};
  if (mine) {
    if (kind == kLinear)
      poll_n<4>(a, &ws[t], nc, v, &L.bad);
    else if (kind == kExact)
      poll_n<2>(a, &ws[2 * nc + t], 2 * nc, *(uint64_t(*)[2])v, &L.bad);
    else
      poll_n<1>(a, &ws[t], nc, *(uint64_t(*)[1])v, &L.bad);
  }
  auto dv = [&](int k) { return mine ? dec_d(v[k]) : 0.0; };
  double w, s_t = 0.0;  // this slice's weight and (residual) its S_t
  if (kind == kLinear) {
    s_t = dv(2);
    o.st = total(s_t);
    o.rho = o.st / total(dv(3));
    o.drho = o.rho - rho0;
    w = fma(-o.drho, dv(1), dv(0));  // the slice's weight against rho
  } else if (kind == kExact) {
    s_t = dv(0);
    w = dv(1);
    o.st = total(s_t);
  } else {
    w = dv(0);
  }
  double excl, z;
  double incl = scan(w, excl, z);
  if (kind == kLinear && !(z > __builtin_ldexp(o.st, -30))) {
    o.retry = 1;
  } else {
    if (kind == kExact && !(z > 0.0)) {
      // rounding left the residual without mass (exact arithmetic never
      // does): draw from p_n, whose weights are e_t, with the same uniform
      o.zero = 1;
      w = s_t;
      incl = scan(w, excl, z);
    }
    const double tau = (double)u * z;
    auto first = [&](bool pred) {
      if (one_wave) {
        const unsigned long long m = __ballot(pred);
        return m ? __ffsll((long long)m) - 1 : -1;
      }
      return block_first(pred, L);
    };
    auto last = [&](bool pred) {
      if (one_wave) {
        const unsigned long long m = __ballot(pred);
        return m ? 63 - __clzll((long long)m) : -1;
      }
      return block_last(pred, L);
    };
    o.r = first(w > 0.0 && tau < incl);
    o.fallback = o.r < 0;
    if (o.r < 0) o.r = last(w > 0.0);
  }
  o.z = z;
  // the chosen slice's exclusive sum, from its own lane / thread
  if (t == (o.r < 0 ? 0 : o.r)) {
    o.base = o.r >= 0 ? excl : 0.0;
    L.own = o;
  }
  __syncthreads();
  o = L.own;
  __syncthreads();
  return o;
}

// Inverse CDF inside the owner's slice: the first element of positive weight
// whose running sum (base + the weights before it, in index order) exceeds
// tau; if rounding leaves none, the last element with positive weight.  The
// slice's order is segment by segment (head, body rounds, tail), threads in
// order inside a segment.  Each thread's segment values (from LDS) are its
// weights against the final rho.  Every wave sums its threads' values per
// segment; after one barrier each wave finds, from those totals, the
// (segment, wave) block that holds tau.  Only that wave goes on: a scan over
// its lanes gives the thread, whose elements (its vector, read from its lane)
// are weighed one per lane, formed as slice_sums formed them, and scanned.
struct Pick {
  int j;        // the drawn index in the row
  double blo;   // running sum before the drawn element
  double bhi;   // running sum through it
  bool mine;    // the one lane of the workgroup that writes the token
};

template <int DT, int R>
__device__ Pick slice_search(const DrawParams& d, const Slice<DT, R>& st, const Slice<DT, R>& sd,
                             const Geom& g, int lo, double drho, double base, double tau, bool fb,
                             Lds& L) {
  using E = Elt<DT>;
  constexpr int NS = R + 2;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  double v[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k)
    v[k] = d.resid ? fma(-drho, L.dr.dd[k][t], L.dr.w[k][t]) : L.dr.w[k][t];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const double x = wave_sum_d(v[k]);
    if (lane == 0) L.red_d[k * kWaves + w] = x;
  }
  __syncthreads();
  // the (segment, wave) block holding tau, the same in every wave: lane i
  // holds block i's total (segment i / kWaves, wave i % kWaves, which is the
  // slice's order), and a scan over the lanes gives the running sums; the
  // fallback takes the last block with weight
  const double x = lane < NS * kWaves ? L.red_d[lane] : 0.0;
  double xe;
  const double xi = wave_scan_d(x, xe);
  const unsigned long long bh = __ballot(!fb && x > 0.0 && tau < base + xi);
  const unsigned long long bp = __ballot(x > 0.0);
  Pick p{lo, base, base, false};
  if (!bp) {  // no mass in the slice (cannot happen for an owner)
    p.mine = t == 0;
    return p;
  }
  if (!bh) fb = true;
  const int bi = bh ? __ffsll((long long)bh) - 1 : 63 - __clzll((long long)bp);
  const int ks = bi / kWaves, ws = bi % kWaves;
  const double before = base + readlane_d(xe, bi);
  if (w != ws) return p;
  double vs = 0.0;
#pragma unroll
  for (int k = 0; k < NS; ++k)
    if (k == ks) vs = v[k];
  double excl;
  const double incl = wave_scan_d(vs, excl);
  const unsigned long long hit = __ballot(!fb && vs > 0.0 && tau < before + incl);
  const unsigned long long pos = __ballot(vs > 0.0);
  if (!hit) fb = true;
  const int ln = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
  const int th = w * 64 + ln;
  const double b0 = before + readlane_d(excl, ln);  // the sum before the thread's elements
  if (ks == 0 || ks == NS - 1) {
    // a head or tail element: the thread's one element of the segment
    p.j = ks == 0 ? lo + th : lo + g.jb + th;
    p.blo = b0, p.bhi = before + readlane_d(incl, ln);
    p.mine = lane == ln;
    return p;
  }
  // the thread's vector of body round ks - 1, from its lane
  const uint4 mt = vsel(st, ks - 1, g);
  const uint4 md = d.resid ? vsel(sd, ks - 1, g) : mt;
  uint4 xt, xd;
  xt.x = __builtin_amdgcn_readlane(mt.x, ln), xt.y = __builtin_amdgcn_readlane(mt.y, ln);
  xt.z = __builtin_amdgcn_readlane(mt.z, ln), xt.w = __builtin_amdgcn_readlane(mt.w, ln);
  xd.x = __builtin_amdgcn_readlane(md.x, ln), xd.y = __builtin_amdgcn_readlane(md.y, ln);
  xd.z = __builtin_amdgcn_readlane(md.z, ln), xd.w = __builtin_amdgcn_readlane(md.w, ln);
  float ft[E::kVec], fd[E::kVec];
  E::unpack(xt, ft);
  E::unpack(xd, fd);
  float lt = NEG_INF, lq = NEG_INF;
#pragma unroll
  for (int e = 0; e < E::kVec; ++e)
    if (lane == e) lt = ft[e], lq = fd[e];
  double wl_ = 0.0;  // the element's weight against rho
  if (lane < E::kVec) {
    const double et = e_of(lt, d.k2, d.rt);
    if (d.resid) {
      const double ed = e_of(lq, d.k2, d.rd);
      const double x = fma(-d.rho0, ed, et);
      wl_ = x > 0.0 ? fma(-drho, ed, x) : 0.0;
    } else {
      wl_ = et;
    }
  }
  double ex;
  const double run = wave_scan_d(wl_, ex);
  const unsigned long long eh = __ballot(wl_ > 0.0 && !fb && tau < b0 + run);
  const unsigned long long ep = __ballot(wl_ > 0.0);
  const int e = eh ? __ffsll((long long)eh) - 1 : (ep ? 63 - __clzll((long long)ep) : 0);
  p.j = lo + g.head + ((ks - 1) * kThreads + th) * E::kVec + e;
  p.blo = b0 + ex, p.bhi = b0 + run;
  p.mine = lane == e;
  return p;
}

// Step 3 of a live sampled row: every workgroup of the group sums its slice
// of the drawn distribution and publishes the sums; the workgroup whose slice
// holds tau = u * Z writes the token.  KNOCK (point-mass drafts): after a
// rejection the residual max(0, p_n - q_n) with q_n the indicator of x_n is
// p_n without x_n, drawn as the plain weights of row n with x_n set to -inf.
__device__ void row_exit(const Args& a, Lds& L, int b, int nrows, bool draws = true);

// Slot `k` of the ring, selected at run time (register by register, so that
// the ring stays in registers).
template <int DT, int R>
__device__ __forceinline__ void ring_pick(const Ring<DT, R>& ring, int k, Slice<DT, R>& s,
                                          Geom& g) {
  s = ring.buf[0];
  g = ring.geo[0];
#pragma unroll
  for (int j = 1; j < Ring<DT, R>::NB; ++j) {
    const bool take = k == j;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      s.v[q].x = take ? ring.buf[j].v[q].x : s.v[q].x;
      s.v[q].y = take ? ring.buf[j].v[q].y : s.v[q].y;
      s.v[q].z = take ? ring.buf[j].v[q].z : s.v[q].z;
      s.v[q].w = take ? ring.buf[j].v[q].w : s.v[q].w;
    }
    s.hd = take ? ring.buf[j].hd : s.hd;
    s.tl = take ? ring.buf[j].tl : s.tl;
    g.head = take ? ring.geo[j].head : g.head;
    g.nv = take ? ring.geo[j].nv : g.nv;
    g.jb = take ? ring.geo[j].jb : g.jb;
    g.len = take ? ring.geo[j].len : g.len;
  }
}

// Slot `k` of an array of row slices, selected at run time (register by
// register, so that the array stays in registers).
template <int N, int DT, int R>
__device__ __forceinline__ void pick_slot(const Slice<DT, R> (&buf)[N], const Geom (&geo)[N],
                                          int k, Slice<DT, R>& s, Geom& g) {
  s = buf[0];
  g = geo[0];
#pragma unroll
  for (int j = 1; j < N; ++j) {
    const bool take = k == j;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      s.v[q].x = take ? buf[j].v[q].x : s.v[q].x;
      s.v[q].y = take ? buf[j].v[q].y : s.v[q].y;
      s.v[q].z = take ? buf[j].v[q].z : s.v[q].z;
      s.v[q].w = take ? buf[j].v[q].w : s.v[q].w;
    }
    s.hd = take ? buf[j].hd : s.hd;
    s.tl = take ? buf[j].tl : s.tl;
    g.head = take ? geo[j].head : g.head;
    g.nv = take ? geo[j].nv : g.nv;
    g.jb = take ? geo[j].jb : g.jb;
    g.len = take ? geo[j].len : g.len;
  }
}

// The softmax sum of a merged pair relative to the raw maximum m, i.e. with
// the rounding of its reference R(m) undone: sum_j 2^((l_j - m) k2).
__device__ __forceinline__ float s_rel(float m, float s, float k2) {
  return m == NEG_INF ? s : s * ex2(-fmaf(m, k2, -ref_of(m, k2)));
}

// Publishes this slice's totals {W0, D, S_t, S_d} (nw = 4) or {W} (nw = 1)
// at word `w0` onward: wave totals through LDS, one barrier, then thread k
// adds the four waves' totals of word k in a fixed order and stores it.
__device__ __forceinline__ void publish_sums(const Args& a, uint64_t* ws, int c, int w0, int nw,
                                             const double (&mine)[4], Lds& L) {
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k < nw) {
      const double x = wave_sum_d(mine[k]);
      if (lane == 0) L.red_d[k * kWaves + w] = x;
    }
  }
  __syncthreads();
  if (t < nw) {
    double x = L.red_d[t * kWaves];
    for (int q = 1; q < kWaves; ++q) x += L.red_d[t * kWaves + q];
    put64(&ws[(w0 + t) * a.NC + c], enc_d(x));
  }
}

// KNOCK: point-mass drafts (q_i is the indicator of x_i); RING: the ring
// holds the last rows streamed (sampling).
template <int DT, int R, bool KNOCK, bool FILT, bool AL, bool PRIO>
__device__ void draw_body(const Args& a, Lds& L, int b, int c, int g, int lo, int nrows,
                          const Decision& dc, Slice<DT, R> st, Slice<DT, R> sd, const Geom& gt);

template <int DT, int R, bool KNOCK, bool RING, bool FILT, bool AL, bool PRIO>
__device__ void draw(const Args& a, Lds& L, int b, int c, int g, int lo, int len, int nrows,
                     const Decision& dc, const Ring<DT, R>& ring) {
  using E = Elt<DT>;
  constexpr int NB = RING ? Ring<DT, R>::NB : 0;
  const int t = threadIdx.x;
  const int n = dc.n;
  const bool resid = !KNOCK && dc.resid;  // a residual of two rows
  const bool knock = KNOCK && dc.resid;   // point-mass draft rejected at n
  // stream indices of the rows drawn from (the inverse of stream_row): t_n
  // and d_n at 2(g-1-n)+1 and +2 when sampling, t_n at g-n with point-mass
  // drafts, t_g first of all for the bonus draw
  const int kt = resid ? 2 * (g - 1 - n) + 1 : (knock ? g - n : 0);
  const int kd = kt + 1;
  Slice<DT, R> st, sd;
  Geom gt;
  // (the picks pass through opaque(): otherwise the optimiser merges "take
  // from the ring" and "load from memory" into one load through a pointer,
  // which sends the whole ring to scratch memory)
  // with point-mass drafts the stream ends with t_0 and its reloads past
  // the end read t_0 again, so a rejection at 0 finds its row in the ring
  const bool from_ring = RING ? kt >= nrows - NB : knock && kt == nrows - 1;
  if (from_ring) {
    ring_pick(ring, kt % Ring<DT, R>::NB, st, gt);
    opaque(st);
  } else {
    const char* tp = row_of<DT>(a, b, g, resid || knock ? n : g) + (int64_t)lo * E::kBytes;
    gt = geom_of<DT, AL>(tp, len);
    load_slice<DT, R, AL>(tp, gt, st);
  }
  sd = st;
  if (resid) {
    // the weights pair element j of both rows: the draft slice takes the
    // target slice's register layout
    Geom gd;
    const bool in_ring = RING && kd >= nrows - NB;
    if (in_ring) {
      ring_pick(ring, kd % Ring<DT, R>::NB, sd, gd);
      opaque(sd);
    }
    if (!in_ring || !(AL || gd.head == gt.head)) {
      const char* dp = row_of<DT>(a, b, g, g + 1 + n) + (int64_t)lo * E::kBytes;
      if (AL || geom_of<DT, AL>(dp, len).head == gt.head)
        load_slice<DT, R, AL>(dp, gt, sd);
      else
        load_slice_as<DT, R>(dp, gt, sd);
    }
  }
  draw_body<DT, R, KNOCK, FILT, AL, PRIO>(a, L, b, c, g, lo, nrows, dc, st, sd, gt);
}

// The draw from the slices of the rows drawn from, in registers: st (t_n, or
// t_g for the bonus draw) and, for a residual, sd (d_n in st's layout).
template <int DT, int R, bool KNOCK, bool FILT, bool AL, bool PRIO>
__device__ void draw_body(const Args& a, Lds& L, int b, int c, int g, int lo, int nrows,
                          const Decision& dc, Slice<DT, R> st, Slice<DT, R> sd, const Geom& gt) {
  const int t = threadIdx.x;
  const int n = dc.n;
  const bool resid = !KNOCK && dc.resid;  // a residual of two rows
  const bool knock = KNOCK && dc.resid;   // point-mass draft rejected at n
  DrawParams d;
  d.k2 = a.k2d;
  d.rt = (double)dc.mt * a.k2d;
  d.rd = resid ? (double)dc.md * a.k2d : 0.0;
  d.rho0 = resid ? (double)s_rel(dc.mt, dc.st, a.k2) / (double)s_rel(dc.md, dc.sd, a.k2) : 0.0;
  d.resid = resid;
  if (FILT) {  // the filtered rows: cut entries weigh 0
    const float* th = a.thr + (int64_t)b * (2 * a.G + 1);
    mask_slice(st, th[resid || knock ? n : g]);
    if (resid) mask_slice(sd, th[a.G + 1 + n]);
  }
  if (KNOCK && knock) knock_out(st, gt, dc.xn - lo);
  uint64_t* ws = a.wsum + (int64_t)b * kWs * a.NC;
  opaque(st), opaque(sd);
  double mine[4];
  slice_sums<DT, R, AL>(d, st, sd, gt, L, mine);
  // the rest is latency-bound: above the other workgroups' draw weights
  if (PRIO) __builtin_amdgcn_s_setprio(2);
  publish_sums(a, ws, c, 0, resid ? 4 : 1, mine, L);
  Owner o = find_owner(a, ws, resid ? kLinear : kPlain, d.rho0, dc.ustar, L);
  bool exact = false;
  if (o.retry && !L.bad) {
    // a residual without mass, or nearly, in exact arithmetic: form the
    // weights again against the exact rho and search those (rare: the
    // correction's rounding could otherwise decide the draw)
    exact = true;
    d.rho0 = o.rho;
    opaque(st), opaque(sd);
    slice_sums<DT, R, AL>(d, st, sd, gt, L, mine);
    publish_sums(a, ws, c, 4, 1, mine, L);
    o = find_owner(a, ws, kExact, 0.0, dc.ustar, L);
  }
  if (L.bad) {  // a slice's sums never arrived (cannot happen in a correct launch)
    write_sentinel(a, b);
    row_exit(a, L, b, nrows);
    return;
  }
  if (knock && !(o.z > 0.0)) {
    // rounding left p_n without mass outside x_n: p_n is a point mass at x_n
    // (the same published sums give every workgroup the same z)
    if (c == 0 && t == 0) {
      atomicOr(&a.hdr[1], kDiagZeroResid);
      a.out_tok[(int64_t)b * (a.G + 1) + n] = dc.xn;
      if (a.pr_z) a.pr_z[b] = 1.f;
      if (a.pr_flo) a.pr_flo[b] = 0.f, a.pr_fhi[b] = 1.f;
    }
    row_exit(a, L, b, nrows);
    return;
  }
  if (o.zero && c == 0 && t == 0) atomicOr(&a.hdr[1], kDiagZeroResid);
  int owner = o.r;
  bool fallback = o.fallback;
  if (owner < 0) {  // no weight anywhere (cannot happen for a live row)
    owner = 0;
    fallback = true;
  }
  // every read of the row's workspace entries is done: leave the row now, so
  // that the exit ticket and the clearing overlap the owner's search (which
  // uses only its registers and LDS)
  row_exit(a, L, b, nrows);
  if (c != owner) return;
  opaque(st), opaque(sd);
  if (o.zero) {
    // residual without mass: the weights of p_n, e_t alone
    d.resid = 0;
    slice_sums<DT, R, AL>(d, st, sd, gt, L, mine);
  }
  const double tau = (double)dc.ustar * o.z;
  // linear: the weights against rho0 corrected by drho; exact: the weights
  // against rho itself (d.rho0 = rho, no correction)
  const Pick pk = slice_search<DT, R>(d, st, sd, gt, lo, exact ? 0.0 : o.drho, o.base, tau,
                                      fallback, L);
  if (pk.mine) {
    a.out_tok[(int64_t)b * (a.G + 1) + n] = pk.j;
    if (a.pr_z) {
      // Z of the drawn distribution in probability units: residual W / S_t;
      // bonus 1; point-mass draft 1 - p_n(x_n) = W / (W + e_t(x_n))
      double zp = 1.0;
      if (resid && !o.zero) zp = o.z / o.st;
      if (knock) zp = o.z / (o.z + e_of(dc.tx, d.k2, d.rt));
      a.pr_z[b] = (float)zp;
    }
    if (a.pr_flo) {  // the normalised CDF just below and at the drawn token
      a.pr_flo[b] = (float)(pk.blo / o.z);
      a.pr_fhi[b] = (float)(pk.bhi / o.z);
    }
  }
}

// ------------------------------------------------------------------ exit
// Clears a row's published pairs (rows 0..nrows-1 of every slice).
__device__ void clear_pairs(const Args& a, int b, int nrows) {
  uint64_t* base = a.part + (int64_t)b * a.NC * a.NR;
  for (int k = threadIdx.x; k < nrows * a.NC; k += kThreads)
    put64(&base[(int64_t)(k / nrows) * a.NR + k % nrows], 0);
}

// Every workgroup of a row takes the row's exit ticket after its last read
// of the row's entries (those loads have returned: their values were used);
// the last one clears the entries and the counter, and the draw's slice sums
// when the call draws a token (greedy workspaces hold none).  Every entry was
// seen by every workgroup before any of them got here, so no store of the
// call can land after the clearing.
__device__ void row_exit(const Args& a, Lds& L, int b, int nrows, bool draws) {
  unsigned* rc = a.ctr + (int64_t)b * kRowWords;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned tk = fetch_add(rc + kExit, 1u);
    after(tk);
    L.last = tk == (unsigned)a.NC - 1;
  }
  __syncthreads();
  if (!L.last) return;
  clear_pairs(a, b, nrows);
  if (draws) {
    uint64_t* ws = a.wsum + (int64_t)b * kWs * a.NC;
    for (int k = threadIdx.x; k < kWs * a.NC; k += kThreads) put64(&ws[k], 0);
  }
  if (threadIdx.x == 0) put_u(rc + kExit, 0u);
}

// ------------------------------------------------------------------ kernel
// Four waves per SIMD (four workgroups per CU) is what the sampling kernel's
// registers allow without spilling.
#ifndef SPEC_MIN_WAVES
#define SPEC_MIN_WAVES 4
#endif
template <int DT, int MODE, int R, bool AL, bool FILT, bool PRIO>
__global__ __launch_bounds__(kThreads, SPEC_MIN_WAVES) void verify_kernel(Args a) {
  constexpr bool kSample = MODE != SPEC_MODE_GREEDY;  // a drawn token (sample, point)
  __shared__ Lds L;
  // When the whole grid is resident (PRIO), the phases run at set wave
  // priorities: 3 for streaming and the wait for the group's pairs (a poll
  // that loses issue to other workgroups' streaming waits whole memory round
  // trips longer), 2 for the merge and decision, 1 for the draw weights (2
  // in the youngest quarter of the grid, whose rows finish last), 2 for the
  // slice-sum wait and the owner's search.  A CU's four workgroups are at
  // different phases, and issue goes to the oldest wave of the highest
  // priority: this way a workgroup still streaming its rows does not lose
  // issue slots to another's draw.  Priority orders issue only; a
  // low-priority wave still issues whenever the others wait, so every wait
  // still ends.  With more workgroups than slots, a slowed tail holds its
  // slot and delays the next workgroup, so plain arbitration wins.
  if (PRIO) __builtin_amdgcn_s_setprio(3);
  if (threadIdx.x == 0) L.bad = 0;  // read after stream_rows' barriers
  const int b = (int)(blockIdx.x / (unsigned)a.NC), c = (int)(blockIdx.x % (unsigned)a.NC);
  const int g = a.gam[b];
  if (g < 0 || g > a.G) {
    if (c == 0) write_sentinel(a, b);
    return;
  }
  const int nrows = MODE == SPEC_MODE_SAMPLE ? 2 * g + 1 : g + 1;
  const int lo = c * a.CL;
  const int len = min(a.V - lo, a.CL);

  Gathered in = gather_small<MODE>(a, b, g);
  Ring<DT, R> ring;
  stream_rows<DT, MODE, R, AL, FILT>(a, L, b, g, nrows, lo, len, ring);
  publish_pairs<kSample>(a, L, b, c, nrows);
  if (kSample) gather_logits<DT, MODE, FILT>(a, b, g, in);  // in flight during the wait

  if (!kSample) {
    // greedy: slice 0 waits for the group's pairs, decides, writes the row
    // and clears the pairs (it is their only reader); the other slices are
    // done
    if (c != 0) return;
    merge_group<false>(a, L, b, nrows);
    if (L.bad)  // a slice's pairs never arrived (cannot happen in a correct launch)
      write_sentinel(a, b);
    else
      decide<DT, MODE>(a, L, b, g, in, true);
    clear_pairs(a, b, nrows);
    return;
  }

  // sampling: wait for the group, merge, decide (every workgroup alike);
  // the polls keep the streaming priority (a poll behind other workgroups'
  // streaming waits whole memory round trips longer), the merge does not
  merge_group<true>(a, L, b, nrows);
  if (PRIO) __builtin_amdgcn_s_setprio(2);
  if (L.bad) {  // a slice's pairs never arrived (cannot happen in a correct launch)
    write_sentinel(a, b);
    row_exit(a, L, b, nrows);
    return;
  }
  decide<DT, MODE>(a, L, b, g, in, c == 0);
  const Decision dc = L.dec;
  // draw weights below the streaming; the youngest quarter of the grid
  // (served last by the memory system, so its rows finish last) above the
  // other quarters' draws
  if (PRIO) {
    if (blockIdx.x * 4 >= 3 * gridDim.x)
      __builtin_amdgcn_s_setprio(2);
    else
      __builtin_amdgcn_s_setprio(1);
  }
  if (!dc.dead) {
    draw<DT, R, MODE == SPEC_MODE_POINT, MODE == SPEC_MODE_SAMPLE, FILT, AL, PRIO>(
        a, L, b, c, g, lo, len, nrows, dc, ring);
  } else {
    row_exit(a, L, b, nrows);
  }
}

// ------------------------------------------------------------------ verify, row by row
// The walk stops at its first rejection n and uses no row after it: only
// position i's rows for i <= n (t_i and d_i when sampling, t_i alone when
// greedy or with point-mass drafts), and t_g when every draft is accepted
// ("Speculative decoding", mhtirogla.ai, "How it works" steps 3-4;
// tusharamrit, the acceptance loop of the proof).  This kernel reads the rows
// a few positions at a time: every workgroup of a row's group loads its
// slices of the rows of positions [i, j), publishes their statistics ((m, S);
// greedy: the max and its index), waits for the group's words of those rows,
// merges them and runs the tests at i, i + 1, ... -- the same tests, from the
// same merged statistics, as the one-pass kernel -- and reads the next
// positions only when all of [i, j) are accepted.  A rejection draws from the
// slices still in registers where it can.  Each group of positions costs one
// hand-off between the group's workgroups; no row after the stop's group of
// positions is read.  The groups are position 0 alone (every row reads it,
// and the first test is the one most often failed), then 2, then 4
// positions (kMaxSpan): a row that keeps accepting needs fewer hand-offs,
// one that stops early reads little past its stop.
constexpr int kMaxSpan = 4;
// a launch of at most this many workgroups leaves CUs idle (256 CUs)
constexpr int kSmallGrid = 256;
// the group cap min(kMaxSpan, kStage / (rows per position * NC)) is at least
// one position at every slice count allowed, so every group advances
static_assert(kStage / (2 * kMaxSlices) >= 1, "a position's pairs must fit the stage");

// The vocabulary rows of a group of positions starting at i, k of them:
// sampling t_i, d_i, t_{i+1}, d_{i+1}, ... (no d_g); otherwise t_i, t_{i+1}, ...
// PER: vocabulary rows per position (2 sampling, 1 otherwise), a template
// argument so that row() folds to one of its forms.
template <int PER>
struct RowSet {
  int i, g, k;
  __device__ int row(int j) const {
    return PER == 2 ? ((j & 1) ? g + 1 + i + (j >> 1) : i + (j >> 1)) : i + j;
  }
};

// Merges the staged pairs of the rows of `rs` (row j's slice c at
// stage[j * nc + c]) into L.M / L.S, with the reduction of the one-pass merge
// (so a row's merged pair is the same bits in both kernels).  Sampling and
// point mode: (max, exp-sum) pairs; greedy: (max, argmax + 1).
template <bool kSample, int LPR, class RS>
__device__ void merge_set(const Args& a, Lds& L, const RS& rs, int nc) {
  static_assert(LPR * 2 * kMaxSpan <= kThreads, "the workgroup merges every row of a set at once");
  const int j = threadIdx.x / LPR, c = threadIdx.x % LPR;
  const bool have = j < rs.k && c < nc;
  const uint64_t st = have ? L.sm.stage[j * nc + c] : 0;
  if (kSample) {
    float m = have ? lo_f(st) : NEG_INF, s = have ? hi_f(st) : 0.f;
    group_ms<LPR>(m, s, a.k2);
    if (c == 0 && j < rs.k) L.M[rs.row(j)] = m, L.S[rs.row(j)] = s;
  } else {
    float v = have ? lo_f(st) : NEG_INF;
    int i = have ? (int)__float_as_uint(hi_f(st)) - 1 : 0x7fffffff;
    group_am<LPR>(v, i);
    if (c == 0 && j < rs.k) L.M[rs.row(j)] = v, L.S[rs.row(j)] = __int_as_float(i);
  }
}

template <bool kSample, class RS>
__device__ void merge_set_wide(const Args& a, Lds& L, const RS& rs, int nc) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int j = w; j < rs.k; j += kWaves) {
    const uint64_t* st = &L.sm.stage[j * nc];
    if (kSample) {
      float m = NEG_INF, s = 0.f;
      for (int c = lane; c < nc; c += 64) ms_merge(m, s, lo_f(st[c]), hi_f(st[c]), a.k2);
      wave_ms_dpp(m, s, a.k2);
      if (lane == 0) L.M[rs.row(j)] = m, L.S[rs.row(j)] = s;
    } else {
      float v = NEG_INF;
      int i = 0x7fffffff;
      for (int c = lane; c < nc; c += 64)
        am_merge(v, i, lo_f(st[c]), (int)__float_as_uint(hi_f(st[c])) - 1);
      wave_am_dpp(v, i);
      if (lane == 0) L.M[rs.row(j)] = v, L.S[rs.row(j)] = __int_as_float(i);
    }
  }
}

// This workgroup's statistics of its slice of row r, as per-wave partials in
// L.sm.wm / L.sm.ws: (m, S) (sampling, point mode), (max, argmax) (greedy).
template <int DT, int R, bool AL, bool FILT, bool kSample>
__device__ void slice_pair(const Args& a, Lds& L, const Slice<DT, R>& s, const Geom& g, int r,
                           float tau, int lo) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (kSample) {
    float m, sm;
    wave_slice_ms<DT, R, AL, FILT>(s, g, a.k2, tau, m, sm);
    if (lane == 0) L.sm.wm[r][w] = m, L.sm.ws[r][w] = sm;
  } else {
    float v;
    int ix;
    slice_am<DT, R>(s, g, lo, v, ix);
    wave_am_dpp(v, ix);
    if (lane == 0) L.sm.wm[r][w] = v, L.sm.ws[r][w] = __int_as_float(ix);
  }
}

// Publishes this workgroup's pairs of the rows of `rs` (the four waves'
// partials merged in a fixed order), waits for the group's pairs of those
// rows and merges them into L.M / L.S.  Filtered: a slice whose entries are
// all cut publishes the identity (-inf, 0), as in the one-pass kernel.
// Greedy words carry the argmax plus one, so that none is zero.
template <bool kSample, class RS>
__device__ void exchange_set(const Args& a, Lds& L, int b, int c, const RS& rs, bool filt) {
  const int t = threadIdx.x, nc = a.NC;
  __syncthreads();
  if (t < rs.k) {
    const int r = rs.row(t);
    float m = L.sm.wm[r][0], sm = L.sm.ws[r][0];
    if (kSample) {
      for (int q = 1; q < kWaves; ++q) ms_merge(m, sm, L.sm.wm[r][q], L.sm.ws[r][q], a.k2);
      if (filt && sm == 0.f) m = NEG_INF;
    } else {
      int i = __float_as_int(sm);
      for (int q = 1; q < kWaves; ++q) am_merge(m, i, L.sm.wm[r][q], __float_as_int(L.sm.ws[r][q]));
      sm = __int_as_float(i + 1);
    }
    put64(&a.part[((int64_t)b * nc + c) * a.NR + r], pack2(m, sm));
  }
  const uint64_t* base = a.part + (int64_t)b * nc * a.NR;
  for (int q = t; q < rs.k * nc; q += kThreads) {
    const int j = q / nc, cc = q % nc;
    L.sm.stage[q] = poll64(a, &base[(int64_t)cc * a.NR + rs.row(j)], &L.bad);
  }
  __syncthreads();
  if (nc <= 16) {
    if (nc <= 4)
      merge_set<kSample, 4>(a, L, rs, nc);
    else if (nc <= 8)
      merge_set<kSample, 8>(a, L, rs, nc);
    else
      merge_set<kSample, 16>(a, L, rs, nc);
  } else {
    merge_set_wide<kSample>(a, L, rs, nc);
  }
  __syncthreads();
}

template <int DT, int MODE, int R, bool AL, bool FILT>
__global__ __launch_bounds__(kThreads, SPEC_MIN_WAVES) void verify_rows_kernel(Args a) {
  constexpr bool kSample = MODE != SPEC_MODE_GREEDY;  // softmax statistics, a drawn token
  constexpr bool kPoint = MODE == SPEC_MODE_POINT;
  constexpr bool kDraft = MODE == SPEC_MODE_SAMPLE;   // draft rows are read
  constexpr int kPer = kDraft ? 2 : 1;                // vocabulary rows per position
  using E = Elt<DT>;
  __shared__ Lds L;
  const int t = threadIdx.x, lane = t & 63;
  if (t == 0) L.bad = 0;
  const int b = (int)(blockIdx.x / (unsigned)a.NC), c = (int)(blockIdx.x % (unsigned)a.NC);
  const int g = a.gam[b];
  if (g < 0 || g > a.G) {
    if (c == 0) write_sentinel(a, b);
    return;
  }
  const int nrows = kDraft ? 2 * g + 1 : g + 1;
  const int lo = c * a.CL;
  const int len = min(a.V - lo, a.CL);
  // The walk (reads, hand-offs, tests) runs at wave priority 3, the draw's
  // weights at 1 (2 from its slice-sum wait on): a row still walking is on
  // the path to the call's end, and issue goes first to its waves; the
  // draws of rows already stopped take the slots the walk leaves.
  __builtin_amdgcn_s_setprio(3);
  // x_i and u_i first; the logits at x_i (which wait for x_i) once the
  // first group's rows are requested, so that wave 0's row loads do not
  // wait for x_i
  Gathered in = gather_small<MODE>(a, b, g);
  // filtered rows: the threshold of vocabulary row r (entries below weigh 0)
  const float* thr = FILT ? a.thr + (int64_t)b * (2 * a.G + 1) : nullptr;
  auto tau_of = [&](int r) { return FILT ? thr[probe_slot(a, g, r)] : NEG_INF; };
  // A ring of NS row slices, eight vectors per thread in all: the rows of a
  // group of positions go through it in order (t_i, d_i, t_{i+1}, d_{i+1},
  // ... when sampling, t_i, t_{i+1}, ... otherwise), row q in slot q mod NS,
  // each loaded once the row before it in its slot is reduced.  NS = 2 (four
  // vectors per thread and row): even rows in sa, odd in sb.  Smaller slices
  // keep more rows in flight (a group of up to eight rows at once with one
  // vector per thread), and sa / sb then receive the stop's rows for the
  // draw.  Rows that are not 16-byte aligned keep two slots (their head and
  // tail elements and geometry per slot would not fit the registers), and
  // so do filtered rows of two vectors per thread (which would spill).
  constexpr int NS = AL && !(FILT && R == 2) ? 8 / R : 2;
  Slice<DT, R> sa, sb;
  Geom ga, gb;
  Slice<DT, R> ring[NS > 2 ? NS : 1];
  Geom gring[NS > 2 ? NS : 1];
  auto load_row = [&](int r, Slice<DT, R>& s, Geom& gg) {
    const char* p = row_of<DT>(a, b, g, r) + (int64_t)lo * E::kBytes;
    gg = geom_of<DT, AL>(p, len);
    load_slice<DT, R, AL>(p, gg, s);
  };
  int n = 0, verdict = 0;  // verdict: 0 accepted, 1 stop, 2 sentinel
  bool reread = false;     // the stop's rows have left the ring
  // a group's staged pairs (kPer rows per position, NC slices each) fit kStage
  const int cap = min(kMaxSpan, kStage / (kPer * a.NC));
  // With fewer workgroups than CUs, the first group takes positions 0 and 1
  // when their rows fill the ring at once (one row per position -- greedy,
  // point-mass drafts -- or a ring of four slots or more): the wider group
  // then costs no read latency in series, the memory system has bandwidth
  // to spare at that size, and a row that accepts x_0 saves a hand-off.
  int span = (kPer == 1 || NS >= 4) && (int)gridDim.x <= kSmallGrid ? min(2, cap) : 1;
  for (int i = 0;;) {
    const int j = min(i + span, g + 1);  // positions [i, j)
    RowSet<kPer> rs;
    rs.i = i, rs.g = g;
    rs.k = kDraft ? 2 * (j - i) - (j > g ? 1 : 0) : j - i;  // no d_g
    if constexpr (NS == 2) {
      load_row(rs.row(0), sa, ga);
      if (rs.k > 1) load_row(rs.row(1), sb, gb);
      if (kSample && i == 0) gather_logits<DT, MODE, FILT>(a, b, g, in);
      for (int q = 0; q < rs.k; q += 2) {
        slice_pair<DT, R, AL, FILT, kSample>(a, L, sa, ga, rs.row(q), tau_of(rs.row(q)), lo);
        if (q + 2 < rs.k) load_row(rs.row(q + 2), sa, ga);
        if (q + 1 < rs.k) {
          slice_pair<DT, R, AL, FILT, kSample>(a, L, sb, gb, rs.row(q + 1),
                                               tau_of(rs.row(q + 1)), lo);
          if (q + 3 < rs.k) load_row(rs.row(q + 3), sb, gb);
        }
      }
    } else {
      // every slot is loaded unconditionally (a slot past the group's last
      // row re-reads that row), so that the compiler counts the loads in
      // flight statically instead of draining them before each load
#pragma unroll
      for (int q = 0; q < NS; ++q) load_row(rs.row(min(q, rs.k - 1)), ring[q], gring[q]);
      if (kSample && i == 0) gather_logits<DT, MODE, FILT>(a, b, g, in);
#pragma unroll
      for (int q = 0; q < 2 * kMaxSpan; ++q) {
        if (q < rs.k)
          slice_pair<DT, R, AL, FILT, kSample>(a, L, ring[q % NS], gring[q % NS], rs.row(q),
                                               tau_of(rs.row(q)), lo);
        if (q + NS < 2 * kMaxSpan)
          load_row(rs.row(min(q + NS, rs.k - 1)), ring[q % NS], gring[q % NS]);
      }
    }
    exchange_set<kSample>(a, L, b, c, rs, FILT);
    if (L.bad) {  // a slice's pairs never arrived (cannot happen in a correct launch)
      write_sentinel(a, b);
      row_exit(a, L, b, nrows, kSample);
      return;
    }
    if (t < 64) {
      if (c == 0 && a.pr_m && lane < rs.k) {
        const int r = rs.row(lane);
        const int slot = probe_slot(a, g, r);
        const float mm = L.M[r];
        a.pr_m[(int64_t)b * (2 * a.G + 1) + slot] = mm;
        // sampling: S relative to the raw max (the rounding of R(m) undone);
        // greedy: the argmax, as a float
        if (a.pr_s)
          a.pr_s[(int64_t)b * (2 * a.G + 1) + slot] =
              !kSample ? (float)__float_as_int(L.S[r])
                       : (mm != NEG_INF ? L.S[r] * ex2(-fmaf(mm, a.k2, -ref_of(mm, a.k2)))
                                        : L.S[r]);
      }
      // the tests at i .. j - 1 (lane p holds x_p, u_p and the logits at x_p);
      // the first that fails, or position g, ends the walk
      const bool valid = (unsigned)in.x < (unsigned)a.V;
      const bool mine = lane >= i && lane < j && lane < g;
      bool fail = true;
      if (mine && valid) {
        if (kSample) {
          const float p = ex2(fmaf(in.tv, a.k2, -ref_of(L.M[lane], a.k2))) / L.S[lane];
          // point-mass drafts: q_i is the indicator of x_i, so q_i(x_i) = 1
          const float q = kPoint ? 1.f
                                 : ex2(fmaf(in.dv, a.k2, -ref_of(L.M[g + 1 + lane], a.k2))) /
                                       L.S[g + 1 + lane];
          if (c == 0 && a.pr_px) {
            a.pr_px[(int64_t)b * a.G + lane] = p;
            a.pr_qx[(int64_t)b * a.G + lane] = q;
          }
          fail = !(in.u * q < p);
        } else {
          fail = in.x != __float_as_int(L.S[lane]);
        }
      }
      const unsigned long long stop = __ballot((mine && fail) || lane == g);
      const unsigned long long win = j >= 64 ? ~0ull : ((1ull << j) - 1);
      const unsigned long long hit = stop & win & ~((1ull << i) - 1);
      int v = 0, at = j;
      if (hit) {
        at = __ffsll((long long)hit) - 1;
        const bool ok = at == g || __builtin_amdgcn_readlane(valid ? 1 : 0, at) != 0;
        v = ok ? 1 : 2;
        // sampling: a row the walk uses must have a finite logit (a dead p_i
        // or q_i fails the test at i, so only the stop position can hold one)
        if (kSample && v == 1 &&
            (L.M[at] == NEG_INF || (kDraft && at < g && L.M[g + 1 + at] == NEG_INF)))
          v = 2;
      }
      if (t == 0) L.pick = v, L.last = at;
    }
    __syncthreads();
    verdict = L.pick;
    if (verdict != 0) {
      n = L.last;
      // the ring holds the group's last two rows: the last position when
      // sampling, the last two otherwise
      const int q = kPer * (n - i);  // t_n's row in the group (d_n follows it)
      if constexpr (NS == 2) {
        if constexpr (kDraft) {
          reread = n < j - 1;
        } else {
          reread = q < rs.k - 2;
          if (!reread && (q & 1)) sa = sb, ga = gb;  // t_n was in sb
        }
      } else {
        // slot s ends holding the group's row min(the last row index equal
        // to s mod NS below 2 kMaxSpan, k - 1) (the loads are unconditional);
        // the stop's rows are used from the ring when that is what their
        // slots hold
        auto resident = [&](int r) {
          const int sl = r % NS;
          return min(sl + NS * ((2 * kMaxSpan - 1 - sl) / NS), rs.k - 1) == r;
        };
        reread = !resident(q) || (kDraft && n < g && !resident(q + 1));
        if (!reread) {
          pick_slot(ring, gring, q % NS, sa, ga);
          if (kDraft) pick_slot(ring, gring, (q + 1) % NS, sb, gb);
        }
      }
      break;
    }
    i = j;
    span = min(2 * span, cap);
  }
  const bool sentinel = verdict == 2;
  if (t < 64) {
    if (c == 0) {
      // lane i owns output position i (gamma_max <= 63); greedy writes the
      // target's argmax at n, the other modes leave it to the draw
      if constexpr (kSample) {
        if (lane <= a.G && !(lane == n && !sentinel))
          a.out_tok[(int64_t)b * (a.G + 1) + lane] = !sentinel && lane < n ? in.x : -1;
      } else {
        if (lane <= a.G) {
          int v = -1;
          if (!sentinel && lane < n)
            v = in.x;
          else if (!sentinel && lane == n)
            v = __float_as_int(L.S[n]);
          a.out_tok[(int64_t)b * (a.G + 1) + lane] = v;
        }
      }
      if (lane == 0) {
        const int kv = a.kv ? a.kv[b] : 0;
        a.out_n[b] = sentinel ? -1 : n;
        a.out_len[b] = sentinel ? kv : kv + n;
      }
    }
    if (kSample) {
      // point mode knocks x_n out of the residual (sampling never reads these)
      const int xn = kPoint ? __builtin_amdgcn_readlane(in.x, n < g ? n : 0) : 0;
      const float tx =
          kPoint ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(in.tv), n < g ? n : 0))
                 : 0.f;
      // u of the draw: u_{n+1} after a rejection at n, u_g for the bonus draw
      const float ustar =
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(in.u), n < g ? n + 1 : g));
      if (t == 0) {
        Decision d;
        d.n = n, d.dead = sentinel, d.resid = n < g;
        d.xn = xn, d.tx = tx, d.ustar = ustar;
        d.mt = L.M[n], d.st = L.S[n];
        d.md = kDraft && n < g ? L.M[g + 1 + n] : 0.f;
        d.sd = kDraft && n < g ? L.S[g + 1 + n] : 1.f;
        L.dec = d;
      }
    }
  }
  if (!kSample) {  // greedy draws nothing
    row_exit(a, L, b, nrows, false);
    return;
  }
  __syncthreads();
  const Decision dc = L.dec;
  if (dc.dead) {
    row_exit(a, L, b, nrows);
    return;
  }
  if (reread) {  // the stop's rows again (read a few microseconds ago: cached)
    load_row(n, sa, ga);
    if (kDraft && n < g) load_row(g + 1 + n, sb, gb);
  }
  if (kDraft && dc.resid && !AL && gb.head != ga.head) {
    // the weights pair element j of both rows: d_n in t_n's register layout
    const char* dp = row_of<DT>(a, b, g, g + 1 + n) + (int64_t)lo * E::kBytes;
    load_slice_as<DT, R>(dp, ga, sb);
  }
  if (!(kDraft && dc.resid)) sb = sa;
  __builtin_amdgcn_s_setprio(1);
  draw_body<DT, R, kPoint, FILT, AL, true>(a, L, b, c, g, lo, nrows, dc, sa, sb, ga);
}

// ------------------------------------------------------------------ filtering
// Top-k / top-p thresholds (the same processing for p and q: "Speculative
// decoding", mhtirogla.ai, "Implementation notes"; tusharamrit, the caveat
// after the proof).  One workgroup per vocabulary row finds tau such that the
// filtered row keeps exactly the entries with l >= tau:
//   top-k: tau_k = the k-th largest value (ties kept);
//   top-p: among the entries kept by top-k, the largest value tau_p such that
//          the entries at or above it carry at least top_p of their mass
//          under softmax(l / T) (all copies of a value together).
// Values are ordered through sortable keys (the float's bits with the sign
// bit flipped, all bits flipped when negative; larger value, larger key) and
// selected by most significant digits, 8 bits per level (two levels for bf16,
// whose keys carry nothing below bit 16; four for fp32), one histogram per
// level over the entries that match the digits chosen so far.  The levels run
// over a candidate list in LDS (the entries above a floor that provably lies
// under the threshold), or over the whole row when the list would overflow.  Masses are
// 2^fma(l, k2, -R(max)) (the weights of the verify) in fixed point, units of
// 2^-42, so their sums are exact integers whatever the order of the additions.
constexpr int kFThreads = 256;
constexpr int kFWaves = kFThreads / 64;
constexpr int kFBins = 256;

struct FArgs {
  const void* tgt;
  const void* dft;
  const int32_t* gam;
  float* thr;  // [B][2G+1]: target rows 0..G, then draft rows 0..G-1
  int B, G, V, NR2, top_k;  // NR2 = 2G+1 slots per batch row
  int drafts;               // 1: draft rows are filtered (sampling), 0: -inf there
  float k2, top_p;
};

constexpr int kFSlots = 32;  // candidate keys each thread can keep in LDS
constexpr int kFCand = kFThreads * kFSlots;

struct FLds {
  unsigned long long h[kFBins];
  uint32_t cand[kFCand];
  float tmax[kFThreads];
  unsigned ccount[kFThreads];  // candidates each thread found
  unsigned long long red[kFWaves];
  unsigned long long mask[kFWaves];
  float fmax[kFWaves];
  int pick;
  unsigned long long above;
};

__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float funkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Digit levels: shift and width of level lv.
template <int DT>
struct FLevels {
  static constexpr int N = DT == SPEC_DTYPE_BF16 ? 2 : 4;
  __device__ static int shift(int lv) { return 24 - 8 * lv; }
  __device__ static int bits(int) { return 8; }
};

__device__ __forceinline__ float fblock_max(float v, FLds& L) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) L.fmax[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = L.fmax[0];
  for (int k = 1; k < kFWaves; ++k) m = fmaxf(m, L.fmax[k]);
  __syncthreads();
  return m;
}

// Inclusive / exclusive prefix sums over the workgroup's threads and the
// total (unsigned 64-bit, exact).
__device__ __forceinline__ void fblock_scan(uint64_t v, FLds& L, uint64_t& incl, uint64_t& excl,
                                            uint64_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t prev;
  const uint64_t x = wave_scan_u64(v, prev);
  if (lane == 63) L.red[w] = x;
  __syncthreads();
  uint64_t off = 0, tot = 0;
  for (int k = 0; k < kFWaves; ++k) {
    if (k < w) off += L.red[k];
    tot += L.red[k];
  }
  incl = off + x;
  excl = off + prev;
  total = tot;
  __syncthreads();
}

// Walking the digits of L.h[0..nb) from the largest down, the first digit at
// which the running sum reaches `need`; `above` = the sum of the digits above
// it, `total` = the sum of all.  need <= total is the caller's guarantee; if
// it did not hold, the lowest non-empty digit is returned.
__device__ __forceinline__ int find_cross(FLds& L, int nb, uint64_t need, uint64_t& above,
                                           uint64_t& total) {
  const int t = threadIdx.x;
  const int per = nb > kFThreads ? nb / kFThreads : 1;
  const int top = nb - 1 - t * per;  // this thread's digits: top, top-1, ..., top-per+1
  uint64_t s = 0;
  for (int i = 0; i < per; ++i)
    if (top - i >= 0) s += L.h[top - i];
  uint64_t incl, excl;
  fblock_scan(s, L, incl, excl, total);
  int th = block_first_m<kFWaves>(s > 0 && incl >= need, L.mask);
  const bool fallback = th < 0;
  if (fallback) {
    // (cannot happen with need <= total) the last thread holding weight
    const unsigned long long m = __ballot(s > 0);
    if ((t & 63) == 0) L.mask[t >> 6] = m;
    __syncthreads();
    for (int k = kFWaves - 1; k >= 0; --k)
      if (L.mask[k]) {
        th = k * 64 + 63 - __clzll((long long)L.mask[k]);
        break;
      }
    __syncthreads();
  }
  if (t == th) {
    uint64_t c = excl;
    int d = -1;
    uint64_t at = 0;
    for (int i = 0; i < per && top - i >= 0; ++i) {
      const uint64_t hv = L.h[top - i];
      if (hv == 0) continue;
      if (fallback || c + hv >= need) {
        d = top - i;
        at = c;
        if (!fallback) break;
      }
      c += hv;
    }
    L.pick = d;
    L.above = at;
  }
  __syncthreads();
  const int d = L.pick;
  above = L.above;
  __syncthreads();
  return d;
}

// Calls f(value) for every element of a row of V entries: 16-byte vector
// loads for the aligned body (sixteen per thread in flight: with about two
// such workgroups per CU the passes are otherwise bound by the latency of
// too few loads), the unaligned head
// and tail element by element.
// VEC (optional): g(fe) is called on each vector's unpacked elements
// instead, so the caller can act on a vector at once.  part > 1: only the
// head and the first 1/part of the vectors.
template <int DT, class F, class VF>
__device__ __forceinline__ void row_for_each_v(const char* row, int V, int part, F f, VF g) {
  using E = Elt<DT>;
  const int t = threadIdx.x;
  int head = (int)(((16u - ((unsigned)(uintptr_t)row & 15u)) & 15u) / E::kBytes);
  if (head > V) head = V;
  const int nv_all = (V - head) / E::kVec;
  const int jb = head + nv_all * E::kVec;
  const int nv = part > 1 ? (nv_all + part - 1) / part : nv_all;
  if (t < head) f(E::one(row, t));
  if (part <= 1 && t < V - jb) f(E::one(row, jb + t));
  const uint4* vp = (const uint4*)(row + head * E::kBytes);
  constexpr int U = 16;
  // the same number of rounds in every lane (g may use cross-lane
  // operations); vectors past the end read as -inf
  for (int q0 = 0; q0 < nv; q0 += kFThreads * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u * kFThreads + t;
      v[u] = q < nv ? vp[q] : make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord,
                                           E::kNegInfWord);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q0 + u * kFThreads >= nv) break;  // uniform
      float fe[E::kVec];
      E::unpack(v[u], fe);
      g(fe);
    }
  }
}

template <int DT, class F>
__device__ __forceinline__ void row_for_each(const char* row, int V, F f) {
  row_for_each_v<DT>(row, V, 1, f, [&](const float* fe) {
#pragma unroll
    for (int e = 0; e < Elt<DT>::kVec; ++e) f(fe[e]);
  });
}

// Histogram bin of a weight 2^e (e <= about 0): bins 1/8 of a unit of e
// wide, the largest weights in the top bin, everything 2^-32 and below in
// bin 0.  Monotone in e, so a bin is a range of values and equal values share
// one.
__device__ __forceinline__ int pmass_bin(float e) {
  const float d = fminf(fmaxf(-e * 8.f, 0.f), (float)(kFBins - 1));
  return kFBins - 1 - (int)d;
}

// The weight 2^e in fixed point: trunc(ex2(e) * 2^42), formed in fp32 as its
// two 32-bit halves: hi = trunc(f * 2^10), lo = trunc((f * 2^10 - hi) * 2^32).
// Every step is exact for 0 <= f < 2^22 (the scalings are powers of two, the
// difference is the fraction bits of f * 2^10), which covers every weight
// here (e <= about 0); checked against the double conversion for every
// float below 2.
__device__ __forceinline__ unsigned long long fixed_mass_e(float e) {
  const float fs = ex2(e) * 1024.f;
  const unsigned hi = (unsigned)fs;
  const unsigned lo = (unsigned)((fs - (float)hi) * 4294967296.f);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long fixed_mass(float l, float k2, float R) {
  return fixed_mass_e(fmaf(l, k2, -R));
}

// Radix selection over the candidate list in LDS (listed) or over the whole
// row: the key of the entry where the count (mass: the fixed-point masses
// against R) from the top reaches `need`, counting keys >= floor_key2 only.
// mass && !given: need is top_p of the mass of those keys (W when non-zero,
// else the first level's histogram total).  packed: the list fills its
// threads' slots in order (top-p alone), so the slots are walked across the
// lanes; else each thread walks its own few filled slots (top-k).
template <int DT>
__device__ __forceinline__ uint32_t radix_select(const FArgs& a, FLds& L, const char* row,
                                                 bool listed, bool packed, float R, bool mass,
                                                 uint64_t need, uint32_t floor_key2, uint64_t W,
                                                 bool given) {
  using Lv = FLevels<DT>;
  const int t = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  for (int lv = 0; lv < Lv::N; ++lv) {
    const int sh = Lv::shift(lv), nb = 1 << Lv::bits(lv);
    for (int i = t; i < nb; i += kFThreads) L.h[i] = 0;
    __syncthreads();
    auto add = [&](uint32_t k) {
      if (k >= floor_key2 && (k & pmask) == prefix) {
        const unsigned long long w = mass ? fixed_mass(funkey(k), a.k2, R) : 1ull;
        if (w) atomicAdd(&L.h[(k >> sh) & (nb - 1)], w);
      }
    };
    if (listed && packed) {
      for (int i = t; i < kFCand; i += kFThreads)
        if ((unsigned)(i % kFSlots) < L.ccount[i / kFSlots]) add(L.cand[i]);
    } else if (listed) {  // this thread's filled slots
      const int n = (int)L.ccount[t];
      for (int j = 0; j < n; ++j) add(L.cand[t * kFSlots + j]);
    } else {
      row_for_each<DT>(row, a.V, [&](float l) { add(fkey(l)); });
    }
    __syncthreads();
    uint64_t above, total;
    if (mass && lv == 0 && !given) {
      // the target: top_p of the mass kept so far, rounded up to a unit
      if (W == 0) {
        uint64_t sum = 0, incl, excl;
        for (int i = t; i < nb; i += kFThreads) sum += L.h[i];
        fblock_scan(sum, L, incl, excl, W);
      }
      need = (uint64_t)ceil((double)a.top_p * (double)W);
      if (need < 1) need = 1;
    }
    const int d = find_cross(L, nb, need, above, total);
    need -= above;
    prefix |= (uint32_t)d << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
  }
  return prefix;
}

// The row whose threshold goes to `out`, or null when the walk cannot use
// this vocabulary row (its threshold is -inf).
template <int DT>
__device__ __forceinline__ const char* filter_row_of(const FArgs& a, int b, int slot) {
  using E = Elt<DT>;
  const int g = a.gam[b];
  const bool is_t = slot <= a.G;
  const bool used =
      g >= 0 && g <= a.G && (is_t ? slot <= g : (a.drafts && slot - a.G - 1 < g));
  if (!used) return nullptr;
  return is_t ? (const char*)a.tgt + ((int64_t)b * (a.G + 1) + slot) * a.V * E::kBytes
              : (const char*)a.dft + ((int64_t)b * a.G + (slot - a.G - 1)) * a.V * E::kBytes;
}

// One workgroup finds the threshold of vocabulary row (b, slot) alone,
// reading the row from memory (one to three passes).
template <int DT>
__device__ __forceinline__ void filter_row(const FArgs& a, int b, int slot, FLds& L) {
  using E = Elt<DT>;
  const int t = threadIdx.x;
  float* out = a.thr + (int64_t)b * (2 * a.G + 1) + slot;
  const char* row = filter_row_of<DT>(a, b, slot);
  if (!row) {
    if (t == 0) *out = NEG_INF;
    return;
  }
  const bool use_k = a.top_k > 0 && a.top_k < a.V;
  const bool use_p = a.top_p < 1.f;

  // A floor under the threshold, so that the selection can work on the
  // entries above it only.  top-k (k <= threads): the k-th largest of the
  // threads' maxima over the first quarter of the row, since k distinct
  // entries reach it.  top-p alone: a histogram of the row's masses over
  // bins of the weight's exponent (1/8 of a unit wide) finds the bin the
  // threshold lies in and the exact mass above it; only that bin's entries
  // become candidates.
  float floor_v = NEG_INF, mx = NEG_INF;
  int p_bin = -1;          // top-p alone: the bin holding the threshold
  uint64_t p_need = 0;     // and the mass still needed within it
  if (use_k && a.top_k <= kFThreads) {
    float tm = NEG_INF;
    row_for_each_v<DT>(row, a.V, 4, [&](float l) { tm = fmaxf(tm, l); }, [&](const float* fe) {
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) tm = fmaxf(tm, fe[e]);
    });
    L.tmax[t] = tm;
    __syncthreads();
    int above = 0;  // rank of this thread's maximum, ties by thread index
    for (int s2 = 0; s2 < kFThreads; ++s2) {
      const float o = L.tmax[s2];
      above += (o > tm) | ((o == tm) & (s2 < t));
    }
    if (above == a.top_k - 1) L.fmax[0] = tm;
    __syncthreads();
    floor_v = L.fmax[0];
    __syncthreads();
  } else if (use_p && !use_k) {
    float tm = NEG_INF;
    row_for_each<DT>(row, a.V, [&](float l) { tm = fmaxf(tm, l); });
    mx = fblock_max(tm, L);
    if (mx == NEG_INF) {  // a dead row: the walk reports it
      if (t == 0) *out = NEG_INF;
      return;
    }
    const float Rp = ref_of(mx, a.k2);
    for (int i = t; i < kFBins; i += kFThreads) L.h[i] = 0;
    __syncthreads();
    // every entry is added (a zero mass adds nothing): no branch per entry
    auto hist = [&](float l) {
      const float e = fmaf(l, a.k2, -Rp);
      atomicAdd(&L.h[pmass_bin(e)], fixed_mass_e(e));
    };
    row_for_each_v<DT>(row, a.V, 1, hist, [&](const float* fe) {
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) hist(fe[e]);
    });
    __syncthreads();
    // the row's total mass: the sum of the bins (exact integers)
    uint64_t ws = 0, incl, excl, W;
    for (int i = t; i < kFBins; i += kFThreads) ws += L.h[i];
    fblock_scan(ws, L, incl, excl, W);
    uint64_t need = (uint64_t)ceil((double)a.top_p * (double)W), above, total;
    if (need < 1) need = 1;
    p_bin = find_cross(L, kFBins, need, above, total);
    p_need = need - above;
  }
  // (the key floor: float comparisons tie -0 with +0, keys put -0 first)
  const uint32_t floor_key =
      floor_v == NEG_INF ? 0u : fkey(floor_v == 0.f ? -0.f : floor_v);

  // the candidates: every entry at or above the floor, each thread into its
  // own kFSlots slots of LDS (no cross-lane work per entry; a thread that
  // finds more sends the row to the whole-row selection); the row's largest
  // value; the total mass when top-p runs alone (its largest value is known
  // by now).  A float compare selects them (it also takes -0 against a +0
  // floor: a harmless extra candidate).
  const bool p_alone = use_p && !use_k;
  float tm2 = NEG_INF;
  unsigned mine = 0;
  if (p_alone) {
    // the threshold's bin: a few hundred entries, so each wave compacts its
    // finds into its own region of the candidate array (a ballot per entry;
    // the branch is wave-uniform and rarely taken).  First a range test on
    // the values (the bin's edges, widened), then the exact bin test.
    const float Rp = ref_of(mx, a.k2);
    const float e_lo = -(float)(kFBins - p_bin) * 0.125f, e_hi = e_lo + 0.125f;
    float lo = p_bin > 0 ? (Rp + e_lo) / a.k2 : NEG_INF;
    float hi = p_bin < kFBins - 1 ? (Rp + e_hi) / a.k2 : INFINITY;
    lo -= 1e-3f * (1.f + fabsf(lo));
    hi += 1e-3f * (1.f + fabsf(hi));
    constexpr unsigned kRegion = kFCand / kFWaves;
    uint32_t* region = L.cand + (t >> 6) * kRegion;
    unsigned cw = 0;  // this wave's finds (uniform)
    auto one = [&](float l) {
      if (__ballot((l >= lo) & (l <= hi))) {
        const bool in = (l >= lo) & (l <= hi) && pmass_bin(fmaf(l, a.k2, -Rp)) == p_bin;
        const unsigned long long m = __ballot(in);
        if (in) {
          const unsigned at = cw + (unsigned)__builtin_amdgcn_mbcnt_hi(
                                       (unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
          if (at < kRegion) region[at] = fkey(l);
        }
        cw += (unsigned)__popcll(m);
      }
    };
    // the unaligned head and tail elements come in some lanes only: kept
    // aside, then taken with every lane (the ballots need whole waves)
    float hv = NEG_INF, tv = NEG_INF;
    bool got_h = false;
    auto aside = [&](float l) {
      if (got_h) tv = l;
      else hv = l, got_h = true;
    };
    row_for_each_v<DT>(row, a.V, 1, aside, [&](const float* fe) {
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) one(fe[e]);
    });
    one(hv);
    one(tv);
    // in the per-thread slot layout the selection reads: thread t's slots
    // are entries [32 t', 32 t' + 32) of its wave's region, t' = t mod 64
    const int rel = (t & 63) * kFSlots;
    const int have = (int)cw - rel;
    mine = cw > kRegion ? (unsigned)kFSlots + 1u  // overflow: the whole row
                        : (unsigned)(have < 0 ? 0 : have > kFSlots ? kFSlots : have);
  } else {
    uint32_t* slots = L.cand + t * kFSlots;
    auto one = [&](float l) {
      tm2 = fmaxf(tm2, l);
      if (l >= floor_v) {
        if (mine < (unsigned)kFSlots) slots[mine] = fkey(l);
        ++mine;
      }
    };
    row_for_each_v<DT>(row, a.V, 1, one, [&](const float* fe) {
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) one(fe[e]);
    });
  }
  L.ccount[t] = mine;
  if (!p_alone) mx = fblock_max(tm2, L);  // (top-p alone: known from its first pass)
  if (mx == NEG_INF) {  // a dead row: the walk reports it
    if (t == 0) *out = NEG_INF;
    return;
  }
  const float R = ref_of(mx, a.k2);
  __syncthreads();
  const bool listed = __syncthreads_and(mine <= (unsigned)kFSlots) != 0;  // else: whole-row passes

  auto select = [&](bool mass, uint64_t need, uint32_t floor_key2, uint64_t W,
                    bool given) -> uint32_t {
    return radix_select<DT>(a, L, row, listed, p_alone, R, mass, need, floor_key2, W, given);
  };
  uint32_t key = 0;
  if (use_k) key = select(false, (uint64_t)a.top_k, floor_key, 0, false);
  if (use_p) {
    // top-k kept: top_p of its own mass (all of it is among the
    // candidates); top-p alone: the mass still needed within the
    // threshold's bin (its candidates; the whole row, with the row's
    // target, when they overflow)
    const uint32_t kp = p_alone ? (listed ? select(true, p_need, 0, 0, true)
                                          : select(true, 0, 0, 0, false))
                                : select(true, 0, key, 0, false);
    key = kp > key ? kp : key;
  }
  // a bf16 key's low 16 bits: zero for positive values, all ones for negative
  if (DT == SPEC_DTYPE_BF16) key |= (key & 0x80000000u) ? 0u : 0xffffu;
  if (t == 0) *out = (use_k || use_p) ? funkey(key) : NEG_INF;
}

template <int DT>
__global__ __launch_bounds__(kFThreads) void filter_kernel(FArgs a) {
  __shared__ FLds L;
  filter_row<DT>(a, (int)(blockIdx.x / (unsigned)a.NR2), (int)(blockIdx.x % (unsigned)a.NR2), L);
}

// ------------------------------------------------------------------ probes
__global__ __launch_bounds__(kThreads) void fill_ninf_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = NEG_INF;
}

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

// prio: phase priorities (the whole grid resident).  Grids larger than the
// chip come from the largest slices (R = 4) unless the tuning forces smaller
// ones, so only R = 4 has a variant without them.
template <int DT, int MODE, bool AL, bool FILT>
void launch_r(int R, bool prio, dim3 grid, hipStream_t s, const Args& a) {
  if (R == 1)
    hipLaunchKernelGGL((verify_kernel<DT, MODE, 1, AL, FILT, true>), grid, dim3(kThreads), 0, s, a);
  else if (R == 2)
    hipLaunchKernelGGL((verify_kernel<DT, MODE, 2, AL, FILT, true>), grid, dim3(kThreads), 0, s, a);
  else if (prio)
    hipLaunchKernelGGL((verify_kernel<DT, MODE, 4, AL, FILT, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((verify_kernel<DT, MODE, 4, AL, FILT, false>), grid, dim3(kThreads), 0, s, a);
}

template <int DT, int MODE, bool AL, bool FILT>
void launch_rows_r(int R, dim3 grid, hipStream_t s, const Args& a) {
  if (R == 1)
    hipLaunchKernelGGL((verify_rows_kernel<DT, MODE, 1, AL, FILT>), grid, dim3(kThreads), 0, s, a);
  else if (R == 2)
    hipLaunchKernelGGL((verify_rows_kernel<DT, MODE, 2, AL, FILT>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((verify_rows_kernel<DT, MODE, 4, AL, FILT>), grid, dim3(kThreads), 0, s, a);
}

// greedy never filters (the filters keep the largest logit)
template <int DT, int MODE>
void launch_rows(int R, bool al, bool filt, dim3 grid, hipStream_t s, const Args& a) {
  constexpr bool kCanFilter = MODE != SPEC_MODE_GREEDY;
  if (kCanFilter && filt) {
    if (al)
      launch_rows_r<DT, MODE, true, kCanFilter>(R, grid, s, a);
    else
      launch_rows_r<DT, MODE, false, kCanFilter>(R, grid, s, a);
  } else {
    if (al)
      launch_rows_r<DT, MODE, true, false>(R, grid, s, a);
    else
      launch_rows_r<DT, MODE, false, false>(R, grid, s, a);
  }
}

// greedy never filters (the filters keep the largest logit)
template <int DT, int MODE>
void launch(int R, bool prio, bool al, bool filt, dim3 grid, hipStream_t s, const Args& a) {
  constexpr bool kCanFilter = MODE != SPEC_MODE_GREEDY;
  if (kCanFilter && filt) {
    if (al)
      launch_r<DT, MODE, true, kCanFilter>(R, prio, grid, s, a);
    else
      launch_r<DT, MODE, false, kCanFilter>(R, prio, grid, s, a);
  } else {
    if (al)
      launch_r<DT, MODE, true, false>(R, prio, grid, s, a);
    else
      launch_r<DT, MODE, false, false>(R, prio, grid, s, a);
  }
}

bool filter_args_ok(int top_k, float top_p) { return top_k >= 0 && top_p > 0.f && top_p <= 1.f; }

// Whether a call filters at all (greedy never does: the filters keep the
// largest logit).
bool filters(int mode, int V, int top_k, float top_p) {
  return mode != SPEC_MODE_GREEDY && ((top_k > 0 && top_k < V) || top_p < 1.f);
}

void launch_filter(const FArgs& f, int dtype, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)f.B * f.NR2));
  if (dtype == SPEC_DTYPE_BF16)
    hipLaunchKernelGGL((filter_kernel<SPEC_DTYPE_BF16>), grid, dim3(kFThreads), 0, s, f);
  else
    hipLaunchKernelGGL((filter_kernel<SPEC_DTYPE_F32>), grid, dim3(kFThreads), 0, s, f);
}

FArgs filter_args(const void* tgt, const void* dft, const int32_t* gam, float* thr, int B, int G,
                  int V, float T, int mode, int top_k, float top_p) {
  FArgs f;
  f.tgt = tgt, f.dft = dft ? dft : tgt, f.gam = gam, f.thr = thr;
  f.B = B, f.G = G, f.V = V, f.NR2 = 2 * G + 1, f.drafts = mode == SPEC_MODE_SAMPLE;
  f.top_k = top_k, f.top_p = top_p;
  f.k2 = (float)(1.4426950408889634 / (double)T);
  return f;
}

int run(const void* tgt, const void* dft, const int32_t* tok, const float* uni, const int32_t* gam,
        const int32_t* kv, int B, int G, int V, int dtype, float T, int mode, int top_k,
        float top_p, int32_t* out_tok, int32_t* out_n, int32_t* out_len, void* ws,
        size_t ws_bytes, void* stream, float* px, float* qx, float* pz, float* pm, float* ps,
        float* pflo, float* pfhi) {
  Plan p;
  int st = make_plan(B, G, V, dtype, mode, &p);
  if (st != SPEC_OK) return st;
  if (!filter_args_ok(top_k, top_p)) return SPEC_ERR_ARG;
  const bool sample = mode == SPEC_MODE_SAMPLE;
  const bool draws = mode != SPEC_MODE_GREEDY;
  const bool filt = filters(mode, V, top_k, top_p);
  if (!tgt || !gam || !out_tok || !out_n || !out_len) return SPEC_ERR_NULL;
  if (G > 0 && !tok) return SPEC_ERR_NULL;
  if ((sample && G > 0 && !dft) || (draws && !uni)) return SPEC_ERR_NULL;
  if (draws && !(T > 0.f && isfinite(T))) return SPEC_ERR_ARG;
  if (!ws || ws_bytes < p.bytes) return SPEC_ERR_WORKSPACE;
  const size_t e = dtype == SPEC_DTYPE_F32 ? 4 : 2;
  if (!sample) dft = nullptr;  // only sampling reads draft logits
  if (!aligned(tgt, e) || (dft && !aligned(dft, e))) return SPEC_ERR_ALIGN;
  if ((pflo == nullptr) != (pfhi == nullptr)) return SPEC_ERR_NULL;
  const void* four[] = {tok, uni, gam, kv, out_tok, out_n, out_len, px, qx, pz, pm, ps, pflo, pfhi};
  for (const void* q : four)
    if (q && !aligned(q, 4)) return SPEC_ERR_ALIGN;
  if (!aligned(ws, 256)) return SPEC_ERR_ALIGN;

  Args a;
  a.tgt = tgt, a.dft = dft ? dft : tgt, a.tok = tok, a.uni = uni, a.gam = gam, a.kv = kv;
  a.out_tok = out_tok, a.out_n = out_n, a.out_len = out_len;
  a.pr_px = px, a.pr_qx = qx, a.pr_z = pz, a.pr_m = pm, a.pr_s = ps;
  a.pr_flo = pflo, a.pr_fhi = pfhi;
  char* w = (char*)ws;
  a.hdr = (unsigned*)w;
  a.ctr = (unsigned*)(w + p.off_ctr);
  a.part = (uint64_t*)(w + p.off_part);
  a.wsum = (uint64_t*)(w + p.off_wsum);
  a.thr = filt ? (const float*)(w + p.off_thr) : nullptr;
  a.B = B, a.G = G, a.V = V, a.NC = p.NC, a.CL = p.CL, a.NR = p.NR;
  a.k2d = draws ? 1.4426950408889634 / (double)T : 1.0;
  a.k2 = (float)a.k2d;
  a.max_spin = 1u << 22;  // ~0.2 s of polling: far beyond any legitimate wait
  // phase priorities only when every workgroup is resident from the start
  // (four per CU is what the largest variants' registers allow)
  const int cus = device_cus();
  const bool prio = cus > 0 && p.total <= (int64_t)4 * cus;
  hipStream_t s = (hipStream_t)stream;
  dim3 grid((unsigned)p.total);
  // every row 16-byte aligned: both bases aligned and a row a whole number
  // of 16-byte vectors
  const bool al = aligned(tgt, 16) && (!sample || G == 0 || aligned(dft, 16)) &&
                  ((size_t)V * e) % 16 == 0;
  if (filt) {  // the thresholds first, into the workspace, on the same stream
    launch_filter(filter_args(tgt, dft, gam, (float*)(w + p.off_thr), B, G, V, T, mode, top_k,
                              top_p),
                  dtype, s);
    const int hs = hip_status(hipGetLastError());
    if (hs != SPEC_OK) return hs;
  }
  // the rows are read position by position, up to the walk's stop (unless
  // the one-pass stream is asked for)
  if (!(g_tune.flags & SPEC_TUNE_ONE_PASS)) {
    if (dtype == SPEC_DTYPE_BF16) {
      if (sample)
        launch_rows<SPEC_DTYPE_BF16, SPEC_MODE_SAMPLE>(p.R, al, filt, grid, s, a);
      else if (draws)
        launch_rows<SPEC_DTYPE_BF16, SPEC_MODE_POINT>(p.R, al, filt, grid, s, a);
      else
        launch_rows<SPEC_DTYPE_BF16, SPEC_MODE_GREEDY>(p.R, al, false, grid, s, a);
    } else {
      if (sample)
        launch_rows<SPEC_DTYPE_F32, SPEC_MODE_SAMPLE>(p.R, al, filt, grid, s, a);
      else if (draws)
        launch_rows<SPEC_DTYPE_F32, SPEC_MODE_POINT>(p.R, al, filt, grid, s, a);
      else
        launch_rows<SPEC_DTYPE_F32, SPEC_MODE_GREEDY>(p.R, al, false, grid, s, a);
    }
    return hip_status(hipGetLastError());
  }
  if (dtype == SPEC_DTYPE_BF16) {
    if (sample)
      launch<SPEC_DTYPE_BF16, SPEC_MODE_SAMPLE>(p.R, prio, al, filt, grid, s, a);
    else if (draws)
      launch<SPEC_DTYPE_BF16, SPEC_MODE_POINT>(p.R, prio, al, filt, grid, s, a);
    else
      launch<SPEC_DTYPE_BF16, SPEC_MODE_GREEDY>(p.R, prio, al, false, grid, s, a);
  } else {
    if (sample)
      launch<SPEC_DTYPE_F32, SPEC_MODE_SAMPLE>(p.R, prio, al, filt, grid, s, a);
    else if (draws)
      launch<SPEC_DTYPE_F32, SPEC_MODE_POINT>(p.R, prio, al, filt, grid, s, a);
    else
      launch<SPEC_DTYPE_F32, SPEC_MODE_GREEDY>(p.R, prio, al, false, grid, s, a);
  }
  return hip_status(hipGetLastError());
}

// ------------------------------------------------------------------ static workspace
// The workspace of spec_verify_noalloc: one array per device, loaded with the
// library's code object (zero-initialised) and held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): it uses the address hipGetSymbolAddress
// returns for the current device, asked once per device.
__device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_WORKSPACE_BYTES];

// Device address of this device's copy of `scratch` (nullptr on error, with
// the HIP error in *err).
void* scratch_ptr(int dev, hipError_t* err) {
  static std::atomic<void*> cached[64];
  *err = hipSuccess;
  if (dev >= 0 && dev < 64) {
    void* p = cached[dev].load(std::memory_order_acquire);
    if (p) return p;
  }
  void* p = nullptr;
  *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || !p) {
    if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
    return nullptr;
  }
  if (dev >= 0 && dev < 64) cached[dev].store(p, std::memory_order_release);
  return p;
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
             gamma_max, V, dtype, temperature, mode, 0, 1.f, out_tokens, out_n_accepted,
             out_new_len, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, nullptr,
             nullptr, nullptr, nullptr);
}

int spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms,
                        const int32_t* gamma_per_row, const int32_t* kv_len_in, int B,
                        int gamma_max, int V, int dtype, float temperature, int mode,
                        int32_t* out_tokens, int32_t* out_n_accepted, int32_t* out_new_len,
                        void* stream) {
  Plan p;
  const int st = make_plan(B, gamma_max, V, dtype, mode, &p);
  if (st != SPEC_OK) return st;
  if (p.bytes > (size_t)SPEC_NOALLOC_WORKSPACE_BYTES) return SPEC_ERR_WORKSPACE;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  void* ws = scratch_ptr(dev, &e);
  if (!ws) return hip_status(e);
  // the previous call on this device left the region zero unless it gave up
  // waiting; clear it anyway (a fill kernel: no memset node in a graph)
  const size_t n16 = p.bytes / 16;
  size_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint4*)ws, n16, (unsigned char*)ws + n16 * 16,
                     (int)(p.bytes % 16));
  const int hs = hip_status(hipGetLastError());
  if (hs != SPEC_OK) return hs;
  return run(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row, kv_len_in, B,
             gamma_max, V, dtype, temperature, mode, 0, 1.f, out_tokens, out_n_accepted,
             out_new_len, ws, p.bytes, stream, nullptr, nullptr, nullptr, nullptr, nullptr,
             nullptr, nullptr);
}

int spec_verify_probe(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms,
                      const int32_t* gamma_per_row, const int32_t* kv_len_in, int B,
                      int gamma_max, int V, int dtype, float temperature, int mode,
                      int32_t* out_tokens, int32_t* out_n_accepted, int32_t* out_new_len,
                      void* workspace, size_t workspace_bytes, void* stream, float* out_px,
                      float* out_qx, float* out_z, float* out_m, float* out_s, float* out_f_lo,
                      float* out_f_hi) {
  if ((out_px == nullptr) != (out_qx == nullptr)) return SPEC_ERR_NULL;
  return run(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row, kv_len_in, B,
             gamma_max, V, dtype, temperature, mode, 0, 1.f, out_tokens, out_n_accepted,
             out_new_len, workspace, workspace_bytes, stream, out_px, out_qx, out_z, out_m, out_s,
             out_f_lo, out_f_hi);
}

int spec_verify_filtered(const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const float* uniforms,
                         const int32_t* gamma_per_row, const int32_t* kv_len_in, int B,
                         int gamma_max, int V, int dtype, float temperature, int mode, int top_k,
                         float top_p, int32_t* out_tokens, int32_t* out_n_accepted,
                         int32_t* out_new_len, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return run(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row, kv_len_in, B,
             gamma_max, V, dtype, temperature, mode, top_k, top_p, out_tokens, out_n_accepted,
             out_new_len, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, nullptr,
             nullptr, nullptr, nullptr);
}

int spec_verify_filtered_probe(const void* target_logits, const void* draft_logits,
                               const int32_t* draft_tokens, const float* uniforms,
                               const int32_t* gamma_per_row, const int32_t* kv_len_in, int B,
                               int gamma_max, int V, int dtype, float temperature, int mode,
                               int top_k, float top_p, int32_t* out_tokens,
                               int32_t* out_n_accepted, int32_t* out_new_len, void* workspace,
                               size_t workspace_bytes, void* stream, float* out_px, float* out_qx,
                               float* out_z, float* out_m, float* out_s, float* out_f_lo,
                               float* out_f_hi) {
  if ((out_px == nullptr) != (out_qx == nullptr)) return SPEC_ERR_NULL;
  return run(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row, kv_len_in, B,
             gamma_max, V, dtype, temperature, mode, top_k, top_p, out_tokens, out_n_accepted,
             out_new_len, workspace, workspace_bytes, stream, out_px, out_qx, out_z, out_m, out_s,
             out_f_lo, out_f_hi);
}

int spec_filter_thresholds(const void* target_logits, const void* draft_logits,
                           const int32_t* gamma_per_row, int B, int gamma_max, int V, int dtype,
                           float temperature, int mode, int top_k, float top_p, float* out_thr,
                           void* stream) {
  if (B < 1 || V < 1 || V > kMaxVocab || gamma_max < 0 || gamma_max > SPEC_GAMMA_MAX_LIMIT)
    return SPEC_ERR_SHAPE;
  if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return SPEC_ERR_ARG;
  if (mode != SPEC_MODE_SAMPLE && mode != SPEC_MODE_POINT) return SPEC_ERR_ARG;
  if (!(temperature > 0.f && isfinite(temperature)) || !filter_args_ok(top_k, top_p))
    return SPEC_ERR_ARG;
  if (!target_logits || !gamma_per_row || !out_thr) return SPEC_ERR_NULL;
  if (mode == SPEC_MODE_SAMPLE && gamma_max > 0 && !draft_logits) return SPEC_ERR_NULL;
  if ((int64_t)B * (2 * gamma_max + 1) >= ((int64_t)1 << 31)) return SPEC_ERR_SHAPE;
  const size_t e = dtype == SPEC_DTYPE_F32 ? 4 : 2;
  if (mode != SPEC_MODE_SAMPLE) draft_logits = nullptr;
  if (!aligned(target_logits, e) || (draft_logits && !aligned(draft_logits, e)) ||
      !aligned(gamma_per_row, 4) || !aligned(out_thr, 4))
    return SPEC_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (!filters(mode, V, top_k, top_p)) {
    // nothing is cut: every threshold is -inf
    const size_t n = (size_t)B * (2 * gamma_max + 1);
    hipLaunchKernelGGL(fill_ninf_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, out_thr, n);
    return hip_status(hipGetLastError());
  }
  launch_filter(filter_args(target_logits, draft_logits, gamma_per_row, out_thr, B, gamma_max, V,
                            temperature, mode, top_k, top_p),
                dtype, s);
  return hip_status(hipGetLastError());
}

int spec_verify_plan(int B, int gamma_max, int V, int dtype, int mode, int64_t* out) {
  if (!out) return SPEC_ERR_NULL;
  Plan p;
  int st = make_plan(B, gamma_max, V, dtype, mode, &p);
  if (st != SPEC_OK) return st;
  out[0] = p.total, out[1] = p.NC, out[2] = p.CL, out[3] = p.R;
  out[4] = p.NR, out[5] = kThreads, out[6] = (int64_t)p.bytes, out[7] = g_tune.target_workgroups;
  return SPEC_OK;
}

int spec_verify_tune(int vectors, int target_workgroups, int flags) {
  if ((flags & ~SPEC_TUNE_ONE_PASS) != 0) return SPEC_ERR_ARG;
  if (vectors != 0 && vectors != 1 && vectors != 2 && vectors != 4) return SPEC_ERR_ARG;
  if (target_workgroups < 0) return SPEC_ERR_ARG;
  Tuning t;
  t.vectors = vectors;
  if (target_workgroups) t.target_workgroups = target_workgroups;
  t.flags = flags;
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
    case SPEC_ERR_ARG: return "invalid argument (mode, dtype, temperature or tuning)";
    case SPEC_ERR_WORKSPACE: return "workspace missing or too small";
    case SPEC_ERR_ALIGN: return "misaligned pointer";
    default: break;
  }
  if (status <= SPEC_ERR_HIP) return hipGetErrorString((hipError_t)(SPEC_ERR_HIP - status));
  return "unknown status";
}

int spec_verify_version(void) { return 400; }

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
