/*
 * spec_oracle.c -- plain, slow, double-precision CPU oracle for the batched
 * verify step of speculative decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library and must never be used as a
 * fallback for it.
 *
 * What it computes (one batch row b, draft length g = gamma[b]):
 *
 *   Sources: "Speculative decoding" (mhtirogla.ai), sections "How it works"
 *   steps 2-5 and "Code" (the verify function); "Speculative decoding: the
 *   secretary who types ahead of the boss" (blog.lo0.es), section "The bare
 *   mechanism", step 3; "Speculative Decoding" (inference.tusharamrit.in),
 *   the loop and the modified rejection-sampling rule; "Speculative
 *   Decoding" (tokentrails.org), steps 2 and 4 and its code block.
 *
 *   1. p_i = softmax(target_logits[b,i,:] / T) for i = 0..g (row g is the
 *      bonus distribution), q_i = softmax(draft_logits[b,i,:] / T) for
 *      i = 0..g-1.  Both sides get the same temperature processing (mhtirogla
 *      "Implementation notes"; tusharamrit caveat after the proof).
 *   2. Walk i = 0..g-1 left to right with draft token x = x_i and uniform u_i:
 *      accept when u_i * q_i(x) < p_i(x) (the division-free form of
 *      u < p/q used in the mhtirogla code); stop at the first rejection.
 *   3. Rejection at n: draw from norm(max(0, p_n - q_n)) with the next unused
 *      uniform u_{n+1}.  All g accepted: draw the bonus token from p_g with
 *      u_g.  The draw is the inverse CDF: tau = u * Z, return the smallest j
 *      with tau < sum_{k<=j} w_k (the mhtirogla `sample`, which scales u by
 *      the sum so an unnormalised weight vector is fine).
 *   4. Greedy mode: accept while x_i equals the target argmax g_i (lowest
 *      index on ties), emit g_n at the first disagreement or g_g when all
 *      agree (mhtirogla "How it works", last paragraph; tokentrails step 2
 *      and its code block).
 *   5. KV rollback: the new cache length is kv_len_in + n (mhtirogla step 5,
 *      "truncate the length").
 *   6. Filtering (top-k, top-p): the same processing applied to p and q
 *      (mhtirogla "Implementation notes"; tusharamrit, the caveat after the
 *      proof).  With logits l and temperature T, top-k keeps every l_j at or
 *      above the k-th largest value (ties kept), then top-p keeps, among those,
 *      the smallest set of largest values whose mass under softmax(l/T)
 *      reaches top_p of the top-k-kept mass (all elements of a value
 *      together).  The kept entries are renormalised; the rest get 0.
 *   7. Point-mass drafts (mode OR_POINT): the drafter proposes x_i outright
 *      -- an n-gram / prompt-lookup match (mhtirogla "Variants" and
 *      "Implementation notes"; tusharamrit "Self-speculation") or a greedy
 *      draft (tokentrails code block) -- so q_i is the indicator of x_i and
 *      no draft logits exist.  Steps 2-3 apply unchanged with that q_i: the
 *      test becomes u_i * 1 < p_i(x_i), and the residual max(0, p_n - q_n)
 *      is p_n with x_n removed.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   - temperature: softmax(logit / T), T > 0 required when sampling; greedy
 *     ignores T.
 *   - uniforms: one stream of gamma_max+1 per row, consumed in order: u_0..u_n
 *     by the tests, then the next unused one by the single draw.
 *   - inverse-CDF fallback: when no j satisfies tau < C_j (rounding), the last
 *     index with positive weight (the page's "last index" could pick a
 *     zero-probability token).
 *   - residual mass Z == 0 after a rejection (impossible in exact arithmetic):
 *     draw from p_n with the same uniform and count it.
 *   - bonus normaliser: the bonus row's own sum.
 *   - data errors (gamma outside [0, gamma_max], a tested draft token outside
 *     [0, V), or, when sampling, a row the walk uses -- p_i and q_i of a
 *     tested position, p_g for the bonus -- whose logits are all -inf; rows
 *     after the stop are never used): n_accepted = -1, tokens all -1,
 *     new_len = kv_len_in.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_SAMPLE 0
#define OR_GREEDY 1
#define OR_POINT 2

/* Mutations used only by negative-control tests, to show that the
 * statistical tests can detect the classic mistakes named on the pages
 * (mhtirogla "Pitfalls"; tusharamrit, the naive rule and the residual). */
#define OR_FAULT_NONE 0
#define OR_FAULT_NO_CLAMP 1      /* residual p - q without max(0, .)        */
#define OR_FAULT_UNSCALED_TAU 2  /* threshold u instead of u * Z             */
#define OR_FAULT_RESAMPLE_P 3    /* after a rejection draw from p, not residual */
#define OR_FAULT_GREEDY_RULE 4   /* accept iff x == argmax p while sampling   */
#define OR_FAULT_FILTER_P_ONLY 5 /* top-k / top-p applied to p but not to q    */

typedef struct {
  const void* target;
  const void* draft;
  int dtype;
  const int32_t* tokens;
  const float* uniforms;
  const int32_t* gamma;
  const int32_t* kv_len;
  int B, G, V;
  double T;
  int mode;
  int fault;
  int top_k;      /* 0: off */
  double top_p;   /* 1: off */
} oracle_ctx;

/* Exact widening of one stored logit to double. */
static double widen(const oracle_ctx* c, const void* base, size_t k) {
  if (c->dtype == OR_F32) return (double)((const float*)base)[k];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[k] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Offset (in elements) of vocabulary row (b, i) in a [B, rows, V] tensor. */
static size_t row_off(const oracle_ctx* c, int b, int rows, int i) {
  return ((size_t)b * (size_t)rows + (size_t)i) * (size_t)c->V;
}

static int cmp_desc(const void* a, const void* b) {
  const double x = *(const double*)a, y = *(const double*)b;
  return (x < y) - (x > y);
}

/* Filtering threshold of one row whose largest logit is m (finite): the
 * filtered distribution keeps exactly the entries with l_j >= tau; -inf when
 * nothing is cut.  top-k: tau_k = the k-th largest value.  top-p: walking the
 * distinct values from the largest, tau_p = the first value at which the mass
 * of everything at or above it reaches top_p * W, W the mass at or above
 * tau_k (masses exp((l - m)/T), summed in that descending order).
 * margin_out: how far that crossing is from top_p * W, relative to W (the
 * smaller of the gaps just before and at the chosen value); +inf when top-p
 * cuts nothing. */
static double filter_threshold(const oracle_ctx* c, const void* base, size_t off, double m,
                               double* margin_out) {
  const int V = c->V;
  if (margin_out) *margin_out = INFINITY;
  const int use_k = c->top_k > 0 && c->top_k < V;
  const int use_p = c->top_p < 1.0;
  if (!use_k && !use_p) return -INFINITY;
  double* v = (double*)malloc(sizeof(double) * (size_t)V);
  for (int j = 0; j < V; ++j) v[j] = widen(c, base, off + j);
  qsort(v, (size_t)V, sizeof(double), cmp_desc);
  double tau = -INFINITY;
  int n = V;  /* entries kept by top-k: a prefix of v */
  if (use_k) {
    tau = v[c->top_k - 1];
    while (n > 0 && v[n - 1] < tau) --n;
  }
  if (use_p) {
    double w_all = 0.0;
    for (int i = 0; i < n; ++i) w_all += exp((v[i] - m) / c->T);
    const double target = c->top_p * w_all;
    double cum = 0.0;
    int i = 0;
    while (i < n) {
      const double val = v[i];
      const double before = cum;
      while (i < n && v[i] == val) cum += exp((v[i++] - m) / c->T);
      if (cum >= target) {
        if (val > tau) tau = val;
        if (margin_out) {
          const double gap = fmin(cum - target, target - before);
          *margin_out = w_all > 0.0 ? gap / w_all : INFINITY;
        }
        break;
      }
    }
  }
  free(v);
  return tau;
}

/* p = softmax(logits / T) in double over the entries with l_j >= tau (the
 * others get 0; tau = -inf keeps all).  Writes the raw-logit maximum and the
 * sum S = sum_{kept j} exp((l_j - max)/T).  Returns 0 when every logit is
 * -inf.  margin_out (optional): the top-p margin of filter_threshold. */
static int softmax_row(const oracle_ctx* c, const void* base, size_t off,
                       double* prob, double* m_out, double* s_out, double* margin_out) {
  const int V = c->V;
  double m = -INFINITY;
  for (int j = 0; j < V; ++j) {
    double l = widen(c, base, off + j);
    if (l > m) m = l;
  }
  if (m_out) *m_out = m;
  if (margin_out) *margin_out = INFINITY;
  if (m == -INFINITY) {
    if (s_out) *s_out = 0.0;
    return 0;
  }
  const double tau = filter_threshold(c, base, off, m, margin_out);
  double s = 0.0;
  for (int j = 0; j < V; ++j) {
    double l = widen(c, base, off + j);
    double e = l >= tau ? exp((l - m) / c->T) : 0.0;
    prob[j] = e;
    s += e;
  }
  for (int j = 0; j < V; ++j) prob[j] /= s;
  if (s_out) *s_out = s;
  return 1;
}

/* Lowest index of the largest raw logit of one row (float comparison, so
 * -0 and +0 tie and the lower index wins). */
static int argmax_row(const oracle_ctx* c, size_t off) {
  int best = 0;
  double bv = widen(c, c->target, off);
  for (int j = 1; j < c->V; ++j) {
    double l = widen(c, c->target, off + j);
    if (l > bv) {
      bv = l;
      best = j;
    }
  }
  return best;
}

/* Inverse-CDF draw over non-negative weights w[0..V): tau = u * Z, the
 * smallest j with tau < C_j; fallback: the last index with w > 0.
 * Writes Z.  cdf_out (optional) receives C_j / Z; flo_out and fhi_out
 * (optional) the drawn index's bracket C_{j-1} / Z and C_j / Z. */
static int draw_index(const oracle_ctx* c, const double* w, double u,
                      double* z_out, double* cdf_out, double* flo_out, double* fhi_out) {
  const int V = c->V;
  double z = 0.0;
  for (int j = 0; j < V; ++j) z += w[j];
  if (z_out) *z_out = z;
  double tau = (c->fault == OR_FAULT_UNSCALED_TAU) ? u : u * z;
  int pick = -1, last_pos = -1;
  double acc = 0.0, pick_lo = 0.0, pick_hi = 0.0, last_lo = 0.0, last_hi = 0.0;
  for (int j = 0; j < V; ++j) {
    const double before = acc;
    acc += w[j];
    if (cdf_out) cdf_out[j] = acc / z;
    if (w[j] > 0.0) last_pos = j, last_lo = before, last_hi = acc;
    if (pick < 0 && tau < acc) pick = j, pick_lo = before, pick_hi = acc;
  }
  if (pick < 0) {
    pick = (last_pos >= 0) ? last_pos : V - 1;
    pick_lo = last_lo, pick_hi = last_hi;
  }
  if (flo_out) *flo_out = pick_lo / z;
  if (fhi_out) *fhi_out = pick_hi / z;
  return pick;
}

typedef struct {
  double* px;       /* [G] p_i(x_i) for tested positions (NaN otherwise)   */
  double* qx;       /* [G] q_i(x_i)                                         */
  double* z;        /* [1] normaliser of the drawn distribution             */
  double* m;        /* [2G+1] raw-logit max per vocabulary row (t0..tG, d0..dG-1) */
  double* s;        /* [2G+1] exp-sum relative to that max                  */
  int32_t* draw_pos;   /* [1] position whose distribution was drawn from (-1: none) */
  int32_t* zero_resid; /* [1] 1 when the residual mass was exactly 0         */
  double* cdf;      /* [V] normalised CDF of the drawn distribution, or NULL */
  double* fmargin;  /* [1] smallest top-p margin over the rows the walk used */
  double* flo;      /* [1] normalised CDF just below the drawn token          */
  double* fhi;      /* [1] normalised CDF at the drawn token                  */
} row_diag;

static void write_sentinel(const oracle_ctx* c, int b, int32_t* tok, int32_t* n_out,
                           int32_t* len_out) {
  for (int i = 0; i <= c->G; ++i) tok[(size_t)b * (c->G + 1) + i] = -1;
  n_out[b] = -1;
  len_out[b] = c->kv_len ? c->kv_len[b] : 0;
}

static void verify_row(const oracle_ctx* c, int b, int32_t* out_tokens, int32_t* out_n,
                       int32_t* out_len, row_diag* d) {
  const int G = c->G, V = c->V;
  const int g = c->gamma[b];
  int32_t* tok = out_tokens + (size_t)b * (G + 1);
  const int32_t* x = c->tokens + (size_t)b * G;
  const float* u = c->uniforms ? c->uniforms + (size_t)b * (G + 1) : NULL;
  const int kv = c->kv_len ? c->kv_len[b] : 0;

  if (d->draw_pos) *d->draw_pos = -1;
  if (d->zero_resid) *d->zero_resid = 0;
  if (g < 0 || g > G) {
    write_sentinel(c, b, out_tokens, out_n, out_len);
    return;
  }

  if (c->mode == OR_GREEDY) {
    int n = g, emit = -1;
    for (int i = 0; i <= g; ++i) {
      int gi = argmax_row(c, row_off(c, b, G + 1, i));
      if (i == g) {
        emit = gi;
        break;
      }
      if (x[i] < 0 || x[i] >= V) {
        write_sentinel(c, b, out_tokens, out_n, out_len);
        return;
      }
      if (x[i] != gi) {
        n = i;
        emit = gi;
        break;
      }
    }
    for (int i = 0; i < n; ++i) tok[i] = x[i];
    tok[n] = emit;
    for (int i = n + 1; i <= G; ++i) tok[i] = -1;
    out_n[b] = n;
    out_len[b] = kv + n;
    return;
  }

  /* Sampling (and point-mass drafts).  Diagnostics first: (max, exp-sum) of
   * every row t_0..t_g, d_0..d_{g-1}; they play no part in the decisions. */
  double* P = (double*)malloc(sizeof(double) * (size_t)(g + 1) * V);
  double* Q = (double*)malloc(sizeof(double) * (size_t)(g > 0 ? g : 1) * V);
  double* w = (double*)malloc(sizeof(double) * (size_t)V);
  int* live_p = (int*)malloc(sizeof(int) * (size_t)(g + 1));
  int* live_q = (int*)malloc(sizeof(int) * (size_t)(g > 0 ? g : 1));
  double fmargin = INFINITY;  /* smallest top-p margin over the rows */
  for (int i = 0; i <= g; ++i) {
    double m, s, mg;
    live_p[i] = softmax_row(c, c->target, row_off(c, b, G + 1, i), P + (size_t)i * V, &m, &s, &mg);
    if (d->m) d->m[i] = m;
    if (d->s) d->s[i] = s;
    fmargin = fmin(fmargin, mg);
  }
  for (int i = 0; i < g; ++i) {
    if (c->mode == OR_POINT) {
      /* q_i = indicator of x_i (an out-of-range x_i is caught by the walk) */
      double* q = Q + (size_t)i * V;
      for (int j = 0; j < V; ++j) q[j] = (j == x[i]) ? 1.0 : 0.0;
      live_q[i] = 1;
      continue;
    }
    double m, s, mg;
    oracle_ctx cq = *c;
    if (c->fault == OR_FAULT_FILTER_P_ONLY) cq.top_k = 0, cq.top_p = 1.0;
    live_q[i] = softmax_row(&cq, c->draft, row_off(c, b, G, i), Q + (size_t)i * V, &m, &s, &mg);
    if (d->m) d->m[G + 1 + i] = m;
    if (d->s) d->s[G + 1 + i] = s;
    fmargin = fmin(fmargin, mg);
  }
  if (d->fmargin) *d->fmargin = fmargin;

  /* Walk left to right.  A row the walk uses (p_i, q_i at a tested
   * position, p_g for the bonus) with no finite logit, or a tested token out
   * of range, is a data error; rows after the stop are never used. */
  int n = g;
  for (int i = 0; i < g; ++i) {
    const double* p = P + (size_t)i * V;
    const double* q = Q + (size_t)i * V;
    int xi = x[i];
    if (!live_p[i] || !live_q[i] || xi < 0 || xi >= V) {
      write_sentinel(c, b, out_tokens, out_n, out_len);
      free(P), free(Q), free(w), free(live_p), free(live_q);
      return;
    }
    if (d->px) d->px[i] = p[xi];
    if (d->qx) d->qx[i] = q[xi];
    int accept;
    if (c->fault == OR_FAULT_GREEDY_RULE) {
      int am = 0;
      for (int j = 1; j < V; ++j)
        if (p[j] > p[am]) am = j;
      accept = (xi == am);
    } else {
      accept = ((double)u[i] * q[xi] < p[xi]);
    }
    if (!accept) {
      n = i;
      break;
    }
  }
  if (n == g && !live_p[g]) {
    write_sentinel(c, b, out_tokens, out_n, out_len);
    free(P), free(Q), free(w), free(live_p), free(live_q);
    return;
  }

  const double* pn = P + (size_t)n * V;
  double ustar = (double)u[n < g ? n + 1 : g];
  if (n < g) {
    const double* qn = Q + (size_t)n * V;
    for (int j = 0; j < V; ++j) {
      double r = pn[j] - qn[j];
      if (c->fault == OR_FAULT_NO_CLAMP)
        w[j] = r;
      else if (c->fault == OR_FAULT_RESAMPLE_P)
        w[j] = pn[j];
      else
        w[j] = r > 0.0 ? r : 0.0;
    }
    double z = 0.0;
    for (int j = 0; j < V; ++j) z += w[j];
    if (z == 0.0) {
      if (d->zero_resid) *d->zero_resid = 1;
      memcpy(w, pn, sizeof(double) * (size_t)V);
    }
  } else {
    memcpy(w, pn, sizeof(double) * (size_t)V);
  }
  int j = draw_index(c, w, ustar, d->z, d->cdf, d->flo, d->fhi);
  if (d->draw_pos) *d->draw_pos = n;

  for (int i = 0; i < n; ++i) tok[i] = x[i];
  tok[n] = j;
  for (int i = n + 1; i <= G; ++i) tok[i] = -1;
  out_n[b] = n;
  out_len[b] = kv + n;
  free(P), free(Q), free(w), free(live_p), free(live_q);
}

/* Returns 0 on success, a negative value for arguments the oracle refuses.
 * Diagnostic outputs may be NULL: px/qx are [B, G] (NaN where a position
 * was not tested), z/draw_pos/zero_resid are [B], m/s are [B, 2G+1]. */
int oracle_verify(const void* target, const void* draft, int dtype, const int32_t* tokens,
                  const float* uniforms, const int32_t* gamma, const int32_t* kv_len, int B,
                  int G, int V, double T, int mode, int fault, int threads,
                  int32_t* out_tokens, int32_t* out_n, int32_t* out_len, double* out_px,
                  double* out_qx, double* out_z, double* out_m, double* out_s,
                  int32_t* out_draw_pos, int32_t* out_zero_resid, int top_k, double top_p,
                  double* out_fmargin, double* out_flo, double* out_fhi) {
  if (!target || !tokens || !gamma || !out_tokens || !out_n || !out_len) return -1;
  if (B < 0 || G < 0 || V <= 0) return -2;
  if (dtype != OR_F32 && dtype != OR_BF16) return -3;
  if (mode != OR_SAMPLE && mode != OR_GREEDY && mode != OR_POINT) return -3;
  if (mode == OR_SAMPLE && !draft) return -3;
  if (mode != OR_GREEDY && (!uniforms || !(T > 0.0) || !isfinite(T))) return -3;
  if (top_k < 0 || !(top_p > 0.0 && top_p <= 1.0)) return -3;
  /* greedy: filtering keeps the largest logit, so it changes nothing */
  if (mode == OR_GREEDY) top_k = 0, top_p = 1.0;
  oracle_ctx c = {target, draft, dtype, tokens, uniforms, gamma, kv_len, B, G, V, T, mode, fault,
                  top_k, top_p};
  const size_t nr = (size_t)(2 * G + 1);
  if (out_px)
    for (size_t k = 0; k < (size_t)B * G; ++k) out_px[k] = NAN;
  if (out_qx)
    for (size_t k = 0; k < (size_t)B * G; ++k) out_qx[k] = NAN;
  if (out_z)
    for (int b = 0; b < B; ++b) out_z[b] = NAN;
  if (out_m)
    for (size_t k = 0; k < (size_t)B * nr; ++k) out_m[k] = NAN;
  if (out_s)
    for (size_t k = 0; k < (size_t)B * nr; ++k) out_s[k] = NAN;
  if (out_fmargin)
    for (int b = 0; b < B; ++b) out_fmargin[b] = INFINITY;
  for (int b = 0; b < B; ++b) {
    if (out_flo) out_flo[b] = NAN;
    if (out_fhi) out_fhi[b] = NAN;
  }
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int b = 0; b < B; ++b) {
    row_diag d = {out_px ? out_px + (size_t)b * G : NULL,
                  out_qx ? out_qx + (size_t)b * G : NULL,
                  out_z ? out_z + b : NULL,
                  out_m ? out_m + (size_t)b * nr : NULL,
                  out_s ? out_s + (size_t)b * nr : NULL,
                  out_draw_pos ? out_draw_pos + b : NULL,
                  out_zero_resid ? out_zero_resid + b : NULL,
                  NULL,
                  out_fmargin ? out_fmargin + b : NULL,
                  out_flo ? out_flo + b : NULL,
                  out_fhi ? out_fhi + b : NULL};
    verify_row(&c, b, out_tokens, out_n, out_len, &d);
  }
  (void)threads;
  return 0;
}

/* Re-runs row b alone and writes the normalised CDF (C_j / Z) of the
 * distribution the oracle drew its last token from into cdf[0..V).
 * Returns the drawn position, or -1 when the row drew nothing (greedy or a
 * data error). */
int oracle_draw_cdf(const void* target, const void* draft, int dtype, const int32_t* tokens,
                    const float* uniforms, const int32_t* gamma, const int32_t* kv_len, int B,
                    int G, int V, double T, int mode, int b, double* cdf, int top_k,
                    double top_p) {
  if (!target || !tokens || !uniforms || !gamma || !cdf) return -1;
  if (mode != OR_SAMPLE && mode != OR_POINT) return -1;
  if (mode == OR_SAMPLE && !draft) return -1;
  if (b < 0 || b >= B) return -1;
  if (top_k < 0 || !(top_p > 0.0 && top_p <= 1.0)) return -1;
  oracle_ctx c = {target, draft, dtype, tokens, uniforms, gamma, kv_len, B, G, V, T, mode,
                  OR_FAULT_NONE, top_k, top_p};
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * (G + 1));
  int32_t* nn = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  int32_t* ln = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  int32_t pos = -1;
  row_diag d = {NULL, NULL, NULL, NULL, NULL, &pos, NULL, cdf, NULL, NULL, NULL};
  verify_row(&c, b, tok, nn, ln, &d);
  free(tok), free(nn), free(ln);
  return pos;
}

/* The inverse-CDF draw alone, over caller-given non-negative weights
 * w[0..V) with uniform u (test hook: it pins the draw's tie-break and its
 * fallback rule directly).  Writes Z = sum w; returns the drawn index. */
int oracle_draw_index(const double* w, int V, double u, double* z_out) {
  if (!w || V <= 0) return -1;
  oracle_ctx c = {NULL, NULL, OR_F32, NULL, NULL, NULL, NULL, 1, 0, V, 1.0, OR_SAMPLE,
                  OR_FAULT_NONE, 0, 1.0};
  return draw_index(&c, w, u, z_out, NULL, NULL, NULL);
}

/* The filtered distribution of one stored logit row (what a drafter that
 * applies the same top-k / top-p would sample from): prob[0..V) and the
 * threshold tau (entries with l >= tau kept).  Returns 0, or -1 for refused
 * arguments or a row with no finite logit. */
int oracle_filter_row(const void* logits, int dtype, int V, double T, int top_k, double top_p,
                      double* prob, double* tau_out, double* margin_out) {
  if (!logits || !prob || V <= 0 || !(T > 0.0) || !isfinite(T)) return -1;
  if (dtype != OR_F32 && dtype != OR_BF16) return -1;
  if (top_k < 0 || !(top_p > 0.0 && top_p <= 1.0)) return -1;
  oracle_ctx c = {logits, NULL, dtype, NULL, NULL, NULL, NULL, 1, 0, V, T, OR_SAMPLE,
                  OR_FAULT_NONE, top_k, top_p};
  double m, s;
  if (!softmax_row(&c, logits, 0, prob, &m, &s, margin_out)) return -1;
  if (tau_out) *tau_out = filter_threshold(&c, logits, 0, m, NULL);
  return 0;
}

/* ---------------------------------------------------------------- drafting
 * Prompt-lookup (n-gram) drafting ("Speculative decoding", mhtirogla.ai,
 * "Implementation notes"; tusharamrit, "Self-speculation"): the drafter
 * finds where the context's latest n tokens occurred before and proposes
 * the tokens that came after that occurrence.
 * Reading: for n = n_max down to n_min, the suffix is the last n tokens of
 * the context c[0..L); its most recent earlier occurrence is the largest j
 * with j + n <= L - 1 (so that a token follows it) and c[j..j+n) equal to
 * the suffix; the first n with an occurrence wins (the longest match), and
 * the draft is c[j+n .. min(j+n+gamma, L)).  No occurrence for any n: no
 * draft.
 * context: int32 [B, stride]; ctx_len[b] in [0, stride] tokens of row b.
 * out_draft: int32 [B, gamma] (-1 after the draft); out_len: [B] draft
 * lengths; out_n, out_pos (optional): the n that matched and the draft's
 * start j + n (-1 when none).  A row whose length lies outside [0, stride]
 * gets no draft and out_n = -2.  Returns 0, or -1 for refused arguments. */
int oracle_ngram_draft(const int32_t* context, const int32_t* ctx_len, int B, int stride,
                       int n_min, int n_max, int gamma, int32_t* out_draft, int32_t* out_len,
                       int32_t* out_n, int32_t* out_pos) {
  if (!context || !ctx_len || !out_draft || !out_len) return -1;
  if (B < 0 || stride < 0 || n_min < 1 || n_max < n_min || gamma < 0) return -1;
  for (int b = 0; b < B; ++b) {
    const int32_t* c = context + (size_t)b * stride;
    const int L = ctx_len[b];
    int32_t* d = out_draft + (size_t)b * gamma;
    for (int i = 0; i < gamma; ++i) d[i] = -1;
    out_len[b] = 0;
    if (out_n) out_n[b] = -1;
    if (out_pos) out_pos[b] = -1;
    if (L < 0 || L > stride) {
      if (out_n) out_n[b] = -2;
      continue;
    }
    for (int n = n_max; n >= n_min; --n) {
      if (L < n + 1) continue;
      int found = -1;
      for (int j = L - n - 1; j >= 0 && found < 0; --j) {
        int same = 1;
        for (int i = 0; i < n && same; ++i) same = c[j + i] == c[L - n + i];
        if (same) found = j;
      }
      if (found >= 0) {
        const int start = found + n;
        int k = 0;
        for (; k < gamma && start + k < L; ++k) d[k] = c[start + k];
        out_len[b] = k;
        if (out_n) out_n[b] = n;
        if (out_pos) out_pos[b] = start;
        break;
      }
    }
  }
  return 0;
}

/* --------------------------------------------------------------- adaptive gamma
 * Each request's next draft length from the acceptance it has seen so far,
 * and no speculation once the batch is large ("Speculative decoding",
 * mhtirogla.ai, "Efficiency" and "Implementation notes": tokens per pass,
 * the wall-clock speedup E / (1 + gamma c), a per-request length that
 * follows the observed acceptance, and turning drafting off when the batch
 * is compute-bound; blog.lo0.es "When speculative does NOT help": the
 * large-batch crossover; tusharamrit "Speculative decoding": the speedup
 * table; dantp-ai "How much speedup, really?": the best lookahead depends
 * on the acceptance rate).
 * Reading:
 *   state per row: discounted accepted count A and tested count T.
 *   observation of a round with g = gamma_used[b] >= 1 and n = n_acc[b] >= 0:
 *     the walk tested min(n + 1, g) drafts and accepted n of them;
 *     A <- d A + n,  T <- d T + min(n + 1, g).
 *   a row without an observation (g = 0, n < 0, or no previous round) only
 *   ages its evidence: A <- d A, T <- d T.  Inactive rows are left alone.
 *   running acceptance  alpha = (A + w0 alpha0) / (T + w0)  (alpha0 when
 *   T + w0 = 0).
 *   E(gamma) = sum_{i=0..gamma} alpha^i   (tokens per pass, page formula)
 *   gamma_b = the smallest gamma in [0, min(gamma_max, limit_b)] maximising
 *     E(gamma) / (1 + gamma c), compared without division:
 *     E(g1) (1 + g2 c) > E(g2) (1 + g1 c).
 *   If the number of active rows is >= batch_off (batch_off >= 1), every
 *   row gets gamma 0 (its state is still updated).
 * Inactive rows (active[b] == 0) get gamma 0 and keep their state.
 * state: double [B][2] {A, T}, updated in place.  out_alpha (optional): the
 * alpha each active row's choice used.  Returns 0, or -1 for refused
 * arguments. */
int oracle_gamma_control(const int32_t* n_acc, const int32_t* gamma_used, const int32_t* active,
                         const int32_t* gamma_limit, double* state, int B, int gamma_max,
                         double decay, double prior_alpha, double prior_weight, double draft_cost,
                         int batch_off, int32_t* out_gamma, double* out_alpha) {
  if (!state || !out_gamma || B < 0 || gamma_max < 0) return -1;
  if ((n_acc == NULL) != (gamma_used == NULL)) return -1;
  if (!(decay >= 0.0 && decay <= 1.0) || !(prior_alpha >= 0.0 && prior_alpha <= 1.0)) return -1;
  if (!(prior_weight >= 0.0) || !(draft_cost >= 0.0) || isinf(prior_weight) || isinf(draft_cost))
    return -1;
  if (batch_off < 0) return -1;
  int n_active = 0;
  for (int b = 0; b < B; ++b) n_active += !active || active[b] != 0;
  const int off = batch_off >= 1 && n_active >= batch_off;
  for (int b = 0; b < B; ++b) {
    out_gamma[b] = 0;
    if (out_alpha) out_alpha[b] = 0.0;
    if (active && active[b] == 0) continue;
    double A = state[2 * b], T = state[2 * b + 1];
    const int g = gamma_used ? gamma_used[b] : 0;
    const int n = n_acc ? n_acc[b] : -1;
    if (g >= 1 && n >= 0 && n <= g) {
      const int tested = n + 1 < g ? n + 1 : g;
      A = decay * A + (double)n;
      T = decay * T + (double)tested;
    } else {
      A = decay * A;
      T = decay * T;
    }
    state[2 * b] = A;
    state[2 * b + 1] = T;
    const double den = T + prior_weight;
    const double alpha = den > 0.0 ? (A + prior_weight * prior_alpha) / den : prior_alpha;
    if (out_alpha) out_alpha[b] = alpha;
    if (off) continue;
    int cap = gamma_max;
    if (gamma_limit && gamma_limit[b] < cap) cap = gamma_limit[b] < 0 ? 0 : gamma_limit[b];
    /* E(0) = 1; E(k) = E(k-1) + alpha^k */
    double best_e = 1.0, pw = 1.0, e = 1.0;
    int best = 0;
    for (int k = 1; k <= cap; ++k) {
      pw = pw * alpha;
      e = e + pw;
      /* e / (1 + k c) > best_e / (1 + best c) */
      if (e * (1.0 + (double)best * draft_cost) > best_e * (1.0 + (double)k * draft_cost)) {
        best = k;
        best_e = e;
      }
    }
    out_gamma[b] = best;
  }
  return 0;
}
