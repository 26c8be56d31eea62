/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) batched verify step of
 * speculative decoding.
 *
 * The operation (sources: "Speculative decoding", mhtirogla.ai, sections
 * "How it works" steps 2-5 and "Code"; "Speculative decoding: the secretary
 * who types ahead of the boss", blog.lo0.es, "The bare mechanism" step 3;
 * "Speculative decoding", inference.tusharamrit.in, the loop and the
 * modified rejection-sampling rule; "Speculative Decoding", tokentrails.org,
 * steps 2 and 4):
 *
 *   For every batch row b with draft length g = gamma_per_row[b]:
 *     p_i = softmax(target_logits[b, i, :] / T), i = 0..g   (row g: bonus)
 *     q_i = softmax(draft_logits[b, i, :] / T),  i = 0..g-1
 *     walking i = 0..g-1, accept x_i = draft_tokens[b, i] while
 *       u_i * q_i(x_i) < p_i(x_i)        (u_i = uniforms[b, i])
 *     at the first rejection n: emit x_0..x_{n-1}, then one token drawn by
 *       inverse CDF from norm(max(0, p_n - q_n)) with uniform u_{n+1};
 *     if all g are accepted: emit x_0..x_{g-1}, then one token drawn from
 *       p_g with uniform u_g.
 *     The inverse CDF returns the smallest j with u * Z < sum_{k<=j} w_k
 *     (Z = sum of the weights); if rounding leaves no such j, the last index
 *     with positive weight.
 *   GREEDY mode ignores T, q and u: g_i = lowest index of the largest
 *   target logit of row i; accept while x_i == g_i; emit x_0..x_{n-1}, g_n.
 *   POINT mode is SAMPLE for a drafter that proposes tokens outright, with
 *   no draft distribution (a greedy draft, an n-gram / prompt-lookup match:
 *   mhtirogla.ai, "Variants" and "Implementation notes"; tusharamrit,
 *   "Self-speculation"): q_i is the indicator of x_i, so x_i is accepted
 *   while u_i < p_i(x_i), and after a rejection at n the draw is from p_n
 *   with x_n removed (Z = 1 - p_n(x_n)).  Draft logits are not read.
 *   new_len[b] = kv_len_in[b] + n (the KV caches keep the accepted drafts;
 *   the emitted correction or bonus token has no cache entry yet).
 *
 * All device work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without synchronising: outputs are valid
 * once the stream has completed the call.  Argument errors are reported by
 * the return value before anything is launched, and then no output is
 * written.  The library allocates no memory and keeps no state other than
 * the caller's workspace (plus a process-wide tuning override, see
 * spec_verify_tune, and each device's compute-unit count, asked once).  The
 * CU count picks between launch variants that differ in speed only (wave
 * priorities when the whole grid fits on the device at once); results are
 * the same.  Calls on distinct workspaces may run concurrently; two calls
 * that share a workspace must be ordered (same stream).  A call's
 * workgroups wait only on workgroups of their own batch row, whose ids are
 * consecutive; one call alone always makes progress.  Concurrent calls
 * whose grids together exceed the device's workgroup slots (four per CU)
 * could, in principle, each hold slots that the other's unstarted row
 * members need: every wait is bounded (about 0.2 s), and a row whose wait
 * runs out gets the sentinel and sets diagnostic bit 0 -- never a wrong
 * token.  Overlapping calls whose grids fit the device together cannot
 * meet this.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum spec_mode { SPEC_MODE_SAMPLE = 0, SPEC_MODE_GREEDY = 1, SPEC_MODE_POINT = 2 };
enum spec_dtype { SPEC_DTYPE_F32 = 0, SPEC_DTYPE_BF16 = 1 };

enum spec_status {
  SPEC_OK = 0,
  SPEC_ERR_NULL = -1,      /* a required pointer is NULL                              */
  SPEC_ERR_SHAPE = -2,     /* B < 1, V < 1, V > 2^20, gamma_max outside [0, 63], or
                              more than 2^31 - 1 workgroups                          */
  SPEC_ERR_ARG = -3,       /* unknown mode or dtype; T not finite and > 0 in SAMPLE
                              or POINT mode; a tuning value spec_verify_tune refuses */
  SPEC_ERR_WORKSPACE = -4, /* workspace NULL or smaller than spec_verify_workspace_bytes */
  SPEC_ERR_ALIGN = -5,     /* logits not aligned to their element size, or an int32/float
                              array not 4-byte aligned                                 */
  SPEC_ERR_HIP = -100      /* a HIP runtime error e is returned as SPEC_ERR_HIP - e     */
};

#define SPEC_GAMMA_MAX_LIMIT 63

/* Bytes of device workspace a call with these sizes needs (host only, pure
 * function of its arguments and of the tuning override).  Returns 0 for
 * sizes spec_verify would reject.
 *
 * The workspace holds one counter per batch row, the softmax statistics of
 * every vocabulary slice, the draw sums of every slice and (SAMPLE, POINT)
 * one filter threshold per vocabulary row.  It must be zero-filled once
 * before its first use (spec_verify_workspace_reset, or any zero fill).
 * Every call that completes clears everything it wrote, leaving the
 * workspace all zero again (the diagnostic word and the thresholds aside:
 * a filtered call writes all the thresholds it reads), so one workspace
 * serves any sequence of stream-ordered calls, of any shapes, whose
 * spec_verify_workspace_bytes does not exceed its size.  A call that gave up
 * waiting (diagnostic bit 0) may leave it dirty: zero-fill it again. */
size_t spec_verify_workspace_bytes(int B, int gamma_max, int V, int dtype, int mode);

/* Zero-fills `bytes` of a workspace with a small fill kernel on `stream`
 * (no memset node, so it may be captured in a HIP graph). */
int spec_verify_workspace_reset(void* workspace, size_t bytes, void* stream);

/* The verify step.  Device pointers unless stated; all arrays dense,
 * row-major, innermost index last:
 *   target_logits  [B, gamma_max+1, V] of dtype (fp32, or bf16 bit patterns)
 *   draft_logits   [B, gamma_max, V]   of dtype; read in SAMPLE mode only
 *                  (may be NULL otherwise)
 *   draft_tokens   int32 [B, gamma_max]; x_i for i < gamma_per_row[b]
 *   uniforms       fp32 [B, gamma_max+1] in [0, 1); may be NULL in GREEDY
 *   gamma_per_row  int32 [B]; each in [0, gamma_max]
 *   kv_len_in      int32 [B], or NULL for 0
 *   temperature    T > 0 (SAMPLE, POINT); ignored in GREEDY
 *   out_tokens     int32 [B, gamma_max+1]: n+1 emitted tokens, then -1
 *   out_n_accepted int32 [B]: n
 *   out_new_len    int32 [B]: kv_len_in + n
 * Any 2-byte (bf16) or 4-byte (fp32) aligned logits base works; rows need
 * not be 16-byte aligned.  Logits must be finite or -inf.
 * Per-row data errors (gamma outside [0, gamma_max]; a tested draft token
 * outside [0, V); in SAMPLE and POINT mode, a row the walk uses -- p_i and
 * (SAMPLE) q_i of a tested position, p_g for the bonus -- whose logits are
 * all -inf) give
 * n_accepted = -1, tokens all -1 and new_len = kv_len_in for that row only.
 * Rows after the first rejection are never used. */
int spec_verify(const void* target_logits, const void* draft_logits,
                const int32_t* draft_tokens, const float* uniforms,
                const int32_t* gamma_per_row, const int32_t* kv_len_in, int B, int gamma_max,
                int V, int dtype, float temperature, int mode, int32_t* out_tokens,
                int32_t* out_n_accepted, int32_t* out_new_len, void* workspace,
                size_t workspace_bytes, void* stream);

/* Largest workspace spec_verify_noalloc can use (8 MiB; spec_verify_workspace_bytes
 * of the call must not exceed it).  At 1024 workgroups per call this covers,
 * e.g., B = 256, gamma_max = 8, V = 151936 (about 0.9 MiB). */
#define SPEC_NOALLOC_WORKSPACE_BYTES (8u << 20)

/* spec_verify without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments (less the workspace), semantics and
 * errors as spec_verify.  The workspace is a device array inside the library,
 * SPEC_NOALLOC_WORKSPACE_BYTES per device, held until the process ends; the
 * call allocates and frees nothing.  Each call first clears the part it uses
 * (a fill kernel on `stream`), then runs spec_verify on it.  Every call on a
 * device shares that device's array: calls that may overlap on one device
 * (different streams, different host threads) race and give undefined
 * results -- order them on one stream.  Returns SPEC_ERR_WORKSPACE when the
 * call needs more than SPEC_NOALLOC_WORKSPACE_BYTES (nothing is launched),
 * SPEC_ERR_HIP - e if the array's device address cannot be obtained. */
int spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms,
                        const int32_t* gamma_per_row, const int32_t* kv_len_in, int B,
                        int gamma_max, int V, int dtype, float temperature, int mode,
                        int32_t* out_tokens, int32_t* out_n_accepted, int32_t* out_new_len,
                        void* stream);

/* spec_verify plus the intermediate values, for parity checks (same
 * arguments and semantics, slower).  Each probe pointer may be NULL:
 *   out_px, out_qx  fp32 [B, gamma_max]: p_i(x_i), q_i(x_i) for every
 *                   i < gamma_per_row[b] with a valid token (untouched
 *                   otherwise; SAMPLE and POINT only, q_i(x_i) = 1 in POINT)
 *   out_z           fp32 [B]: normaliser Z of the drawn distribution
 *   out_m, out_s    fp32 [B, 2*gamma_max+1]: per vocabulary row (target
 *                   rows 0..gamma_max, then draft rows 0..gamma_max-1) the
 *                   largest raw logit and S = sum_j exp((l_j - max) / T)
 *                   (GREEDY: out_m only, out_s holds the argmax as float;
 *                   GREEDY and POINT leave the draft slots untouched)
 *   Without SPEC_TUNE_ONE_PASS the rows are read in groups of positions
 *   (0; 1-2; then up to four at a time -- on launches of at most 256
 *   workgroups the first group may hold 0-1) up to the group holding the
 *   walk's stop n, and only what was read is reported: out_px / out_qx for the
 *   positions of the groups read (which may run past n), out_m / out_s for
 *   their rows t_i (and d_i in SAMPLE; t_g when it was read); the other
 *   entries are untouched.
 *   out_f_lo,       fp32 [B]: the CDF bracket of the drawn token j, i.e. the
 *   out_f_hi        normalised cumulative weight of the tokens before j and
 *                   through j (u lies in [f_lo, f_hi) unless the fallback
 *                   rule chose j); both NULL or both given; SAMPLE and POINT
 *                   only, untouched for rows with a data error.
 * The CDF values are formed in double precision and rounded to fp32 here. */
int spec_verify_probe(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms,
                      const int32_t* gamma_per_row, const int32_t* kv_len_in, int B,
                      int gamma_max, int V, int dtype, float temperature, int mode,
                      int32_t* out_tokens, int32_t* out_n_accepted, int32_t* out_new_len,
                      void* workspace, size_t workspace_bytes, void* stream, float* out_px,
                      float* out_qx, float* out_z, float* out_m, float* out_s, float* out_f_lo,
                      float* out_f_hi);

/* spec_verify with the same top-k / top-p filtering applied to p and q
 * before the walk (sources: mhtirogla.ai "Implementation notes";
 * tusharamrit, the caveat after the proof: the draft and the target must
 * process their logits identically).  For each vocabulary row the verify
 * uses, with logits l and temperature T:
 *   top-k (top_k > 0): keep every l_j at or above the k-th largest value of
 *     the row (ties at that value all kept);
 *   top-p (top_p < 1): then keep, among those, the smallest set of largest
 *     values whose mass under softmax(l / T) reaches top_p of the mass kept
 *     by top-k, all copies of a value together;
 *   the kept entries are renormalised and the others have probability 0;
 *   the walk, residual and draw are then those of spec_verify on the
 *   filtered rows (x_i should come from the filtered q; a token the filter
 *   cuts from q_i has q_i(x_i) = 0 and is accepted iff p_i(x_i) > 0).
 * top_k = 0 and top_p = 1 turn a filter off; with both off this is
 * spec_verify.  GREEDY ignores both (the filters keep the largest logit).
 * POINT filters p only (there is no q).  Masses are fp32 exponentials
 * 2^(l k2 - R) (k2 = log2(e)/T rounded to fp32), summed exactly in fixed point
 * (units of 2^-42 of the row's largest weight).  Each mass is within about
 * 1e-7 relative of exp((l - max)/T) near the top of the row and within
 * |l - max|/T * 1e-7 further down (the rounding of the exponent and of k2), so
 * a cumulative mass is within about 1e-6 of the row's kept mass from the
 * exact one: a row whose top-p cut lies that close to the boundary may cut
 * one value apart from an exact computation.  Two launches on `stream`: the
 * thresholds (into
 * the workspace), then the verify.  Errors: those of spec_verify, and
 * SPEC_ERR_ARG for top_k < 0 or top_p outside (0, 1]. */
int spec_verify_filtered(const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const float* uniforms,
                         const int32_t* gamma_per_row, const int32_t* kv_len_in, int B,
                         int gamma_max, int V, int dtype, float temperature, int mode, int top_k,
                         float top_p, int32_t* out_tokens, int32_t* out_n_accepted,
                         int32_t* out_new_len, void* workspace, size_t workspace_bytes,
                         void* stream);

/* spec_verify_filtered plus the probes of spec_verify_probe (of the filtered
 * rows: out_s holds the filtered S). */
int spec_verify_filtered_probe(const void* target_logits, const void* draft_logits,
                               const int32_t* draft_tokens, const float* uniforms,
                               const int32_t* gamma_per_row, const int32_t* kv_len_in, int B,
                               int gamma_max, int V, int dtype, float temperature, int mode,
                               int top_k, float top_p, int32_t* out_tokens,
                               int32_t* out_n_accepted, int32_t* out_new_len, void* workspace,
                               size_t workspace_bytes, void* stream, float* out_px, float* out_qx,
                               float* out_z, float* out_m, float* out_s, float* out_f_lo,
                               float* out_f_hi);

/* The thresholds alone: out_thr fp32 [B, 2*gamma_max+1] (device; target rows
 * 0..gamma_max, then draft rows 0..gamma_max-1), the value tau of each
 * vocabulary row the walk may use such that the filtered row keeps exactly
 * the entries with l >= tau; -inf where nothing is cut, for rows beyond
 * gamma_per_row[b] (and draft rows in POINT mode), and for rows with no
 * finite logit.  mode: SAMPLE or POINT.  Asynchronous on `stream`; needs no
 * workspace. */
int spec_filter_thresholds(const void* target_logits, const void* draft_logits,
                           const int32_t* gamma_per_row, int B, int gamma_max, int V, int dtype,
                           float temperature, int mode, int top_k, float top_p, float* out_thr,
                           void* stream);

/* Launch plan of a call with these sizes (host only).  Each batch row is
 * served by `slices` workgroups; workgroup c owns elements [c * slice_len,
 * (c + 1) * slice_len) of every vocabulary row of the batch row.  Fills
 * out[0..7] with {workgroups, slices per vocabulary row, slice length
 * (elements), 16-byte vectors per thread and vocabulary row, vocabulary rows
 * per batch row at gamma_max, threads per workgroup, workspace bytes, target
 * workgroup count}.  Returns SPEC_OK or an argument error. */
int spec_verify_plan(int B, int gamma_max, int V, int dtype, int mode, int64_t* out);

/* Flags of spec_verify_tune. */
enum spec_tune_flags {
  /* Calls of every mode (filtered or not) stream every vocabulary row of a
   * batch row in one pass and decide all positions at once, instead of the
   * default: reading the rows position by position (t_i, and d_i in SAMPLE,
   * for i = 0, 1, ...) and stopping at the walk's first rejection (the rows
   * after it are never used), at the cost of one hand-off between a row's
   * workgroups per group of positions.  Results are the same either way. */
  SPEC_TUNE_ONE_PASS = 1
};

/* Process-wide override of the launch tuning (for benchmarking sweeps).
 * vectors: 16-byte vectors per thread and vocabulary row, which sets the
 * slice length (vectors * 4 KiB of logits): 1, 2 or 4, or 0 to choose it
 * from the sizes -- the largest slices that still
 * give at least target_workgroups workgroups.  target_workgroups: 0 keeps
 * the default (1024).  flags: 0 or SPEC_TUNE_ONE_PASS (any other bit is
 * SPEC_ERR_ARG).  Changes spec_verify_workspace_bytes; not thread-safe
 * against concurrent calls. */
int spec_verify_tune(int vectors, int target_workgroups, int flags);

/* Reads the workspace's diagnostic word (device -> host copy on `stream`,
 * synchronous): bit 0 set if a workgroup ever gave up waiting for the rest
 * of its batch row's workgroups (cannot happen in a correct launch), bit 1
 * set if a residual with zero mass fell back to p (POINT: to x_n, the only
 * token p_n then has). */
int spec_verify_diagnostics(const void* workspace, uint32_t* out_flags, void* stream);

const char* spec_verify_strerror(int status);
int spec_verify_version(void);

/* Streaming-read bandwidth probe: reads `bytes` (a multiple of 16) from
 * src, writes one float per workgroup into out (at least
 * spec_probe_read_blocks(bytes) floats).  Used to measure the box's
 * achievable HBM read rate next to the 8 TB/s specification. */
int spec_probe_read(const void* src, size_t bytes, float* out, void* stream);
int spec_probe_read_blocks(size_t bytes);

/* Plain copy of `bytes` (a multiple of 16) from src to dst: the reference
 * kernel of known traffic against which hardware byte counters are scaled. */
int spec_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
