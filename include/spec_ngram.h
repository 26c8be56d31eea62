/*
 * spec_ngram.h -- C ABI of the MI355X (gfx950) prompt-lookup (n-gram)
 * drafter, the model-free step that feeds the verify's POINT mode.
 *
 * The operation (sources: "Speculative decoding", mhtirogla.ai,
 * "Implementation notes" and "Variants": the drafter copies what followed
 * the last earlier match of the current n-gram; "Speculative decoding",
 * inference.tusharamrit.in, "Self-speculation": search the context for its
 * current suffix and propose what followed it the last time it appeared):
 *
 *   For every batch row b with context c = context[b, 0 .. L), L = ctx_len[b]:
 *     for n = n_max down to n_min, the suffix is c[L-n .. L); its most recent
 *     earlier occurrence is the largest j with j + n <= L - 1 (a token must
 *     follow it; it may overlap the suffix) and c[j .. j+n) == c[L-n .. L).
 *     The first n that has one wins (the longest match) and the draft is
 *     c[j+n .. min(j+n+gamma, L)).  No occurrence for any n: no draft.
 *
 * Outputs feed spec_verify in SPEC_MODE_POINT unchanged: out_draft as its
 * draft_tokens [B, gamma_max = gamma] and out_len as its gamma_per_row.  A
 * row with an empty draft then samples its one token from p_0.
 *
 * Calls are asynchronous on `stream` like spec_verify (argument errors are
 * returned before anything is launched, and then no output is written).
 * The status codes are those of spec_verify.h.
 */
#ifndef SPEC_NGRAM_H
#define SPEC_NGRAM_H

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_NGRAM_MAX_N 64          /* largest n_max                        */
#define SPEC_NGRAM_MAX_GAMMA 256     /* largest draft length                 */
#define SPEC_NGRAM_MAX_STRIDE (1 << 25) /* largest context row, in tokens    */

/* Bytes of device workspace spec_ngram_draft needs for B rows (0 for B < 1):
 * one match key and one arrival counter per row, 256 bytes apart.  Zero-fill
 * it once before its first use (spec_verify_workspace_reset, or any zero
 * fill); every call that completes leaves it zero again, so one workspace
 * serves any sequence of stream-ordered calls with at most that many rows.
 * Two calls that share a workspace must not overlap (same stream). */
size_t spec_ngram_workspace_bytes(int B);

/* Prompt-lookup drafting.  All arrays are device memory, row-major.
 *   context    int32 [B, stride] token ids (any values); may be NULL when
 *              stride == 0.  Read only.
 *   ctx_len    int32 [B]: L of each row.  A row whose L lies outside
 *              [0, stride] gets no draft and out_n = -2 (the others are
 *              unaffected).
 *   B >= 0 (0: nothing is launched), 0 <= stride <= SPEC_NGRAM_MAX_STRIDE,
 *   1 <= n_min <= n_max <= SPEC_NGRAM_MAX_N, 0 <= gamma <= SPEC_NGRAM_MAX_GAMMA.
 *   out_draft  int32 [B, gamma]: the draft, then -1 (may be NULL if gamma == 0)
 *   out_len    int32 [B]: draft length, 0 .. gamma
 *   out_n      int32 [B] or NULL: the n that matched, -1 if none, -2 for a
 *              row with an invalid length
 *   out_pos    int32 [B] or NULL: where the copied continuation starts in
 *              the row (j + n), -1 if none
 *   workspace  at least spec_ngram_workspace_bytes(B) bytes, 256-byte
 *              aligned, zero on entry (see above)
 * Every int32 array must be 4-byte aligned (SPEC_ERR_ALIGN).  Returns
 * SPEC_ERR_SHAPE for B or stride out of range, SPEC_ERR_ARG for n_min,
 * n_max or gamma out of range, SPEC_ERR_NULL for a missing required
 * pointer, SPEC_ERR_WORKSPACE for a missing or short workspace. */
int spec_ngram_draft(const int32_t* context, const int32_t* ctx_len, int B, int stride,
                     int n_min, int n_max, int gamma, int32_t* out_draft, int32_t* out_len,
                     int32_t* out_n, int32_t* out_pos, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Drafting and the draft-length rule of spec_adapt.h in one call: the
 * drafter as spec_ngram_draft, then for every row the rule
 * (spec_gamma_control with gamma_max = gamma and gamma_limit = the row's
 * draft length), run by the last step of the drafting launch.  out_gamma
 * (int32 [B]) is the verify's gamma_per_row for this round; out_len keeps
 * the drafted length.  The rule's arguments (n_accepted, gamma_used,
 * active, state, decay, prior_alpha, prior_weight, draft_cost, batch_off,
 * out_alpha) mean what they mean for spec_gamma_control, with the same
 * errors; gamma must also be <= SPEC_GAMMA_MAX_LIMIT.  Results are
 * bit-identical to spec_ngram_draft followed by spec_gamma_control.
 * Batches above 1,024 rows run the two as separate launches on `stream`. */
int spec_ngram_draft_adaptive(const int32_t* context, const int32_t* ctx_len, int B, int stride,
                              int n_min, int n_max, int gamma, const int32_t* n_accepted,
                              const int32_t* gamma_used, const int32_t* active, double* state,
                              double decay, double prior_alpha, double prior_weight,
                              double draft_cost, int batch_off, int32_t* out_draft,
                              int32_t* out_len, int32_t* out_n, int32_t* out_pos,
                              int32_t* out_gamma, double* out_alpha, void* workspace,
                              size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_NGRAM_H */
