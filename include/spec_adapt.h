/*
 * spec_adapt.h -- C ABI of the MI355X (gfx950) adaptive draft-length
 * controller: each request's next draft length from its running acceptance,
 * and speculation off at large batch.
 *
 * Sources: "Speculative decoding", mhtirogla.ai, "Efficiency" (tokens per
 * pass E = sum_{i<=gamma} alpha^i and wall-clock speedup E / (1 + gamma c))
 * and "Implementation notes" (a per-request length that follows the observed
 * acceptance; no drafting once the batch is compute-bound); "Speculative
 * decoding: the secretary who types ahead of the boss", blog.lo0.es, "When
 * speculative does NOT help" (the large-batch crossover); "Speculative
 * decoding", inference.tusharamrit.in (adapt gamma from recent acceptance);
 * "Speculative decoding", dantp-ai.github.io, "How much speedup, really?"
 * (an optimal lookahead for every acceptance rate).
 *
 * The rule, per batch row b (all arithmetic in fp64, in this order):
 *   observation of the previous round, when n_accepted and gamma_used are
 *   given and g = gamma_used[b] >= 1, 0 <= n = n_accepted[b] <= g:
 *     A <- decay * A + n,  T <- decay * T + min(n + 1, g)
 *   (the walk tested min(n + 1, g) drafts and accepted n); any other row
 *   only ages its evidence: A <- decay * A, T <- decay * T.
 *   alpha = (A + prior_weight * prior_alpha) / (T + prior_weight), or
 *   prior_alpha when T + prior_weight == 0.
 *   gamma_b = the smallest gamma in [0, min(gamma_max, gamma_limit[b])]
 *   maximising E(gamma) / (1 + gamma * draft_cost), E built as
 *   E(0) = 1, E(k) = E(k-1) + alpha^k (alpha^k by repeated products), and
 *   gamma k preferred over the best so far j when
 *   E(k) * (1 + j * draft_cost) > E(j) * (1 + k * draft_cost).
 *   If batch_off >= 1 and the number of active rows is >= batch_off, every
 *   row gets gamma 0 (states are still updated).
 *   Inactive rows (active[b] == 0) get gamma 0 and keep their state.
 *
 * A round of model-free speculation runs spec_ngram_draft (draft up to
 * gamma_max), then this call with gamma_limit = the draft lengths, then
 * spec_verify in SPEC_MODE_POINT with gamma_per_row = out_gamma; the next
 * round passes that verify's n_accepted and this out_gamma back in.  With a
 * draft model, out_gamma is how many tokens to draft (gamma_limit NULL).
 *
 * Asynchronous on `stream` like spec_verify; argument errors are returned
 * before anything is launched.  Status codes are those of spec_verify.h.
 */
#ifndef SPEC_ADAPT_H
#define SPEC_ADAPT_H

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Device arrays, row-major:
 *   n_accepted   int32 [B] or NULL: the previous round's accepted counts
 *                (spec_verify's out_n_accepted; -1 rows are not observed)
 *   gamma_used   int32 [B] or NULL: that round's draft lengths; NULL exactly
 *                when n_accepted is NULL (no previous round)
 *   active       int32 [B] or NULL (all active): 0 marks an empty slot
 *   gamma_limit  int32 [B] or NULL: per-row upper bound (negative = 0)
 *   state        double [B][2] {A, T}, read and written; zero for a new
 *                request (zero a slot's pair when it takes a new request)
 *   out_gamma    int32 [B]; may be the same array as gamma_used (each row
 *                is read before it is written, by the same thread)
 *   out_alpha    double [B] or NULL: the running acceptance each active row
 *                used (0 for inactive rows)
 * B >= 0 (0: nothing is launched), 0 <= gamma_max <= SPEC_GAMMA_MAX_LIMIT,
 * decay and prior_alpha in [0, 1], prior_weight and draft_cost finite and
 * >= 0, batch_off >= 0 (0: never off).  int32 arrays 4-byte and doubles
 * 8-byte aligned.  Returns SPEC_ERR_SHAPE (B, gamma_max), SPEC_ERR_ARG
 * (the parameters), SPEC_ERR_NULL (state, out_gamma, or one of
 * n_accepted / gamma_used without the other), SPEC_ERR_ALIGN. */
int spec_gamma_control(const int32_t* n_accepted, const int32_t* gamma_used,
                       const int32_t* active, const int32_t* gamma_limit, double* state, int B,
                       int gamma_max, double decay, double prior_alpha, double prior_weight,
                       double draft_cost, int batch_off, int32_t* out_gamma, double* out_alpha,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_ADAPT_H */
