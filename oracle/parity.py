"""Comparison of a GPU verify result with the oracle (test infrastructure).

Acceptance rule:
  * greedy: tokens, accepted counts and new lengths bit-exact;
  * sampling (and point-mass drafts, where q_i(x_i) = 1 and only target rows
    have statistics): probabilities p_i(x_i), q_i(x_i) within 1e-5 relative (values
    below 1e-30 within 1e-35 absolute, where fp32 exp loses relative
    accuracy and no decision depends on them); every row whose tokens,
    count or new length differ must be attributable to rounding: its first
    divergence is either an accept decision with |u - p/q| < 1e-5, or a draw
    where the oracle's normalised CDF between the two tokens stays within
    1e-5 of u (and the GPU's token has positive weight).
  * at most one row in 10^4 may differ at all (>= 99.99 % of rows
    identical): floor(1e-4 * rows) mismatched rows over a run.  The drawn
    distribution is formed in double precision on the GPU, so its CDF
    boundaries sit within ~1e-13 of the oracle's and a draw differs only
    when u falls that close to one; the acceptance test runs in fp32
    against statistics good to ~1e-7, so a decision differs only when u is
    that close to p/q.  Both are far rarer than 1e-4 per row.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle

TOL = 1e-5
TINY, TINY_ABS = 1e-30, 1e-35
CDF_TOL = 2e-7  # the GPU's bracket is fp64, rounded to fp32 (half an ulp below 1: 3e-8)
MISMATCH_RATE = 1e-4


def allowed_mismatches(rows: int) -> int:
    """Rows allowed to differ: >= 99.99 % of the rows must be identical."""
    return int(MISMATCH_RATE * rows)


@dataclass
class Report:
    rows: int = 0
    mismatched: list = field(default_factory=list)      # (row, reason)
    attributed: list = field(default_factory=list)      # (row, reason)
    prob_errors: list = field(default_factory=list)     # (row, pos, what, gpu, oracle)
    max_rel_p: float = 0.0
    max_rel_stats: float = 0.0
    max_cdf_err: float = 0.0

    @property
    def ok(self) -> bool:
        unexplained = len(self.mismatched) - len(self.attributed)
        rate_ok = len(self.mismatched) <= allowed_mismatches(self.rows)
        return unexplained == 0 and rate_ok and not self.prob_errors

    def merge(self, other: "Report"):
        self.rows += other.rows
        self.mismatched += other.mismatched
        self.attributed += other.attributed
        self.prob_errors += other.prob_errors
        self.max_rel_p = max(self.max_rel_p, other.max_rel_p)
        self.max_rel_stats = max(self.max_rel_stats, other.max_rel_stats)
        self.max_cdf_err = max(self.max_cdf_err, other.max_cdf_err)

    def summary(self) -> str:
        return (f"rows={self.rows} mismatched={len(self.mismatched)} "
                f"(allowed {allowed_mismatches(self.rows)}) "
                f"attributed={len(self.attributed)} prob_errors={len(self.prob_errors)} "
                f"max_rel_p={self.max_rel_p:.2e} max_rel_stats={self.max_rel_stats:.2e} "
                f"max_cdf_err={self.max_cdf_err:.2e}")


def _close(gpu, ref):
    ref = np.asarray(ref, np.float64)
    gpu = np.asarray(gpu, np.float64)
    tiny = np.abs(ref) < TINY
    err = np.abs(gpu - ref)
    ok = np.where(tiny, err <= TINY_ABS, err <= TOL * np.abs(ref))
    rel = np.where(tiny, 0.0, err / np.where(tiny, 1.0, np.abs(ref)))
    return ok, rel


_MODES = {"sample": oracle.SAMPLE, "greedy": oracle.GREEDY, "point": oracle.POINT}


# Top-p cuts closer than this to the boundary (relative to the kept mass) may
# differ by one value: the GPU's masses are fp32 exponentials, each within
# ~1e-7 relative near the top of the row and ~|l - max|/T * 1e-7 further down
# (the exponent's and k2's fp32 rounding), which bounds the error of a
# cumulative mass by a few 1e-7 of the kept mass; 1e-6 covers it.
FILTER_MARGIN = 1e-6


def _filters(case):
    return case.extra.get("top_k", 0), case.extra.get("top_p", 1.0)


def run_oracle(case, threads=0):
    mode = _MODES[case.mode]
    k, p = _filters(case)
    return oracle.verify(case.target, case.draft, case.tokens, case.uniforms, case.gamma,
                         case.kv_len, temperature=case.T, mode=mode, threads=threads,
                         top_k=k, top_p=p)


def compare(case, tokens, n_acc, new_len, probe=None, ref=None, row_offset=0,
            all_rows=False) -> Report:
    """Compare GPU outputs (numpy) for one batch with the oracle.

    Probe statistics are checked for the rows the walk uses -- positions
    0..n of the oracle's stop n (p_i, q_i at x_i; the pairs of t_i and d_i;
    t_g when every draft is accepted) -- since the walk reads no row after
    its stop; all_rows=True checks every row of every batch row (for kernels
    that stream them all)."""
    if ref is None:
        ref = run_oracle(case)
    rep = Report(rows=case.B)
    greedy = case.mode == "greedy"
    if greedy:
        for b in range(case.B):
            if (n_acc[b] != ref.n_accepted[b] or new_len[b] != ref.new_len[b]
                    or not np.array_equal(tokens[b], ref.tokens[b])):
                rep.mismatched.append((row_offset + b, "greedy differs"))
        return rep

    near_cut = ref.fmargin < FILTER_MARGIN
    if probe is not None:
        g = case.gamma
        for b in range(case.B):
            if ref.n_accepted[b] < 0 or near_cut[b]:
                continue
            n_or = int(ref.n_accepted[b])
            tested = int(g[b]) if all_rows else min(n_or + 1, int(g[b]))
            for i in range(tested):
                if np.isnan(ref.px[b, i]):
                    continue
                for what, gv, ov in (("p", probe["px"][b, i], ref.px[b, i]),
                                     ("q", probe["qx"][b, i], ref.qx[b, i])):
                    ok, rel = _close(gv, ov)
                    rep.max_rel_p = max(rep.max_rel_p, float(rel))
                    if not ok:
                        rep.prob_errors.append((row_offset + b, i, what, float(gv), float(ov)))
            # per vocabulary row statistics: max exact, S within 1e-5 relative
            gb = int(g[b])
            nt = gb + 1 if all_rows else min(n_or, gb) + 1  # t_0 .. t_n
            nd = gb if all_rows else min(n_or + 1, gb)      # d_0 .. d_n (d_g does not exist)
            slots = list(range(nt))
            if case.mode == "sample":
                slots += [case.G + 1 + i for i in range(nd)]
            for sl in slots:
                if probe["m"][b, sl] != np.float32(ref.m[b, sl]):
                    rep.prob_errors.append((row_offset + b, sl, "m", float(probe["m"][b, sl]),
                                            float(ref.m[b, sl])))
                ok, rel = _close(probe["s"][b, sl], ref.s[b, sl])
                rep.max_rel_stats = max(rep.max_rel_stats, float(rel))
                if not ok:
                    rep.prob_errors.append((row_offset + b, sl, "S", float(probe["s"][b, sl]),
                                            float(ref.s[b, sl])))
            # normaliser of the drawn distribution
            zr, zg = ref.z[b], probe["z"][b]
            if not (abs(zg - zr) <= TOL * abs(zr) + 1e-6):
                rep.prob_errors.append((row_offset + b, -1, "Z", float(zg), float(zr)))
            # the drawn token's CDF bracket, where both sides drew the same
            # token: the GPU's fp64 CDF (rounded to fp32 on output) against
            # the oracle's, and the GPU's own bracket holds its uniform
            if "flo" in probe and np.array_equal(tokens[b], ref.tokens[b]):
                for what, gv, ov in (("F_lo", probe["flo"][b], ref.flo[b]),
                                     ("F_hi", probe["fhi"][b], ref.fhi[b])):
                    err = abs(float(gv) - float(ov))
                    rep.max_cdf_err = max(rep.max_cdf_err, err)
                    if not err <= CDF_TOL:
                        rep.prob_errors.append((row_offset + b, -1, what, float(gv), float(ov)))
                n = int(ref.n_accepted[b])
                us = float(case.uniforms[b, n + 1 if n < g[b] else g[b]])
                if not (probe["flo"][b] - CDF_TOL <= us <= probe["fhi"][b] + CDF_TOL):
                    rep.prob_errors.append((row_offset + b, -1, "u outside [F_lo, F_hi]",
                                            float(probe["flo"][b]), us))

    for b in range(case.B):
        same = (n_acc[b] == ref.n_accepted[b] and new_len[b] == ref.new_len[b]
                and np.array_equal(tokens[b], ref.tokens[b]))
        if same:
            continue
        rep.mismatched.append((row_offset + b, "sample differs"))
        why = (f"top-p cut within {ref.fmargin[b]:.1e} of the boundary" if near_cut[b]
               else _attribute(case, b, int(n_acc[b]), tokens[b], ref))
        if why:
            rep.attributed.append((row_offset + b, why))
    return rep


def _attribute(case, b, n_gpu, tok_gpu, ref):
    n_or = int(ref.n_accepted[b])
    if n_gpu < 0 or n_or < 0:
        return None
    u = case.uniforms[b].astype(np.float64)
    if n_gpu != n_or:
        k = min(n_gpu, n_or)
        ratio = ref.px[b, k] / ref.qx[b, k] if ref.qx[b, k] > 0 else np.inf
        if abs(u[k] - ratio) < TOL and np.array_equal(tok_gpu[:k], ref.tokens[b, :k]):
            return f"accept decision at {k}: |u - p/q| = {abs(u[k] - ratio):.2e}"
        return None
    if not np.array_equal(tok_gpu[:n_or], ref.tokens[b, :n_or]):
        return None
    jg, jo = int(tok_gpu[n_or]), int(ref.tokens[b, n_or])
    if not (0 <= jg < case.V):
        return None
    k, p = _filters(case)
    cdf, pos = oracle.draw_cdf(case.target, case.draft, case.tokens, case.uniforms, case.gamma, b,
                               temperature=case.T, mode=_MODES[case.mode], top_k=k, top_p=p)
    if pos != n_or:
        return None
    us = u[n_or + 1] if n_or < case.gamma[b] else u[int(case.gamma[b])]
    lo, hi = min(jg, jo), max(jg, jo)
    f_lo = cdf[lo]
    f_hi1 = cdf[hi - 1]
    w_gpu = cdf[jg] - (cdf[jg - 1] if jg > 0 else 0.0)
    if f_lo >= us - TOL and f_hi1 <= us + TOL and w_gpu > 0:
        return f"draw boundary: u={us:.7f} F[{lo}]={f_lo:.7f} F[{hi - 1}]={f_hi1:.7f}"
    return None
