"""Closed-form yield and speedup of speculative decoding (test infrastructure).

These are the formulas the pages state under an i.i.d. acceptance rate alpha.
They are used by the tests to check the oracle's (and the GPU path's)
realised tokens per pass; nothing on the verify path calls them.

Sources: "Speculative decoding" (mhtirogla.ai), summary line and "How it
works" (E and the speedup E / (1 + gamma*c)), "Complexity and constants"
(alpha = sum min(p, q)); "Speculative decoding: the secretary who types ahead
of the boss" (blog.lo0.es), "The maths that matters" (E, speedup and the
ceiling 1/(1 - alpha)); "Speculative decoding" (inference.tusharamrit.in),
the yield and speedup section (E, speedup, break-even).
"""
from __future__ import annotations

import numpy as np


def expected_tokens(alpha: float, gamma: int) -> float:
    """E = (1 - alpha^(gamma+1)) / (1 - alpha); gamma+1 when alpha == 1.

    The blog.lo0.es rendering writes the geometric sum with an extra
    alpha^(gamma+1) term; the closed form on the right of that equation (and
    on the other three pages) is used here.
    """
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def expected_tokens_product(alphas) -> float:
    """Mean emitted count with per-position acceptance probabilities
    alpha_0..alpha_{g-1}: sum_{k=0..g} prod_{i<k} alpha_i (one token per
    accepted draft plus the one drawn token).  Equals expected_tokens when
    all alphas are equal."""
    total, run = 1.0, 1.0
    for a in alphas:
        run *= a
        total += run
    return total


def ceiling(alpha: float) -> float:
    """Limit of E as gamma grows: 1 / (1 - alpha)."""
    return 1.0 / (1.0 - alpha)


def speedup(alpha: float, gamma: int, c: float) -> float:
    """Wall-clock speedup E / (gamma*c + 1), c = draft cost per target pass."""
    return expected_tokens(alpha, gamma) / (gamma * c + 1.0)


def acceptance_rate(p: np.ndarray, q: np.ndarray) -> float:
    """alpha = sum_x min(p(x), q(x)) = 1 - TV(p, q)."""
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())
