"""Pins for the oracle's adaptive draft-length controller.

The pages give the objective (tokens per pass E = (1 - a^(g+1)) / (1 - a) and
the wall-clock speedup E / (1 + g c): mhtirogla.ai "Efficiency",
inference.tusharamrit.in worked speedup cases, blog.lo0.es "The maths that
matters") and say that g should follow each request's running acceptance
and that speculation should stop at large batch.  The pins: the objective
through the pages' closed form (numpy, with division) against the
oracle's summed, division-free comparison; the printed speedups; the
discounted counts against their closed-form sums; special cases; and a
simulation in which the running acceptance finds a known true rate.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_values.json")


def closed_speedup(a, g, c):
    a = np.float64(a)
    e = g + 1.0 if a == 1.0 else (1.0 - a ** (g + 1)) / (1.0 - a)
    return e / (1.0 + g * c)


def best_gamma(a, c, cap):
    """argmax of the closed-form speedup over 0..cap (smallest on ties), and
    whether the runner-up is too close to call."""
    s = np.array([closed_speedup(a, g, c) for g in range(cap + 1)])
    k = int(np.argmax(s))
    others = np.delete(s, k)
    close = others.size and np.max(others) >= s[k] * (1 - 1e-12)
    return k, bool(close)


def prior_only(alpha, c, cap, B=1):
    """Controller output with no evidence: alpha is the prior."""
    st = np.zeros((B, 2))
    g, a = oracle.gamma_control(st, gamma_max=cap, prior_alpha=alpha, prior_weight=1.0,
                                draft_cost=c)
    return g, a


def test_printed_speedups_and_choice():
    """The closed form reproduces every speedup the pages print; where the
    page's own gamma loses to another one, the controller does not pick it."""
    for row in json.load(open(GOLDEN))["speedup"]:
        a, g, c = row["alpha"], row["gamma"], row["c"]
        s = closed_speedup(a, g, c)
        assert round(s, row["digits"]) == pytest.approx(row["value"]), row
        got, _ = prior_only(a, c, 16)
        want, close = best_gamma(a, c, 16)
        assert not close and got[0] == want
        assert closed_speedup(a, int(got[0]), c) >= s
    # the page's losing case (a = 0.4, c = 0.3, gamma = 4: 0.75x) speculates one token
    assert prior_only(0.4, 0.3, 4)[0][0] == 1


@pytest.mark.parametrize("cap", [0, 1, 4, 8, 63])
def test_choice_matches_closed_form(cap):
    rng = np.random.default_rng(cap)
    alphas = np.concatenate([rng.random(300), [0.0, 1.0, 0.5, 0.999999]])
    costs = np.concatenate([rng.random(300) * 0.5, [0.0, 0.3, 1.0, 2.0]])
    for a in alphas:
        for c in costs[:: 17]:
            got, al = prior_only(a, c, cap)
            assert al[0] == a
            want, close = best_gamma(a, c, cap)
            if not close:
                assert got[0] == want, (a, c, cap)


def test_special_cases_and_monotone():
    assert prior_only(0.0, 0.05, 8)[0][0] == 0          # nothing is ever accepted
    assert prior_only(0.0, 0.0, 8)[0][0] == 0           # all tie: the shortest
    assert prior_only(0.3, 0.0, 8)[0][0] == 8           # free drafts: as many as allowed
    assert prior_only(1.0, 0.5, 8)[0][0] == 8           # certain acceptance, c < 1
    assert prior_only(0.9, 0.05, 0)[0][0] == 0          # cap 0
    # more acceptance never shortens the draft; a dearer draft never lengthens it
    prev = -1
    for a in np.linspace(0, 1, 101):
        g = prior_only(a, 0.1, 12)[0][0]
        assert g >= prev
        prev = g
    prev = 99
    for c in np.linspace(0, 1.5, 61):
        g = prior_only(0.8, c, 12)[0][0]
        assert g <= prev
        prev = g


def test_discounted_counts_closed_form():
    """After rounds t = 1..R, A = sum d^(R-t) n_t and T = sum d^(R-t) tested_t
    over the rounds with an observation (every round ages the evidence)."""
    rng = np.random.default_rng(3)
    B, R, d = 50, 40, 0.85
    st = np.zeros((B, 2))
    ns, ts = [], []
    for _ in range(R):
        g = rng.integers(0, 9, size=B).astype(np.int32)
        n = np.array([rng.integers(0, gi + 1) if gi else 0 for gi in g], np.int32)
        n[rng.random(B) < 0.05] = -1                       # data errors: no observation
        oracle.gamma_control(st, n, g, gamma_max=8, decay=d)
        ok = (g >= 1) & (n >= 0)
        ns.append(np.where(ok, n, 0).astype(np.float64))
        ts.append(np.where(ok, np.minimum(n + 1, g), 0).astype(np.float64))
    w = d ** np.arange(R - 1, -1, -1)
    np.testing.assert_allclose(st[:, 0], w @ np.array(ns), rtol=1e-12)
    np.testing.assert_allclose(st[:, 1], w @ np.array(ts), rtol=1e-12)


def test_running_acceptance_formula():
    st = np.array([[3.0, 4.0], [0.0, 0.0], [5.0, 10.0]])
    _, a = oracle.gamma_control(st, None, None, decay=1.0, prior_alpha=0.6, prior_weight=2.0)
    np.testing.assert_allclose(a, [(3 + 1.2) / 6, 0.6, (5 + 1.2) / 12], rtol=1e-15)
    st = np.zeros((1, 2))
    _, a = oracle.gamma_control(st, None, None, prior_alpha=0.3, prior_weight=0.0)
    assert a[0] == 0.3                                      # no evidence, no prior weight


def test_batch_switch_off_and_inactive_rows():
    rng = np.random.default_rng(5)
    B = 40
    g = rng.integers(1, 5, size=B).astype(np.int32)
    n = rng.integers(0, 5, size=B).astype(np.int32) % (g + 1)
    active = (rng.random(B) < 0.75).astype(np.int32)
    s_on, s_off = np.zeros((B, 2)), np.zeros((B, 2))
    kw = dict(gamma_max=6, prior_alpha=0.9, draft_cost=0.02)
    g_on, _ = oracle.gamma_control(s_on, n, g, active=active, batch_off=int(active.sum()) + 1, **kw)
    g_off, _ = oracle.gamma_control(s_off, n, g, active=active, batch_off=int(active.sum()), **kw)
    assert (g_off == 0).all() and (g_on[active == 1] > 0).all()
    np.testing.assert_array_equal(s_on, s_off)              # the state updates either way
    assert (g_on[active == 0] == 0).all() and (s_on[active == 0] == 0).all()


def test_gamma_limit():
    st = np.zeros((4, 2))
    g, _ = oracle.gamma_control(st, gamma_limit=[0, 2, 9, -3], gamma_max=6, prior_alpha=0.95,
                                draft_cost=0.01)
    assert g.tolist() == [0, 2, 6, 0]


def test_tracks_a_true_acceptance_rate():
    """Requests whose drafts are accepted independently with a fixed true
    rate: after many rounds the running acceptance is near it and the draft
    length is the best one for it."""
    rng = np.random.default_rng(11)
    true = np.array([0.2, 0.5, 0.7, 0.85, 0.95] * 20)
    B, c, cap, d = len(true), 0.05, 10, 0.995
    st = np.zeros((B, 2))
    n = g = None
    for _ in range(3000):
        gam, alpha = oracle.gamma_control(st, n, g, gamma_max=cap, decay=d, prior_alpha=0.5,
                                          prior_weight=1.0, draft_cost=c)
        # accepted count of a round: the first rejection among gam tests
        u = rng.random((B, cap))
        rej = u >= true[:, None]
        first = np.where(rej.any(axis=1), rej.argmax(axis=1), cap)
        n, g = np.minimum(first, gam).astype(np.int32), gam
    # discounted counts over ~200 rounds: a few hundredths of spread
    assert np.abs(alpha - true).max() < 0.08
    for a_true in np.unique(true):
        want, close = best_gamma(a_true, c, cap)
        rows = true == a_true
        if not close:
            assert abs(np.median(gam[rows]) - want) <= 1, (a_true, gam[rows], want)


def test_refused_arguments():
    st = np.zeros((2, 2))
    for kw in (dict(decay=1.5), dict(decay=-0.1), dict(prior_alpha=1.1), dict(prior_weight=-1.0),
               dict(draft_cost=-0.1), dict(draft_cost=np.inf), dict(batch_off=-1),
               dict(gamma_max=-1)):
        with pytest.raises(ValueError):
            oracle.gamma_control(st, **kw)
    with pytest.raises(ValueError):
        oracle.gamma_control(st, [1, 1], None)
