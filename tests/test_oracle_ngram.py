"""Pins for the oracle's prompt-lookup (n-gram) drafting.

The pages describe the drafter as copying what followed the last earlier
occurrence of the context's current suffix (mhtirogla.ai "Speculative
decoding", Implementation notes; inference.tusharamrit.in "Speculative
decoding", Self-speculation).  The oracle is pinned by hand-worked examples
and by a brute force built on Python's own substring search (str.rfind), which
finds the last occurrence that ends before the context's final token.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_examples.json")


def _text(tokens):
    # one code point per token, so substring search is token-aligned
    return "".join(chr(0x100 + int(t)) for t in tokens)


def brute(tokens, L, n_min, n_max, gamma):
    """Longest n first; the last occurrence of the n-token suffix lying inside
    the first L - 1 tokens; the continuation cut at gamma and at L."""
    s = _text(tokens[:L])
    for n in range(n_max, n_min - 1, -1):
        if L < n + 1:
            continue
        j = s.rfind(s[L - n:], 0, L - 1)
        if j >= 0:
            start = j + n
            return list(tokens[start:min(start + gamma, L)]), n, start
    return [], -1, -1


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["what"][:40])
def test_worked_examples(case):
    ctx = np.array([case["context"]], np.int32)
    r = oracle.ngram_draft(ctx, [len(case["context"])], n_min=case["n_min"],
                           n_max=case["n_max"], gamma=case["gamma"])
    assert list(r.draft[0, :r.length[0]]) == case["draft"]
    assert (r.draft[0, r.length[0]:] == -1).all()
    assert r.n[0] == case["n"] and r.pos[0] == case["pos"]


@pytest.mark.parametrize("alphabet", [2, 3, 5, 50])
def test_brute_force_random(alphabet):
    rng = np.random.default_rng(100 + alphabet)
    B, stride = 300, 40
    ctx = rng.integers(0, alphabet, size=(B, stride), dtype=np.int32)
    lens = rng.integers(0, stride + 1, size=B).astype(np.int32)
    for n_min, n_max, gamma in ((1, 4, 4), (2, 3, 8), (1, 1, 1), (3, 7, 5), (1, 6, 0)):
        r = oracle.ngram_draft(ctx, lens, n_min=n_min, n_max=n_max, gamma=gamma)
        for b in range(B):
            d, n, pos = brute(ctx[b], int(lens[b]), n_min, n_max, gamma)
            assert list(r.draft[b, :r.length[b]]) == d, (b, n_min, n_max)
            assert (r.draft[b, r.length[b]:] == -1).all()
            assert (r.n[b], r.pos[b]) == (n, pos), (b, n_min, n_max)


def test_invariants_long_rows():
    """Properties that hold at any size: the copied tokens follow an exact
    earlier occurrence of the suffix, no later occurrence of it exists, and no
    longer suffix occurs at all."""
    rng = np.random.default_rng(7)
    B, stride, n_min, n_max, gamma = 16, 3000, 1, 4, 6
    ctx = rng.integers(0, 40, size=(B, stride), dtype=np.int32)
    lens = rng.integers(stride // 2, stride + 1, size=B).astype(np.int32)
    r = oracle.ngram_draft(ctx, lens, n_min=n_min, n_max=n_max, gamma=gamma)
    for b in range(B):
        L, n, pos, k = int(lens[b]), int(r.n[b]), int(r.pos[b]), int(r.length[b])
        c = ctx[b]
        assert n_min <= n <= n_max
        assert (c[pos - n:pos] == c[L - n:L]).all() and pos <= L - 1
        assert k == min(gamma, L - pos) and (r.draft[b, :k] == c[pos:pos + k]).all()
        s = _text(c[:L])
        assert s.rfind(s[L - n:], pos - n + 1, L - 1) == -1     # none later
        if n < n_max:
            assert s.rfind(s[L - n - 1:], 0, L - 1) == -1        # none longer


def test_invalid_lengths_and_arguments():
    ctx = np.arange(12, dtype=np.int32).reshape(2, 6) % 3
    r = oracle.ngram_draft(ctx, [-1, 7], n_min=1, n_max=2, gamma=3)
    assert (r.length == 0).all() and (r.n == -2).all() and (r.pos == -1).all()
    assert (r.draft == -1).all()
    for kw in (dict(n_min=0), dict(n_min=3, n_max=2), dict(gamma=-1)):
        args = dict(n_min=1, n_max=2, gamma=2) | kw
        with pytest.raises(ValueError):
            oracle.ngram_draft(ctx, [6, 6], **args)


def test_empty_batch():
    r = oracle.ngram_draft(np.zeros((0, 5), np.int32), np.zeros(0, np.int32), gamma=3)
    assert r.draft.shape == (0, 3) and r.length.shape == (0,)
