"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print (tests/golden), special cases that reduce to a library routine
(numpy searchsorted over a cumulative sum, numpy argmax, scipy's softmax),
identities (the residual normaliser), and invariants the pages state.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from oracle import closed_form as cf
from speculative_decoding_verification_07_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _probs(stored, T):
    """Library softmax of stored logits at temperature T (float64)."""
    return softmax(inputs.widen(stored).astype(np.float64) / T, axis=-1)


def _inverse_cdf(w, u):
    """Textbook inverse-CDF draw: first j with u * sum(w) < cumsum(w)[j]."""
    c = np.cumsum(w)
    return int(np.searchsorted(c, np.float64(u) * c[-1], side="right"))


def _single_position_batch(p, q, xs, us):
    """B rows of a gamma=1 problem with fixed p (both target rows) and q."""
    B = len(xs)
    lp = np.log(np.asarray(p, np.float64)).astype(np.float32)
    lq = np.log(np.asarray(q, np.float64)).astype(np.float32)
    target = np.broadcast_to(lp, (B, 2, len(p))).copy()
    draft = np.broadcast_to(lq, (B, 1, len(q))).copy()
    tokens = np.asarray(xs, np.int32).reshape(B, 1)
    uniforms = np.asarray(us, np.float32).reshape(B, 2)
    gamma = np.ones(B, np.int32)
    return target, draft, tokens, uniforms, gamma


# ---------------------------------------------------------------- page 1 example
def test_page1_acceptance_terms_and_residual():
    g = _gold("page1_worked_example.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    # every possible draft token, with a uniform that rejects (0.99 > p/q for x in {2, 3})
    xs = np.array([0, 1, 2, 3])
    us = np.array([[0.99, 0.5]] * 4)
    t, d, x, u, gam = _single_position_batch(p, q, xs, us)
    r = oracle.verify(t, d, x, u, gam, temperature=1.0)
    # p_i(x) and q_i(x) are the page's probabilities
    np.testing.assert_allclose(r.px[:, 0], p, rtol=1e-6)
    np.testing.assert_allclose(r.qx[:, 0], q, rtol=1e-6)
    # acceptance probability min(1, p/q) weighted by q sums to the printed 0.700
    acc = np.minimum(1.0, r.px[:, 0] / r.qx[:, 0])
    np.testing.assert_allclose(q @ acc, g["acceptance_rate"], atol=1e-6)
    np.testing.assert_allclose(q * acc, g["acceptance_terms"], atol=1e-6)
    # x in {0, 1}: p >= q, accepted whatever u; x in {2, 3}: p/q < 0.99, rejected
    assert list(r.n_accepted) == [1, 1, 0, 0]
    # rejected rows draw from norm(max(0, p - q)) = [0.25, 0.05, 0, 0] / 0.30
    for row in (2, 3):
        np.testing.assert_allclose(r.z[row], g["residual_mass"], atol=1e-6)
        cdf, pos = oracle.draw_cdf(t, d, x, u, gam, row)
        assert pos == 0
        want = np.cumsum(g["residual_unnormalised"]) / g["residual_mass"]
        np.testing.assert_allclose(cdf, want, atol=1e-6)
        # u = 0.5 < 0.25/0.30, so the drawn token is 0
        assert r.tokens[row, 0] == 0


def test_page1_selftest_replay():
    """The page's own statistical self-test, replayed with its generator and
    stream order: one uniform to draw x from q, one for the test, one for the
    single draw.  The first emitted token must follow p within 0.005 and the
    acceptance rate must be 0.700 (checked to 4 sigma)."""
    from oracle.pagerng import XorShift64Star

    g = _gold("page1_worked_example.json")
    st = g["selftest"]
    n = st["trials"]
    p, q = np.array(g["p"]), np.array(g["q"])
    rng = XorShift64Star(int(st["seed_hex"], 16))
    f = rng.uniforms(3 * n).reshape(n, 3)
    xs = np.array([_inverse_cdf(q, f[k, 0]) for k in range(n)])
    t, d, x, u, gam = _single_position_batch(p, q, xs, f[:, 1:])
    r = oracle.verify(t, d, x, u, gam, temperature=1.0)
    freq = np.bincount(r.tokens[:, 0], minlength=4) / n
    assert np.all(np.abs(freq - p) < st["frequency_tolerance"]), freq
    alpha = np.mean(r.n_accepted == 1)
    sigma = np.sqrt(0.7 * 0.3 / n)
    assert abs(alpha - st["printed_acceptance"]) < 4 * sigma + 5e-4, alpha


# ---------------------------------------------------------------- special cases
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gamma0_is_inverse_cdf_sampling(dtype):
    """gamma = 0 is plain sampling from p_0 by inverse CDF with u_0."""
    case = inputs.make_case(1, rnd=3, B=300, G=2, V=997, dtype=dtype, T=0.9)
    gamma = np.zeros(case.B, np.int32)
    r = oracle.verify(case.target, case.draft, case.tokens, case.uniforms, gamma,
                      case.kv_len, temperature=0.9)
    p0 = _probs(case.target[:, 0], 0.9)
    want = [_inverse_cdf(p0[b], case.uniforms[b, 0]) for b in range(case.B)]
    assert list(r.tokens[:, 0]) == want
    assert np.all(r.tokens[:, 1:] == -1)
    assert np.all(r.n_accepted == 0)
    np.testing.assert_array_equal(r.new_len, case.kv_len)


def test_gamma0_greedy_is_argmax_with_ties():
    rng = np.random.default_rng(7)
    B, V = 64, 300
    t = rng.normal(0, 2, size=(B, 1, V)).astype(np.float32)
    # exact ties of the maximum at two or three indices, and a -0/+0 tie
    for b in range(0, B, 2):
        idx = rng.choice(V, size=3, replace=False)
        t[b, 0, idx] = t[b, 0].max() + 1.0
    t[1, 0, :] = -1.0
    t[1, 0, 40] = -0.0
    t[1, 0, 10] = 0.0
    r = oracle.verify(t, None, np.zeros((B, 0), np.int32), None, np.zeros(B, np.int32),
                      mode=oracle.GREEDY)
    assert list(r.tokens[:, 0]) == list(np.argmax(t[:, 0], axis=1))
    assert r.tokens[1, 0] == 10


def test_identical_draft_accepts_everything():
    """q == p: u*q < p holds for every u < 1, so all gamma drafts are
    accepted and the bonus token is an inverse-CDF draw from p_gamma."""
    case = inputs.make_case(2, rnd=1, B=40, V=500)
    draft = case.target[:, :case.G].copy()
    r = oracle.verify(case.target, draft, case.tokens, case.uniforms, case.gamma,
                      temperature=case.T)
    assert np.all(r.n_accepted == case.gamma)
    pg = _probs(case.target[:, case.G], case.T)
    want = [_inverse_cdf(pg[b], case.uniforms[b, case.G]) for b in range(case.B)]
    assert list(r.tokens[:, case.G]) == want
    np.testing.assert_array_equal(r.tokens[:, :case.G], case.tokens)


def test_disjoint_supports_reject_and_draw_from_p():
    """p(x) = 0 for every draft token (supports disjoint): the first test
    rejects whatever u is, and the residual max(0, p - q) is p itself."""
    rng = np.random.default_rng(11)
    B, G, V = 50, 3, 64
    t = rng.normal(0, 1, size=(B, G + 1, V)).astype(np.float32)
    d = rng.normal(0, 1, size=(B, G, V)).astype(np.float32)
    t[:, :, : V // 2] = -np.inf     # p lives on the upper half
    d[:, :, V // 2:] = -np.inf      # q lives on the lower half
    x = rng.integers(0, V // 2, size=(B, G)).astype(np.int32)
    u = rng.random((B, G + 1)).astype(np.float32)
    r = oracle.verify(t, d, x, u, np.full(B, G, np.int32), temperature=1.0)
    assert np.all(r.n_accepted == 0)
    p0 = _probs(t[:, 0], 1.0)
    want = [_inverse_cdf(p0[b], u[b, 1]) for b in range(B)]
    assert list(r.tokens[:, 0]) == want
    np.testing.assert_allclose(r.z, 1.0, atol=1e-12)


def test_probabilities_match_library_softmax():
    case = inputs.make_case(3, rnd=2, B=6, V=3000)
    r = oracle.verify(case.target, case.draft, case.tokens, case.uniforms, case.gamma,
                      temperature=case.T)
    P = _probs(case.target, case.T)
    Q = _probs(case.draft, case.T)
    for b in range(case.B):
        for i in range(case.G):
            if np.isnan(r.px[b, i]):
                continue
            x = case.tokens[b, i]
            assert r.px[b, i] == pytest.approx(P[b, i, x], rel=1e-12)
            assert r.qx[b, i] == pytest.approx(Q[b, i, x], rel=1e-12)
    # raw max and the log of the exp-sum relative to it
    lt = inputs.widen(case.target).astype(np.float64)
    np.testing.assert_array_equal(r.m[:, : case.G + 1], lt.max(axis=-1))
    want = logsumexp((lt - lt.max(axis=-1, keepdims=True)) / case.T, axis=-1)
    np.testing.assert_allclose(np.log(r.s[:, : case.G + 1]), want, rtol=1e-12, atol=1e-12)


def test_residual_normaliser_identity():
    """sum max(0, p - q) = 1 - sum min(p, q) (the rejection probability)."""
    case = inputs.make_case(4, rnd=1, B=24, V=2000)
    r = oracle.verify(case.target, case.draft, case.tokens, case.uniforms, case.gamma,
                      temperature=case.T)
    P = _probs(case.target, case.T)
    Q = _probs(case.draft, case.T)
    rejected = np.nonzero(r.n_accepted < case.gamma)[0]
    assert len(rejected) > 5
    for b in rejected:
        n = r.n_accepted[b]
        assert r.draw_pos[b] == n
        assert r.z[b] == pytest.approx(1.0 - np.minimum(P[b, n], Q[b, n]).sum(), abs=1e-12)


@pytest.mark.parametrize("cfg,mode", [(1, "sample"), (2, "sample"), (3, "sample"), (5, "sample"),
                                      (3, "greedy"), (4, "greedy")])
def test_invariants(cfg, mode):
    case = inputs.make_case(cfg, rnd=5, mode=mode, B=32, V=1500)
    m = oracle.GREEDY if mode == "greedy" else oracle.SAMPLE
    r = oracle.verify(case.target, case.draft, case.tokens, case.uniforms, case.gamma,
                      case.kv_len, temperature=case.T, mode=m)
    P = _probs(case.target, case.T)
    Q = _probs(case.draft, case.T)
    for b in range(case.B):
        n, g = r.n_accepted[b], case.gamma[b]
        assert 0 <= n <= g
        tok = r.tokens[b]
        np.testing.assert_array_equal(tok[:n], case.tokens[b, :n])
        assert 0 <= tok[n] < case.V
        assert np.all(tok[n + 1:] == -1)
        assert r.new_len[b] == case.kv_len[b] + n
        if mode == "greedy":
            assert tok[n] == np.argmax(inputs.widen(case.target[b, n]))
            if n < g:
                assert case.tokens[b, n] != tok[n]
        elif n < g:
            # the correction has positive residual weight and is not x_n
            assert tok[n] != case.tokens[b, n]
            assert P[b, n, tok[n]] > Q[b, n, tok[n]]


def test_data_errors_write_sentinel():
    case = inputs.make_case(2, rnd=9, B=6, V=400)
    g = case.gamma.copy()
    g[0] = -1                 # gamma below range
    g[1] = case.G + 1         # gamma above range
    x = case.tokens.copy()
    x[2, 0] = case.V          # tested token out of range
    t = case.target.copy()
    t[3, 0, :] = 0xFF80       # bf16 -inf: p_0, which every walk uses, has no finite logit
    d = case.draft.copy()
    d[4, 0, :] = 0xFF80       # q_0 likewise (row 4 tests position 0: gamma >= 1)
    assert g[4] >= 1
    r = oracle.verify(t, d, x, case.uniforms, g, case.kv_len, temperature=case.T)
    for b in range(5):
        assert r.n_accepted[b] == -1
        assert np.all(r.tokens[b] == -1)
        assert r.new_len[b] == case.kv_len[b]
    assert r.n_accepted[5] >= 0
    # a dead row after the stop is never used: the result is unchanged
    case3 = inputs.make_case(3, rnd=10, B=32, V=300)
    r0 = oracle.verify(case3.target, case3.draft, case3.tokens, case3.uniforms, case3.gamma,
                       temperature=case3.T)
    rows = [b for b in range(case3.B) if r0.n_accepted[b] < case3.gamma[b] - 1]
    assert len(rows) >= 4
    t3, d3 = case3.target.copy(), case3.draft.copy()
    for b in rows:
        n = r0.n_accepted[b]
        t3[b, n + 1, :] = 0xFF80
        d3[b, n + 1, :] = 0xFF80
        t3[b, case3.gamma[b], :] = 0xFF80   # the bonus row is not used after a rejection
    r1 = oracle.verify(t3, d3, case3.tokens, case3.uniforms, case3.gamma, temperature=case3.T)
    np.testing.assert_array_equal(r1.tokens, r0.tokens)
    np.testing.assert_array_equal(r1.n_accepted, r0.n_accepted)
    # ... but a dead bonus row is used when every draft is accepted
    full = [b for b in range(case3.B) if r0.n_accepted[b] == case3.gamma[b]]
    assert full
    if full:
        t4 = case3.target.copy()
        t4[full[0], case3.gamma[full[0]], :] = 0xFF80
        r2 = oracle.verify(t4, case3.draft, case3.tokens, case3.uniforms, case3.gamma,
                           temperature=case3.T)
        assert r2.n_accepted[full[0]] == -1
    # an out-of-range token after the first rejection is never tested
    case2 = inputs.make_case(3, rnd=9, B=16, V=400)
    r0 = oracle.verify(case2.target, case2.draft, case2.tokens, case2.uniforms, case2.gamma,
                       temperature=case2.T)
    b = int(np.argmin(r0.n_accepted))
    n = r0.n_accepted[b]
    assert n < case2.G - 1
    x2 = case2.tokens.copy()
    x2[b, n + 1] = -5
    r1 = oracle.verify(case2.target, case2.draft, x2, case2.uniforms, case2.gamma,
                       temperature=case2.T)
    np.testing.assert_array_equal(r1.tokens[b], r0.tokens[b])
    # greedy: an all -inf row is well defined (every index ties, the lowest wins)
    tg = np.full((2, 1, 50), -np.inf, np.float32)
    rg = oracle.verify(tg, None, np.zeros((2, 0), np.int32), None, np.zeros(2, np.int32),
                       mode=oracle.GREEDY)
    assert list(rg.tokens[:, 0]) == [0, 0]


# ---------------------------------------------------------------- point-mass drafts
@pytest.mark.parametrize("cfg,dtype,G", [(1, "f32", 2), (3, "bf16", 4), (5, "f32", 8)])
def test_point_mode_is_the_textbook_rule(cfg, dtype, G):
    """q_i = indicator of x_i: accept while u_i < p_i(x_i); at the first
    rejection draw from p_n with x_n removed (library softmax, numpy inverse
    CDF); otherwise the bonus from p_g; Z = 1 - p_n(x_n)."""
    case = inputs.make_case(cfg, rnd=11, mode="point", B=96, G=G, V=700, dtype=dtype)
    r = oracle.verify(case.target, None, case.tokens, case.uniforms, case.gamma, case.kv_len,
                      temperature=case.T, mode=oracle.POINT)
    P = _probs(case.target, case.T)
    seen = set()
    for b in range(case.B):
        g, x, u = int(case.gamma[b]), case.tokens[b], case.uniforms[b]
        n = g
        for i in range(g):
            assert r.px[b, i] == pytest.approx(P[b, i, x[i]], rel=1e-12, abs=1e-300)
            assert r.qx[b, i] == 1.0
            if not np.float64(u[i]) < P[b, i, x[i]]:
                n = i
                break
        assert r.n_accepted[b] == n
        if n < g:
            w = P[b, n].copy()
            w[x[n]] = 0.0
            want = _inverse_cdf(w, u[n + 1])
            assert r.z[b] == pytest.approx(1.0 - P[b, n, x[n]], rel=1e-12)
            assert r.tokens[b, n] != x[n]
        else:
            want = _inverse_cdf(P[b, g], u[g])
        assert r.tokens[b, n] == want
        np.testing.assert_array_equal(r.tokens[b, :n], x[:n])
        assert np.all(r.tokens[b, n + 1:] == -1)
        assert r.new_len[b] == case.kv_len[b] + n
        seen.add("reject" if n < g else "full")
    assert seen == {"reject", "full"}


def test_point_mode_equals_sampling_with_one_hot_draft():
    """A draft row whose logits are -inf except at x_i has q_i = indicator of
    x_i exactly, so the general rule must give the same result bit for bit."""
    case = inputs.make_case(2, rnd=12, mode="point", B=40, V=900)
    one_hot = np.full(case.draft.shape, 0xFF80, np.uint16)   # bf16 -inf
    for b in range(case.B):
        for i in range(int(case.gamma[b])):
            one_hot[b, i, case.tokens[b, i]] = 0x3F80             # bf16 1.0
    pt = oracle.verify(case.target, None, case.tokens, case.uniforms, case.gamma, case.kv_len,
                       temperature=case.T, mode=oracle.POINT)
    gen = oracle.verify(case.target, one_hot, case.tokens, case.uniforms, case.gamma,
                        case.kv_len, temperature=case.T)
    np.testing.assert_array_equal(pt.tokens, gen.tokens)
    np.testing.assert_array_equal(pt.n_accepted, gen.n_accepted)
    np.testing.assert_array_equal(pt.z, gen.z)
    np.testing.assert_array_equal(pt.px, gen.px)
    assert np.all(pt.n_accepted < case.gamma) and np.any(pt.n_accepted > 0)


def test_point_mode_data_errors_and_gamma0():
    case = inputs.make_case(1, rnd=13, mode="point", B=5, V=300)
    x = case.tokens.copy()
    x[0, 0] = -1                                # tested token out of range
    t = case.target.copy()
    t[1, 0, :] = -np.inf                        # p_0 has no finite logit
    g = case.gamma.copy()
    g[2] = case.G + 1
    r = oracle.verify(t, None, x, case.uniforms, g, case.kv_len, temperature=case.T,
                      mode=oracle.POINT)
    for b in range(3):
        assert r.n_accepted[b] == -1 and np.all(r.tokens[b] == -1)
        assert r.new_len[b] == case.kv_len[b]
    assert np.all(r.n_accepted[3:] >= 0)
    # gamma = 0 is plain inverse-CDF sampling from p_0, as in sampling mode
    z = np.zeros(case.B, np.int32)
    r0 = oracle.verify(case.target, None, case.tokens, case.uniforms, z, temperature=case.T,
                       mode=oracle.POINT)
    P = _probs(case.target[:, 0], case.T)
    assert list(r0.tokens[:, 0]) == [_inverse_cdf(P[b], case.uniforms[b, 0])
                                     for b in range(case.B)]


# ---------------------------------------------------------------- top-k / top-p
def _row_logits(rng, V, dtype, ties=False):
    x = rng.normal(0, 2.5, size=V).astype(np.float32)
    if ties:  # repeated values around the middle and at the top
        x[rng.choice(V, size=V // 4, replace=False)] = np.float32(0.5)
        x[rng.choice(V, size=3, replace=False)] = x.max()
    return inputs.store(x, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ties", [False, True])
def test_filter_top_k_is_the_kth_largest_value(dtype, ties):
    rng = np.random.default_rng(31)
    for k in (1, 2, 7, 50, 399):
        row = _row_logits(rng, 400, dtype, ties)
        l = inputs.widen(row).astype(np.float64)
        prob, tau = oracle.filter_row(row, temperature=0.8, top_k=k)
        kth = np.partition(l, -k)[-k]          # numpy's k-th largest value
        assert tau == kth
        kept = l >= kth
        assert kept.sum() >= k and (l > kth).sum() < k
        ref = softmax(np.where(kept, l / 0.8, -np.inf))
        np.testing.assert_allclose(prob, ref, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_filter_top_p_keeps_the_smallest_sufficient_set(dtype):
    rng = np.random.default_rng(32)
    for top_p in (1e-9, 0.3, 0.9, 0.999):
        for ties in (False, True):
            row = _row_logits(rng, 600, dtype, ties)
            l = inputs.widen(row).astype(np.float64)
            prob, tau = oracle.filter_row(row, temperature=1.3, top_p=top_p)
            full = softmax(l / 1.3)                 # library softmax, unfiltered
            kept = l >= tau
            assert full[kept].sum() >= top_p * (1 - 1e-12)
            # dropping the smallest kept value (all its copies) falls short
            smaller = l > tau
            assert full[smaller].sum() < top_p
            np.testing.assert_allclose(prob, np.where(kept, full, 0) / full[kept].sum(),
                                       rtol=1e-12, atol=1e-300)
            if top_p == 1e-9:
                assert tau == l.max()


def test_filter_top_p_applies_to_the_top_k_distribution():
    rng = np.random.default_rng(33)
    row = _row_logits(rng, 500, "f32")
    l = row.astype(np.float64)
    k, top_p = 40, 0.6
    _, tau_k = oracle.filter_row(row, top_k=k)
    prob, tau = oracle.filter_row(row, top_k=k, top_p=top_p)
    pk = softmax(np.where(l >= tau_k, l, -np.inf))   # renormalised top-k distribution
    assert tau >= tau_k
    assert pk[l >= tau].sum() >= top_p and pk[l > tau].sum() < top_p


def test_filter_off_is_bit_identical_and_greedy_ignores_it():
    case = inputs.make_case(2, rnd=14, B=12, V=700)
    a = oracle.verify(case.target, case.draft, case.tokens, case.uniforms, case.gamma,
                      case.kv_len, temperature=case.T)
    b = oracle.verify(case.target, case.draft, case.tokens, case.uniforms, case.gamma,
                      case.kv_len, temperature=case.T, top_k=700, top_p=1.0)
    for f in ("tokens", "n_accepted", "px", "qx", "z", "s"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert np.all(np.isinf(b.fmargin))
    g = inputs.make_case(3, rnd=14, mode="greedy", B=8, V=700)
    r0 = oracle.verify(g.target, None, g.tokens, None, g.gamma, mode=oracle.GREEDY)
    r1 = oracle.verify(g.target, None, g.tokens, None, g.gamma, mode=oracle.GREEDY,
                       top_k=1, top_p=0.01)
    np.testing.assert_array_equal(r0.tokens, r1.tokens)
    with pytest.raises(ValueError):
        oracle.verify(g.target, None, g.tokens, None, g.gamma, mode=oracle.GREEDY, top_k=-1)
    with pytest.raises(ValueError):
        oracle.verify(g.target, None, g.tokens, None, g.gamma, mode=oracle.GREEDY, top_p=0.0)


@pytest.mark.parametrize("mode", ["sample", "point"])
def test_filtered_verify_is_the_rule_on_filtered_distributions(mode):
    """With filtering, the probabilities the walk tests are those of the
    filtered rows (numpy check), the drawn token has positive filtered weight,
    and k = 1 reduces sampling to accepting exactly the argmax tokens."""
    case = inputs.make_case(3, rnd=15, mode=mode, B=24, V=900)
    m = oracle.POINT if mode == "point" else oracle.SAMPLE
    k, top_p = 30, 0.8
    r = oracle.verify(case.target, case.draft, case.tokens, case.uniforms, case.gamma,
                      case.kv_len, temperature=case.T, mode=m, top_k=k, top_p=top_p)
    for b in range(case.B):
        n, g = int(r.n_accepted[b]), int(case.gamma[b])
        for i in range(min(n + 1, g)):
            pf, _ = oracle.filter_row(case.target[b, i], temperature=case.T, top_k=k, top_p=top_p)
            assert r.px[b, i] == pytest.approx(pf[case.tokens[b, i]], rel=1e-12, abs=1e-300)
            if mode == "sample":
                qf, _ = oracle.filter_row(case.draft[b, i], temperature=case.T, top_k=k,
                                          top_p=top_p)
                assert r.qx[b, i] == pytest.approx(qf[case.tokens[b, i]], rel=1e-12, abs=1e-300)
        pn, _ = oracle.filter_row(case.target[b, n], temperature=case.T, top_k=k, top_p=top_p)
        assert pn[r.tokens[b, n]] > 0
    one = oracle.verify(case.target, case.draft, case.tokens, case.uniforms, case.gamma,
                        case.kv_len, temperature=case.T, mode=m, top_k=1)
    for b in range(case.B):
        n = int(one.n_accepted[b])
        am = [int(np.argmax(inputs.widen(case.target[b, i]))) for i in range(n + 1)]
        assert list(one.tokens[b, :n + 1]) == am[: n + 1]


# ---------------------------------------------------------------- closed forms
def _rounds_to(value, printed, digits):
    return round(value, digits) == pytest.approx(printed, abs=1e-9)


def test_closed_form_reproduces_page_numbers():
    g = _gold("closed_form_values.json")
    for e in g["expected_tokens"]:
        assert _rounds_to(cf.expected_tokens(e["alpha"], e["gamma"]), e["value"], e["digits"]), e
    for e in g["ceiling"]:
        assert _rounds_to(cf.ceiling(e["alpha"]), e["value"], e["digits"]), e
    for e in g["speedup"]:
        assert _rounds_to(cf.speedup(e["alpha"], e["gamma"], e["c"]), e["value"], e["digits"]), e
    for mis in g["expected_tokens_misprint"]:
        got = cf.expected_tokens(mis["alpha"], mis["gamma"])
        assert got == pytest.approx(mis["formula"], abs=5e-4), mis
        assert abs(got - mis["printed"]) < 0.01, mis
    gains = g["relative_gains"]
    e = cf.expected_tokens
    assert _rounds_to(e(0.9, 4) / e(0.7, 4) - 1, gains[0]["value"], 2)
    assert _rounds_to(e(0.7, 10) / e(0.7, 4) - 1, gains[1]["value"], 2)
    # the product form reduces to the closed form for equal alphas, and the
    # ceiling is its limit
    assert cf.expected_tokens_product([0.8] * 4) == pytest.approx(e(0.8, 4), rel=1e-14)
    assert e(0.9, 400) == pytest.approx(cf.ceiling(0.9), rel=1e-12)


def test_acceptance_rate_is_one_minus_total_variation():
    g = _gold("page1_worked_example.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    assert cf.acceptance_rate(p, q) == pytest.approx(g["acceptance_rate"], abs=1e-12)
    assert cf.acceptance_rate(p, q) == pytest.approx(1 - 0.5 * np.abs(p - q).sum(), abs=1e-12)


# ---------------------------------------------------------------- the draw itself
def test_draw_index_is_the_textbook_inverse_cdf():
    """The oracle's draw over given weights equals numpy's searchsorted over
    the cumulative sum (first j with u Z < C_j), including zero weights,
    which are never chosen ("Speculative decoding", mhtirogla.ai, the
    `sample` routine of "Code")."""
    rng = np.random.default_rng(5)
    for trial in range(200):
        V = int(rng.integers(1, 300))
        w = rng.random(V) * (rng.random(V) < 0.6)
        if not w.any():
            w[int(rng.integers(V))] = 1.0
        u = float(rng.random())
        j, z = oracle.draw_index(w, u)
        assert z == pytest.approx(w.sum(), rel=1e-12)
        assert j == _inverse_cdf(w, u), (trial, V, u)
        assert w[j] > 0


def test_draw_index_fallback_is_last_positive_weight():
    """When no running sum exceeds u Z (here u = 1, one past the uniforms'
    range) the draw returns the last index of positive weight -- not V-1,
    which the page's `sample` would return even when it has weight 0."""
    w = np.array([0.0, 0.3, 0.0, 0.7, 0.0, 0.0])
    j, z = oracle.draw_index(w, 1.0)
    assert j == 3 and z == pytest.approx(1.0)
    # a single positive weight anywhere
    for k in range(6):
        e = np.zeros(6)
        e[k] = 2.5
        assert oracle.draw_index(e, 1.0)[0] == k
        assert oracle.draw_index(e, 0.0)[0] == k


def test_zero_residual_falls_back_to_p():
    """Identical target and draft logits with the drafted token at a -inf
    logit: p(x) = q(x) = 0, so u q(x) < p(x) fails and the walk rejects at
    0, yet max(0, p - q) is 0 everywhere.  The oracle then draws from p_0
    with the next uniform (the reading for a residual without mass) and
    flags the row; the token is numpy's inverse CDF of softmax(t_0)."""
    rng = np.random.default_rng(11)
    B, G, V = 6, 3, 257
    lt = rng.normal(0, 2, size=(B, G + 1, V)).astype(np.float32)
    xs = rng.integers(0, V, size=(B, G)).astype(np.int32)
    for b in range(B):
        lt[b, 0, xs[b, 0]] = -np.inf
    ld = lt[:, :G].copy()
    us = rng.random((B, G + 1), dtype=np.float32)
    gam = np.full(B, G, np.int32)
    r = oracle.verify(lt, ld, xs, us, gam, temperature=0.9)
    p0 = softmax(lt[:, 0].astype(np.float64) / 0.9, axis=-1)
    for b in range(B):
        assert r.n_accepted[b] == 0 and r.zero_resid[b] == 1
        assert r.tokens[b, 0] == _inverse_cdf(p0[b], us[b, 1])
        assert np.all(r.tokens[b, 1:] == -1)
        assert r.z[b] == pytest.approx(1.0, rel=1e-12)
