"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``pin_*`` function takes a loaded oracle and raises ``AssertionError`` when the
oracle disagrees with an independent fact: a published known-answer vector, a value the
pages print, a library routine (scipy softmax), a textbook sort-based sampler written
here in numpy, a closed form, or an exact law checked by Monte-Carlo.  None of them
re-types the oracle's own code.  The same functions run against the planted mutants of
the oracle (negative controls): every mutant must fail at least one pin.
"""
from __future__ import annotations

import math
import os

import numpy as np
from scipy import special, stats

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CHI2_P_MIN = 1e-3


# ---------------------------------------------------------------------------------------
# independent helpers (numpy / scipy only)
# ---------------------------------------------------------------------------------------

def softmax_T(l, T):
    return special.softmax(np.asarray(l, dtype=np.float64) / T)


def textbook_topk_topp(l, T, K, P):
    """Sort-based sampler on a tie-free row: keep the K most likely tokens, then the
    smallest most-likely prefix holding at least P of the renormalised mass."""
    l = np.asarray(l, dtype=np.float64)
    V = l.shape[0]
    order = np.argsort(-l, kind="stable")
    keep = np.zeros(V, dtype=bool)
    n = K if 0 < K < V else V
    keep[order[:n]] = True
    if P < 1.0:
        p = softmax_T(l[order[:n]], T)
        c = np.cumsum(p)
        m = int(np.searchsorted(c, P * c[-1], side="left")) + 1
        keep[:] = False
        keep[order[:min(m, n)]] = True
    out = np.zeros(V)
    out[keep] = softmax_T(l[keep], T)
    return out


def expected_accept_length(alphas):
    """Closed form of the expected committed tokens per verify step with fresh drafts:
    1 + sum over depths d of the probability that the first d drafts are all accepted."""
    total, run = 1.0, 1.0
    for a in alphas:
        run *= a
        total += run
    return total


def chi2_pvalue(counts, probs):
    counts = np.asarray(counts, dtype=np.float64)
    probs = np.asarray(probs, dtype=np.float64)
    n = counts.sum()
    mask = probs > 0
    assert np.all(counts[~mask] == 0), "mass observed on a zero-probability outcome"
    exp = probs[mask] / probs[mask].sum() * n
    return stats.chisquare(counts[mask], exp).pvalue


def f32(x):
    return np.asarray(x, dtype=np.float32)


def _rows(rng, n, V, sigma=2.0):
    return rng.normal(0.0, sigma, size=(n, V))


def read_golden_table(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


def _parse_num(tok):
    if tok.startswith("ln"):
        return math.log(float(tok[2:]))
    return float(tok)


# ---------------------------------------------------------------------------------------
# random streams
# ---------------------------------------------------------------------------------------

def pin_philox_kat(o):
    for line in read_golden_table("philox4x32_10_kat.txt"):
        v = [int(t, 16) for t in line.split()]
        out = o.philox(v[0:4], v[4:6])
        assert [int(x) for x in out] == v[6:10], f"Philox KAT mismatch for {line}"


def pin_stream_layout(o):
    """The accept and Gumbel uniforms are the documented words of the documented counters."""
    seed = (0x1234ABCD << 32) | 0x9E3779B9
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for b, i, off in [(0, 0, 0), (5, 3, 7), (1023, 6, 99), (7, 1, 2**32 - 1)]:
        w = o.philox([i >> 2, b, 0, off], key)[i & 3]
        assert o.accept_uniform(seed, b, i, off) == float(int(w) >> 8) * 2.0 ** -24
    for tag in (1, 2):
        for b, j, x, off in [(0, 0, 0, 0), (3, 2, 157183, 5), (255, 4, 4097, 99)]:
            w = o.philox([x >> 2, b, (tag << 24) | j, off], key)[x & 3]
            assert o.gumbel_uniform(seed, tag, b, j, x, off) == ((int(w) >> 9) + 0.5) * 2.0 ** -23


def pin_uniform_distribution(o):
    us = np.array([o.accept_uniform(0, b, i, 0) for b in range(2000) for i in range(4)])
    assert us.min() >= 0.0 and us.max() < 1.0
    assert stats.kstest(us, "uniform").pvalue > CHI2_P_MIN
    gs = np.array([o.gumbel_uniform(3, 1, 2, 1, x, 11) for x in range(8000)])
    assert gs.min() > 0.0 and gs.max() < 1.0
    assert stats.kstest(gs, "uniform").pvalue > CHI2_P_MIN


# ---------------------------------------------------------------------------------------
# the sampler distribution
# ---------------------------------------------------------------------------------------

def pin_softmax_temperature(o):
    rng = np.random.default_rng(11)
    for l in _rows(rng, 6, 300, 3.0):
        for T in (0.37, 1.0, 1.9):
            p, info = o.row_probs(l, T)
            np.testing.assert_allclose(p, softmax_T(l, T), rtol=0, atol=1e-14)
            assert info["argmax"] == int(np.argmax(l))


def pin_topk_textbook(o):
    rng = np.random.default_rng(12)
    for l in _rows(rng, 6, 500):
        for K in (1, 2, 17, 50, 499):
            p, _ = o.row_probs(l, 0.8, K, 1.0)
            np.testing.assert_allclose(p, textbook_topk_topp(l, 0.8, K, 1.0), rtol=0, atol=1e-14)


def pin_topp_textbook(o):
    rng = np.random.default_rng(13)
    for l in _rows(rng, 6, 500):
        for P in (0.05, 0.5, 0.9, 0.95, 0.999):
            p, _ = o.row_probs(l, 1.3, 0, P)
            np.testing.assert_allclose(p, textbook_topk_topp(l, 1.3, 0, P), rtol=0, atol=1e-14)


def pin_topk_then_topp_textbook(o):
    rng = np.random.default_rng(14)
    for l in _rows(rng, 6, 400, 1.5):
        for K, P in ((50, 0.95), (10, 0.5), (200, 0.9)):
            p, _ = o.row_probs(l, 0.7, K, P)
            np.testing.assert_allclose(p, textbook_topk_topp(l, 0.7, K, P), rtol=0, atol=1e-14)


def pin_golden_tie_cases(o):
    for line in read_golden_table("sampler_tie_cases.txt"):
        name, logits, T, K, P, want = [s.strip() for s in line.split("|")]
        l = [_parse_num(t) for t in logits.split()]
        p, _ = o.row_probs(l, float(T), int(K), float(P))
        np.testing.assert_allclose(p, [float(t) for t in want.split()], rtol=0, atol=1e-12, err_msg=name)


def pin_off_switches(o):
    rng = np.random.default_rng(15)
    for l in _rows(rng, 4, 64):
        base, _ = o.row_probs(l, 1.1)
        for K, P in ((0, 1.0), (64, 1.0), (1000, 1.0), (0, 1.5), (64, float("inf"))):
            p, _ = o.row_probs(l, 1.1, K, P)
            np.testing.assert_array_equal(p, base)
        p1, _ = o.row_probs(l, 1.1, 1, 1.0)   # top-1 on a tie-free row is the greedy one-hot
        g, _ = o.row_probs(l, 0.0)
        np.testing.assert_array_equal(p1, g)
        assert g[int(np.argmax(l))] == 1.0


def pin_topp_margin_golden(o):
    """The top-p decision distances against hand-worked rows (tests/golden/topp_margin_cases.txt): at the
    chosen value, at the next larger distinct value, after top-k renormalisation, with ties kept whole,
    under a temperature, and off."""
    for line in read_golden_table("topp_margin_cases.txt"):
        name, logits, T, K, P, at, prev = [t.strip() for t in line.split("|")]
        l = [_parse_num(t) for t in logits.split()]
        _, info = o.row_probs(l, float(T), int(K), float(P))
        want = {"topp_at": float(at), "topp_prev": float(prev)}
        want["topp_margin"] = min(want.values())
        for key, w in want.items():
            g = info[key]
            if math.isinf(w):
                assert math.isinf(g), (name, key, g)
            else:
                assert abs(g - w) <= 1e-12, (name, key, g, w)


# ---------------------------------------------------------------------------------------
# verify step
# ---------------------------------------------------------------------------------------

def _tiny_case(rng, B, k, V, sigma_t=1.0, sigma_n=0.7):
    t = rng.normal(0.0, sigma_t, size=(k + 1, V)).astype(np.float32)
    d = (t[:k] + rng.normal(0.0, sigma_n, size=(k, V))).astype(np.float32)
    return (np.broadcast_to(t, (B, k + 1, V)).copy(), np.broadcast_to(d, (B, k, V)).copy())


def _fresh_drafts(o, draft, T, K, P):
    """Draw every batch row's drafts from its own plain-sampler stream (independent trials)."""
    B, k, V = draft.shape
    tok, _, _ = o.sample(draft.reshape(B * k, V), np.repeat(T, k), np.repeat(K, k), np.repeat(P, k),
                         np.repeat(np.arange(B), k), np.tile(np.arange(k), B), seed=7, offset=3)
    return tok.reshape(B, k)


def _params(B, T=1.0, K=0, P=1.0):
    return f32(np.full(B, T)), np.full(B, K, dtype=np.int32), f32(np.full(B, P))


def pin_alpha_identities(o):
    rng = np.random.default_rng(21)
    B, k, V = 3, 3, 64
    t, d = _tiny_case(rng, B, k, V)
    for T, K, P in ((1.0, 0, 1.0), (0.6, 10, 1.0), (1.3, 0, 0.8), (0.9, 20, 0.9)):
        Ta, Ka, Pa = _params(B, T, K, P)
        drafts = np.zeros((B, k), dtype=np.int32)
        r = o.spec_verify(t, d, drafts, Ta, Ka, Pa, seed=1)
        for i in range(k):
            p = textbook_topk_topp(t[0, i].astype(np.float64), T, K, P)
            q = textbook_topk_topp(d[0, i].astype(np.float64), T, K, P)
            tv_alpha = 1.0 - 0.5 * np.abs(p - q).sum()   # total-variation identity
            np.testing.assert_allclose(r.alpha[:, i], tv_alpha, atol=1e-12)
    # identical rows: alpha = 1; disjoint one-hot supports (top-1, different argmax): alpha = 0
    Ta, Ka, Pa = _params(B, 1.0, 0, 1.0)
    r = o.spec_verify(t, t[:, :k].copy(), np.zeros((B, k), np.int32), Ta, Ka, Pa)
    np.testing.assert_allclose(r.alpha, 1.0, atol=1e-12)
    t2 = np.zeros((1, 2, 8), np.float32)
    d2 = np.zeros((1, 1, 8), np.float32)
    t2[0, 0, 2] = 5.0
    d2[0, 0, 6] = 5.0
    r = o.spec_verify(t2, d2, np.array([[6]]), *_params(1, 1.0, 1, 1.0))
    assert r.alpha[0, 0] == 0.0
    assert r.tokens[0, 0] == 2 and r.accept_len[0] == 1   # rejected; residual is the target one-hot
    assert np.all((r.alpha >= 0) & (r.alpha <= 1))


def pin_identity_accepts_all(o):
    """Bit-identical draft and target rows: every draft is accepted (p/q = 1 > u)."""
    rng = np.random.default_rng(22)
    B, k, V = 200, 3, 50
    t, _ = _tiny_case(rng, B, k, V)
    for T, K, P in ((1.0, 0, 1.0), (0.7, 5, 0.9)):
        Ta, Ka, Pa = _params(B, T, K, P)
        d = t[:, :k].copy()
        drafts = _fresh_drafts(o, d, Ta, Ka, Pa)
        r = o.spec_verify(t, d, drafts, Ta, Ka, Pa, seed=5)
        assert np.all(r.accept_len == k + 1)
        np.testing.assert_array_equal(r.tokens[:, :k], drafts)


def pin_greedy_chain(o):
    """Greedy (T = 0): accept while the draft is the target argmax; the extra token is the
    target argmax at the first mismatch (lowest index on exact ties)."""
    rng = np.random.default_rng(23)
    B, k, V = 64, 3, 40
    t = rng.integers(-4, 5, size=(B, k + 1, V)).astype(np.float32)   # many exact ties
    d = rng.integers(-4, 5, size=(B, k, V)).astype(np.float32)
    drafts = rng.integers(0, V, size=(B, k)).astype(np.int32)
    am = np.argmax(t, axis=2)   # numpy argmax returns the first maximum
    hit = rng.random((B, k)) < 0.6
    drafts = np.where(hit, am[:, :k], drafts).astype(np.int32)
    r = o.spec_verify(t, d, drafts, *_params(B, 0.0, 7, 0.5))
    for b in range(B):
        n = 0
        while n < k and drafts[b, n] == am[b, n]:
            n += 1
        want = list(drafts[b, :n]) + [am[b, n]] + [-1] * (k - n)
        assert list(r.tokens[b]) == want, (b, list(r.tokens[b]), want)
        assert r.accept_len[b] == n + 1
        np.testing.assert_array_equal(r.logprobs[b], 0.0)
        np.testing.assert_array_equal(r.alpha[b], (am[b, :k] == np.argmax(d[b], axis=1)).astype(float))


def pin_marginal_k1(o):
    """Committed first token ~ p_0 (chi-square over 1e5 independent trials, V = 8)."""
    rng = np.random.default_rng(31)
    B, k, V = 100_000, 1, 8
    t, d = _tiny_case(rng, B, k, V, 1.0, 0.9)
    T, K, P = _params(B, 1.0)
    r = o.spec_verify(t, d, _fresh_drafts(o, d, T, K, P), T, K, P, seed=9, offset=1)
    counts = np.bincount(r.tokens[:, 0], minlength=V)
    assert chi2_pvalue(counts, softmax_T(t[0, 0], 1.0)) > CHI2_P_MIN


def pin_marginal_k2(o):
    """k = 2, truncated sampler: token 0 ~ p_0; token 1 given that draft 0 was accepted ~ p_1."""
    rng = np.random.default_rng(32)
    B, k, V = 100_000, 2, 16
    t, d = _tiny_case(rng, B, k, V, 1.2, 0.8)
    T, K, P = _params(B, 0.9, 12, 0.95)
    r = o.spec_verify(t, d, _fresh_drafts(o, d, T, K, P), T, K, P, seed=4, offset=2)
    p0 = textbook_topk_topp(t[0, 0].astype(np.float64), 0.9, 12, 0.95)
    p1 = textbook_topk_topp(t[0, 1].astype(np.float64), 0.9, 12, 0.95)
    assert chi2_pvalue(np.bincount(r.tokens[:, 0], minlength=V), p0) > CHI2_P_MIN
    sel = r.accept_len >= 2
    assert chi2_pvalue(np.bincount(r.tokens[sel, 1], minlength=V), p1) > CHI2_P_MIN


def pin_marginal_bonus(o):
    """With drafts equal to targets except the last target row, every draft is accepted and
    the bonus token ~ p_k."""
    rng = np.random.default_rng(33)
    B, k, V = 100_000, 2, 8
    t, _ = _tiny_case(rng, B, k, V, 1.0)
    d = t[:, :k].copy()
    T, K, P = _params(B, 1.0)
    r = o.spec_verify(t, d, _fresh_drafts(o, d, T, K, P), T, K, P, seed=6)
    assert np.all(r.accept_len == k + 1)
    assert chi2_pvalue(np.bincount(r.tokens[:, k], minlength=V), softmax_T(t[0, k], 1.0)) > CHI2_P_MIN


def pin_joint_law_v3(o):
    """V = 3, k = 2, fixed drafts: the law of (accepted count n, extra token y) is
    P(n=j, y) = prod_{i<j} a_i * (1 - a_j) * r_j(y) for j < k and prod a_i * p_k(y) for j = k,
    with a_i = min(1, p_i(x_i)/q_i(x_i)) and r_j the normalised positive part of p_j - q_j."""
    B, k, V = 100_000, 2, 3
    tl = np.array([[0.2, 1.0, -0.5], [0.9, -0.3, 0.4], [-0.2, 0.6, 0.1]], np.float32)
    dl = np.array([[1.1, 0.1, -0.2], [0.1, 0.5, 0.3]], np.float32)
    x = np.array([0, 1], np.int32)
    t = np.broadcast_to(tl, (B, k + 1, V)).copy()
    d = np.broadcast_to(dl, (B, k, V)).copy()
    r = o.spec_verify(t, d, np.broadcast_to(x, (B, k)).copy(), *_params(B, 1.0), seed=12, offset=4)
    p = [softmax_T(tl[i], 1.0) for i in range(k + 1)]
    q = [softmax_T(dl[i], 1.0) for i in range(k)]
    a = [min(1.0, p[i][x[i]] / q[i][x[i]]) for i in range(k)]
    law = np.zeros((k + 1, V))
    run = 1.0
    for j in range(k):
        res = np.maximum(p[j] - q[j], 0.0)
        law[j] = run * (1.0 - a[j]) * res / res.sum()
        run *= a[j]
    law[k] = run * p[k]
    n = r.accept_len - 1
    y = r.tokens[np.arange(B), n]
    counts = np.zeros((k + 1, V))
    np.add.at(counts, (n, y), 1)
    assert chi2_pvalue(counts.ravel(), law.ravel()) > CHI2_P_MIN


def pin_expected_accept_length(o):
    """Mean committed tokens with fresh drafts = 1 + a_0 + a_0 a_1 (closed form from the alphas)."""
    rng = np.random.default_rng(41)
    B, k, V = 100_000, 2, 12
    t, d = _tiny_case(rng, B, k, V, 1.0, 0.6)
    T, K, P = _params(B, 1.0)
    r = o.spec_verify(t, d, _fresh_drafts(o, d, T, K, P), T, K, P, seed=3, offset=8)
    alphas = [np.minimum(softmax_T(t[0, i], 1.0), softmax_T(d[0, i], 1.0)).sum() for i in range(k)]
    want = expected_accept_length(alphas)
    se = r.accept_len.std() / math.sqrt(B)
    assert abs(r.accept_len.mean() - want) < 4.5 * se, (r.accept_len.mean(), want, se)


def pin_expected_accept_length_given_drafts(o):
    """Fixed drafts, randomness over u only: E[accept_len] = 1 + sum_d prod_{j<d} min(1, p_j/q_j)."""
    rng = np.random.default_rng(42)
    B, k, V = 100_000, 3, 10
    t, d = _tiny_case(rng, B, k, V, 1.0, 0.8)
    x = np.array([1, 4, 7], np.int32)
    r = o.spec_verify(t, d, np.broadcast_to(x, (B, k)).copy(), *_params(B, 1.0), seed=17, offset=5)
    a = [min(1.0, softmax_T(t[0, i], 1.0)[x[i]] / softmax_T(d[0, i], 1.0)[x[i]]) for i in range(k)]
    want = expected_accept_length(a)
    se = r.accept_len.std() / math.sqrt(B)
    assert abs(r.accept_len.mean() - want) < 4.5 * se, (r.accept_len.mean(), want, se)


def pin_pages_accept_length(o):
    """The closed form reproduces the pages' printed expected accept lengths from their alphas."""
    vals = dict(line.split() for line in read_golden_table("accept_length_table.txt"))
    a1, a2 = float(vals["alpha_depth1"]), float(vals["alpha_depth2_given_1"])
    assert round(expected_accept_length([a1]), 2) == float(vals["expected_accept_length_k1"])
    assert round(expected_accept_length([a1, a2]), 2) == float(vals["expected_accept_length_k2"])


def pin_logprobs(o):
    """Reported logprobs are ln p_i(token_i) under the processed target distribution."""
    rng = np.random.default_rng(51)
    B, k, V = 50, 2, 30
    t, d = _tiny_case(rng, B, k, V, 1.5, 0.9)
    for T, K, P in ((1.0, 0, 1.0), (0.8, 10, 0.9)):
        Ta, Ka, Pa = _params(B, T, K, P)
        r = o.spec_verify(t, d, _fresh_drafts(o, d, Ta, Ka, Pa), Ta, Ka, Pa, seed=2)
        with np.errstate(divide="ignore"):
            _check_logprobs(r, t, B, k, T, K, P)


def _check_logprobs(r, t, B, k, T, K, P):
    for b in range(B):
        for i in range(k + 1):
            if i < r.accept_len[b]:
                p = textbook_topk_topp(t[b, i].astype(np.float64), T, K, P)
                np.testing.assert_allclose(r.logprobs[b, i], np.log(p[r.tokens[b, i]]), atol=1e-12)
            else:
                assert r.tokens[b, i] == -1 and r.logprobs[b, i] == 0.0


def pin_raw_logprobs(o):
    """Raw logprobs are ln softmax of the unprocessed target logits at each committed token, whatever the
    sampling parameters: closed forms (a uniform row gives -ln V; a row with one raised entry gives
    a - ln(e^a + (V-1))), scipy's log_softmax on random rows at T != 1 with truncation, equality with the
    processed logprobs when T = 1 without truncation, NaN for sentinel rows and 0 after the committed slots."""
    V = 64
    flat = np.zeros((1, 2, V), np.float32)
    got = o.raw_logprobs(flat, np.array([[3, 9]]), np.array([2]), temperature=np.array([0.5], np.float32))
    np.testing.assert_allclose(got, [[-math.log(V), -math.log(V)]], rtol=0, atol=1e-15)
    a = 2.5
    two = np.zeros((1, 2, V), np.float32)
    two[0, :, 7] = a
    got = o.raw_logprobs(two, np.array([[7, 8]]), np.array([2]), temperature=np.array([2.0], np.float32))
    z = math.exp(a) + (V - 1)
    np.testing.assert_allclose(got, [[a - math.log(z), -math.log(z)]], rtol=0, atol=1e-14)
    got = o.raw_logprobs(two, np.array([[7, -1]]), np.array([1]))
    assert got[0, 1] == 0.0
    got = o.raw_logprobs(two, np.array([[-1, -1]]), np.array([0]))
    assert np.all(np.isnan(got))
    rng = np.random.default_rng(52)
    B, k, V = 40, 2, 30
    t, d = _tiny_case(rng, B, k, V, 1.5, 0.9)
    for T, K, P in ((1.0, 0, 1.0), (0.7, 8, 0.85)):
        Ta, Ka, Pa = _params(B, T, K, P)
        r = o.spec_verify(t, d, _fresh_drafts(o, d, Ta, Ka, Pa), Ta, Ka, Pa, seed=4)
        raw = o.raw_logprobs(t, r.tokens, r.accept_len, temperature=Ta)
        for b in range(B):
            for i in range(k + 1):
                if i < r.accept_len[b]:
                    ref = special.log_softmax(t[b, i].astype(np.float64))[r.tokens[b, i]]
                    np.testing.assert_allclose(raw[b, i], ref, rtol=0, atol=1e-12)
                    if T == 1.0 and K == 0 and P == 1.0:
                        np.testing.assert_allclose(raw[b, i], r.logprobs[b, i], rtol=0, atol=1e-12)
                else:
                    assert raw[b, i] == 0.0


def pin_residual_mass(o):
    """At a rejection, the residual mass equals 1 - alpha at that position."""
    rng = np.random.default_rng(52)
    B, k, V = 400, 2, 20
    t, d = _tiny_case(rng, B, k, V, 1.0, 1.0)
    T, K, P = _params(B, 1.0)
    r = o.spec_verify(t, d, _fresh_drafts(o, d, T, K, P), T, K, P, seed=8)
    n = r.accept_len - 1
    rej = n < k
    assert rej.any()
    np.testing.assert_allclose(r.residual_mass[rej], 1.0 - r.alpha[np.arange(B)[rej], n[rej]], atol=1e-12)


def pin_invalid_rows(o):
    """Rows with unusable inputs come back as sentinels; the other rows are untouched."""
    rng = np.random.default_rng(53)
    B, k, V = 8, 2, 16
    t, d = _tiny_case(rng, B, k, V)
    T, K, P = _params(B, 1.0)
    drafts = np.zeros((B, k), np.int32)
    t[1, 0, 3] = np.nan
    d[2, 1, 5] = np.inf
    t[3, 2, :] = -np.inf
    T[4] = -1.0
    K[5] = -3
    P[6] = 0.0
    drafts[7, 1] = V
    r = o.spec_verify(t, d, drafts, T, K, P)
    bad = [1, 2, 3, 4, 5, 6, 7]
    assert np.all(r.accept_len[bad] == 0) and np.all(r.tokens[bad] == -1)
    assert np.all(np.isnan(r.logprobs[bad])) and np.all(np.isnan(r.alpha[bad]))
    assert r.accept_len[0] >= 1 and np.all(np.isfinite(r.alpha[0]))
    # -inf entries are legal (probability zero)
    t2, d2 = _tiny_case(rng, 1, 1, 16)
    t2[0, :, ::2] = -np.inf
    r2 = o.spec_verify(t2, d2, np.array([[1]]), *_params(1, 1.0))
    assert r2.accept_len[0] >= 1 and r2.tokens[0, r2.accept_len[0] - 1] % 2 == 1


def pin_determinism(o):
    rng = np.random.default_rng(54)
    B, k, V = 300, 2, 32
    t, d = _tiny_case(rng, B, k, V)
    T, K, P = _params(B, 1.0)
    drafts = _fresh_drafts(o, d, T, K, P)
    r1 = o.spec_verify(t, d, drafts, T, K, P, seed=77, offset=4, num_threads=1)
    r2 = o.spec_verify(t, d, drafts, T, K, P, seed=77, offset=4, num_threads=5)
    np.testing.assert_array_equal(r1.tokens, r2.tokens)
    np.testing.assert_array_equal(r1.logprobs, r2.logprobs)
    r3 = o.spec_verify(t, d, drafts, T, K, P, seed=77, offset=5)
    assert not np.array_equal(r1.tokens, r3.tokens)


def pin_plain_sampler_marginal(o):
    """The plain sampler draws from the processed distribution (it produces the drafts)."""
    rng = np.random.default_rng(61)
    R, V = 100_000, 10
    l = rng.normal(0.0, 1.3, size=V).astype(np.float32)
    T, K, P = 0.8, 7, 0.9
    tok, lp, _ = o.sample(np.broadcast_to(l, (R, V)).copy(), np.full(R, T), np.full(R, K), np.full(R, P),
                          np.arange(R), np.zeros(R), seed=5, offset=6)
    p = textbook_topk_topp(l.astype(np.float64), T, K, P)
    assert chi2_pvalue(np.bincount(tok, minlength=V), p) > CHI2_P_MIN
    np.testing.assert_allclose(lp, np.log(p[tok]), atol=1e-12)


# ---------------------------------------------------------------------------------------
# commit step
# ---------------------------------------------------------------------------------------

class _ToyHybrid:
    """A toy hybrid model in exact integer arithmetic, L layers deep.  Each layer keeps a recurrent
    state (a wrapping multiply-add of the fed token's embedding, so it depends on the order of every
    token fed so far), a conv window holding the last W-1 fed embeddings, and a key/value list with one
    entry per fed token.  ``step`` feeds one token, as plain decode does; ``verify`` feeds k+1 tokens from a
    committed state and keeps the state after every position, as a verify forward does."""

    def __init__(self, rng, L, D, rdtype, W, C, vocab=1000):
        self.L, self.D, self.W, self.C = L, D, W, C
        self.rdtype = rdtype
        self.mult = (rng.integers(0, 1 << 15, size=L) * 2 + 1).astype(rdtype)
        self.emb = rng.integers(0, 1 << 16, size=(vocab, max(D, C)), dtype=np.int64)

    def e(self, x, l, n, dtype):
        return ((self.emb[x, :n] + 977 * l) % (1 << 16)).astype(dtype)

    def step(self, rec, conv, kv, x):
        """rec [L, D], conv [L, W-1, C], kv list; returns the state after feeding token x."""
        rec = rec.copy()
        conv = conv.copy()
        for l in range(self.L):
            rec[l] = rec[l] * self.mult[l] + self.e(x, l, self.D, self.rdtype)
            conv[l] = np.concatenate([conv[l, 1:], self.e(x, l, self.C, np.uint16)[None, :]], axis=0)
        return rec, conv, kv + [x]

    def verify(self, rec, conv, fed):
        recs, convs = [], []
        for x in fed:
            rec, conv, _ = self.step(rec, conv, [], x)
            recs.append(rec)
            convs.append(conv)
        return np.stack(recs, axis=1), np.stack(convs, axis=1)   # [L, k+1, ...]


def _commit_rounds(o, L, D, rdtype, W, C, B, k, rounds, seed):
    rng = np.random.default_rng(seed)
    toy = _ToyHybrid(rng, L, D, rdtype, W, C)
    num_slots = B + 3
    slot = rng.permutation(num_slots)[:B].astype(np.int32)
    rec_cache = rng.integers(0, 250, size=(L, num_slots, D)).astype(rdtype)
    conv_cache = rng.integers(0, 60000, size=(L, num_slots, W - 1, C)).astype(np.uint16)
    free = np.setdiff1d(np.arange(num_slots), slot)
    free_rec, free_conv = rec_cache[:, free].copy(), conv_cache[:, free].copy()
    # sequential-decode reference per row
    seq = [(rec_cache[:, slot[b]].copy(), conv_cache[:, slot[b]].copy(), []) for b in range(B)]
    kv = np.full((B, 4 * rounds * (k + 1)), -1, np.int64)   # verify writes every fed position
    seq_len = np.zeros(B, np.int32)
    last = rng.integers(0, 1000, size=B)
    for r in range(rounds):
        fed = np.concatenate([last[:, None], rng.integers(0, 1000, size=(B, k))], axis=1)
        vrec = np.empty((L, B, k + 1, D), rdtype)
        vconv = np.empty((L, B, k + 1, W - 1, C), np.uint16)
        for b in range(B):
            vrec[:, b], vconv[:, b] = toy.verify(rec_cache[:, slot[b]], conv_cache[:, slot[b]], fed[b])
            kv[b, seq_len[b]:seq_len[b] + k + 1] = fed[b]
        acc = rng.integers(1, k + 2, size=B).astype(np.int32)
        acc[0] = k + 1                            # a full accept and a minimal one every round
        acc[1 % B] = 1
        bad_slot = np.zeros(B, bool)
        if r == 1:
            acc[2 % B] = 0                        # sentinel row: the step is discarded
            acc[3 % B] = k + 2
        if r == 2:
            bad_slot[4 % B] = True
        slot_arg = np.where(bad_slot, num_slots, slot).astype(np.int32)
        status = o.commit([(vrec, rec_cache), (vconv, conv_cache)], slot_arg, acc, seq_len)
        for b in range(B):
            ok = 1 <= acc[b] <= k + 1 and not bad_slot[b]
            assert status[b] == (0 if ok else (1 if not 1 <= acc[b] <= k + 1 else 2))
            if ok:
                st = seq[b]
                for x in fed[b, :acc[b]]:
                    st = toy.step(*st, x)
                seq[b] = st
                last[b] = rng.integers(0, 1000)    # the token drawn at this step, fed next time
            rec_b, conv_b, kv_b = seq[b]
            np.testing.assert_array_equal(rec_cache[:, slot[b]], rec_b)
            np.testing.assert_array_equal(conv_cache[:, slot[b]], conv_b)
            assert seq_len[b] == len(kv_b)
            np.testing.assert_array_equal(kv[b, :seq_len[b]], kv_b)
        np.testing.assert_array_equal(rec_cache[:, free], free_rec)
        np.testing.assert_array_equal(conv_cache[:, free], free_conv)


def pin_commit_matches_sequential_decode(o):
    """After full and partial commits the recurrent state, the conv window and the key/value prefix of
    every row equal those of decoding the committed tokens one at a time (the pages check exactly this on
    their model).  Four rounds per case on a toy integer model with several layers, slots permuted in a
    larger pool, rows that must be left alone (accept length 0 or k+2, slot out of range), and state rows
    of 1, 3 and 68 bytes.  Slots no row maps to keep their bytes."""
    _commit_rounds(o, L=3, D=1, rdtype=np.uint8, W=4, C=1, B=6, k=2, rounds=4, seed=70)
    _commit_rounds(o, L=2, D=3, rdtype=np.uint8, W=2, C=3, B=5, k=1, rounds=4, seed=71)
    _commit_rounds(o, L=4, D=17, rdtype=np.uint32, W=4, C=5, B=7, k=4, rounds=4, seed=72)


def _commit_slot_rounds(o, L, D, rdtype, W, C, B, k, rounds, seed):
    rng = np.random.default_rng(seed)
    toy = _ToyHybrid(rng, L, D, rdtype, W, C)
    P = B * (k + 2) + 5                                   # pool: a committed slot and k+1 scratch slots per row
    perm = rng.permutation(P).astype(np.int32)
    state_slot = perm[:B].copy()
    pos_slot = perm[B:B * (k + 2)].reshape(B, k + 1).copy()
    spare = perm[B * (k + 2):]
    pool_rec = rng.integers(0, 250, size=(L, P, D)).astype(rdtype)
    pool_conv = rng.integers(0, 60000, size=(L, P, W - 1, C)).astype(np.uint16)
    spare_rec, spare_conv = pool_rec[:, spare].copy(), pool_conv[:, spare].copy()
    seq = [(pool_rec[:, state_slot[b]].copy(), pool_conv[:, state_slot[b]].copy(), []) for b in range(B)]
    seq_len = np.zeros(B, np.int32)
    last = rng.integers(0, 1000, size=B)
    for r in range(rounds):
        fed = np.concatenate([last[:, None], rng.integers(0, 1000, size=(B, k))], axis=1)
        for b in range(B):                                # verify: read the committed slot, write scratch slots
            vr, vc = toy.verify(pool_rec[:, state_slot[b]], pool_conv[:, state_slot[b]], fed[b])
            pool_rec[:, pos_slot[b]] = vr
            pool_conv[:, pos_slot[b]] = vc
        acc = rng.integers(1, k + 2, size=B).astype(np.int32)
        acc[0] = k + 1
        acc[1 % B] = 1
        if r == 1:
            acc[2 % B] = 0
        before = np.sort(np.concatenate([state_slot, pos_slot.ravel()]))
        status = o.commit_slots(state_slot, pos_slot, acc, P, seq_len)
        np.testing.assert_array_equal(np.sort(np.concatenate([state_slot, pos_slot.ravel()])), before)
        for b in range(B):
            assert status[b] == (0 if 1 <= acc[b] <= k + 1 else 1)
            if status[b] == 0:
                st = seq[b]
                for x in fed[b, :acc[b]]:
                    st = toy.step(*st, x)
                seq[b] = st
                last[b] = rng.integers(0, 1000)
            np.testing.assert_array_equal(pool_rec[:, state_slot[b]], seq[b][0])
            np.testing.assert_array_equal(pool_conv[:, state_slot[b]], seq[b][1])
            assert seq_len[b] == len(seq[b][2])
        np.testing.assert_array_equal(pool_rec[:, spare], spare_rec)
        np.testing.assert_array_equal(pool_conv[:, spare], spare_conv)


def pin_commit_slots_matches_sequential_decode(o):
    """Commit by slot numbers over a pool where verify writes each position's state to a scratch slot of
    its row: after full and partial commits the state in each row's committed slot equals one-token-at-a-
    time decoding, the committed and scratch slots stay a permutation of the pool (no slot lost, none
    shared), rows with an unusable accept length keep their slots, and a slot outside the pool is refused."""
    _commit_slot_rounds(o, L=3, D=1, rdtype=np.uint8, W=4, C=1, B=6, k=2, rounds=4, seed=80)
    _commit_slot_rounds(o, L=2, D=9, rdtype=np.uint32, W=3, C=4, B=5, k=4, rounds=4, seed=81)
    ss = np.array([0, 7], np.int32)
    ps = np.array([[1, 2], [3, 4]], np.int32)
    st = o.commit_slots(ss, ps, [2, 2], 7)
    assert list(st) == [0, 2] and list(ss) == [2, 7] and ps.tolist() == [[1, 0], [3, 4]]


# ---------------------------------------------------------------------------------------
# tree verification
# ---------------------------------------------------------------------------------------

def _one_hot_drafts(B, k, V, drafts):
    """Draft logit rows whose sampler distribution is one-hot at the draft token: 0 there, -inf elsewhere."""
    d = np.full((B, k, V), -np.inf, dtype=np.float32)
    for b in range(B):
        for i in range(k):
            d[b, i, drafts[b, i]] = 0.0
    return d


def pin_tree_chain_equals_chain_verify(o):
    """A tree in which every node has one child is chain verification whose draft distributions are one-hot
    at the draft tokens: same committed tokens, accept lengths and logprobs, row for row, across greedy,
    untruncated, top-k and top-p rows; the path is nodes 1..n."""
    rng = np.random.default_rng(90)
    B, k, V = 600, 3, 24
    t = rng.normal(0.0, 1.3, size=(B, k + 1, V)).astype(np.float32)
    drafts = np.zeros((B, k), np.int32)
    for b in range(B):   # mostly likely tokens, so that some rows accept deep
        for i in range(k):
            drafts[b, i] = int(np.argmax(t[b, i])) if rng.random() < 0.7 else int(rng.integers(0, V))
    T = f32(rng.choice([0.0, 0.7, 1.0, 1.4], size=B))
    K = rng.choice([0, 3, 8], size=B).astype(np.int32)
    P = f32(rng.choice([1.0, 0.9, 0.6], size=B))
    c = o.spec_verify(t, _one_hot_drafts(B, k, V, drafts), drafts, T, K, P, seed=11, offset=2)
    par = np.tile(np.arange(-1, k, dtype=np.int32), (B, 1))
    par[:, 0] = 0
    ntok = np.concatenate([np.zeros((B, 1), np.int32), drafts], axis=1)
    r = o.tree_verify(t, par, ntok, T, K, P, seed=11, offset=2)
    np.testing.assert_array_equal(r.accept_len, c.accept_len)
    np.testing.assert_array_equal(r.tokens, c.tokens)
    np.testing.assert_allclose(r.logprobs, c.logprobs, rtol=0, atol=1e-12)
    for b in range(B):
        n = c.accept_len[b] - 1
        assert list(r.path[b, :n]) == list(range(1, n + 1)) and np.all(r.path[b, n:] == -1)
    assert (c.accept_len == k + 1).sum() > 20 and (c.accept_len == 1).sum() > 20


def _tree_law(p_rows, parent, tok, V):
    """Exact law of the committed sequence for one tree: {token tuple: probability}.  p_rows[i] is the
    sampler distribution after node i; a drawn token that matches a child moves the walk to that child."""
    N = len(parent)
    children = {u: [c for c in range(1, N) if parent[c] == u] for u in range(N)}
    law = {}

    def walk(u, prefix, prob):
        for y in range(V):
            py = p_rows[u][y]
            if py == 0.0:
                continue
            nxt = [c for c in children[u] if tok[c] == y]
            if nxt and children[u]:
                walk(nxt[0], prefix + (y,), prob * py)
            else:
                law[prefix + (y,)] = law.get(prefix + (y,), 0.0) + prob * py
    walk(0, (), 1.0)
    return law


def pin_tree_joint_law(o):
    """The committed sequence of tree verification follows the target sampler exactly: chi-square of the
    whole sequence law over 1e5 independent rows of one tree (with a top-k that removes tokens, so some
    children have probability 0), against the law enumerated from textbook sampler distributions; the mean
    accept length matches its closed form 1 + sum over non-root nodes of the product of p along the edges."""
    rng = np.random.default_rng(91)
    V, R = 6, 100_000
    parent = [0, 0, 0, 0, 1, 4, 0]
    tok = [0, 2, 0, 5, 3, 1, 4]
    N = len(parent)
    parent[6] = 2
    l = rng.normal(0.0, 1.2, size=(N, V)).astype(np.float32)
    l[0, 2] += 1.5
    l[1, 3] += 1.5
    T, K, P = 0.8, 5, 1.0
    p_rows = [textbook_topk_topp(l[i].astype(np.float64), T, K, P) for i in range(N)]
    law = _tree_law(p_rows, parent, tok, V)
    r = o.tree_verify(np.broadcast_to(l, (R, N, V)).copy(), np.tile(parent, (R, 1)), np.tile(tok, (R, 1)),
                      *_params(R, T, K, P), seed=21, offset=5)
    keys = sorted(law)
    index = {kk: i for i, kk in enumerate(keys)}
    counts = np.zeros(len(keys))
    for b in range(R):
        seq = tuple(int(x) for x in r.tokens[b, :r.accept_len[b]])
        assert seq in index, f"impossible sequence {seq}"
        counts[index[seq]] += 1
    probs = np.array([law[kk] for kk in keys])
    big = probs * R >= 5
    c2 = np.append(counts[big], counts[~big].sum())
    p2 = np.append(probs[big], probs[~big].sum())
    assert chi2_pvalue(c2, p2) > CHI2_P_MIN
    # closed form of the expected accept length
    def path_prob(v):
        pr, u = 1.0, v
        while u != 0:
            pr *= p_rows[parent[u]][tok[u]]
            u = parent[u]
        return pr
    expected = 1.0 + sum(path_prob(v) for v in range(1, N))
    np.testing.assert_allclose(sum(len(kk) * law[kk] for kk in keys), expected, rtol=1e-12)
    sd = np.std(r.accept_len)
    assert abs(r.accept_len.mean() - expected) < 5 * sd / math.sqrt(R)


def pin_tree_rules(o):
    """Greedy walks follow the lowest-index argmax through the children (ties included) and end on the
    argmax; a child outside the kept set is never accepted; unusable trees and rows become sentinels."""
    V = 8
    l = np.zeros((1, 4, V), np.float32)
    l[0, 0, [3, 6]] = 2.0        # tie at the root: 3 is the lowest-index argmax
    l[0, 1, 5] = 1.0
    l[0, 3, 1] = 4.0
    par = np.array([[0, 0, 0, 1]], np.int32)
    tok = np.array([[0, 6, 3, 5]], np.int32)
    r = o.tree_verify(l, par, tok, *_params(1, 0.0))
    assert r.accept_len[0] == 2 and list(r.path[0, :2]) == [2, -1] and list(r.tokens[0, :3]) == [3, 0, -1]
    # node 2 is a leaf: its row's argmax is token 0 (all zeros): the bonus is the argmax
    r = o.tree_verify(l, par, np.array([[0, 3, 6, 5]], np.int32), *_params(1, 0.0))
    assert list(r.tokens[0, :3]) == [3, 5, 1] and list(r.path[0, :2]) == [1, 3]
    # top-k 1 at T > 0 is one-hot too: a child that is not the argmax is never accepted
    l1 = l.copy()
    l1[0, 0, 6] = 1.9             # no tie now: top-k 1 keeps token 3 alone
    rr = o.tree_verify(np.broadcast_to(l1, (200, 4, V)).copy(), np.tile([0, 0, 0, 1], (200, 1)),
                       np.tile([0, 6, 2, 5], (200, 1)), *_params(200, 1.0, 1))
    assert np.all(rr.accept_len == 1) and np.all(rr.tokens[:, 0] == 3)
    # unusable: parent not earlier, token out of range, siblings with one token, NaN in an unvisited row
    bad = [(np.array([[0, 0, 2, 1]]), tok), (par, np.array([[0, 6, 3, V]])), (par, np.array([[0, 6, 6, 5]]))]
    for pa, tk in bad:
        rb = o.tree_verify(l, pa, tk, *_params(1, 1.0))
        assert rb.accept_len[0] == 0 and np.all(rb.tokens == -1) and np.all(np.isnan(rb.logprobs))
    ln = l.copy()
    ln[0, 3, 7] = np.nan
    rb = o.tree_verify(ln, par, tok, *_params(1, 1.0))
    assert rb.accept_len[0] == 0
    # a single node: the token is drawn from the root's distribution
    r1 = o.tree_verify(l[:, :1].copy(), np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32), *_params(1, 0.0))
    assert r1.accept_len[0] == 1 and r1.tokens[0, 0] == 3


# ---------------------------------------------------------------------------------------
# per-row diagnostics: which rows a correct rounding could change, and how
# ---------------------------------------------------------------------------------------

def _diag_case(o, seed):
    """A verify batch whose rows mix untruncated, top-k and top-p parameters (tiny V, fresh drafts), with
    the textbook distributions of every row: (t, d, drafts, T, K, P, p[B][k+1], q[B][k])."""
    rng = np.random.default_rng(seed)
    B, k, V = 240, 3, 12
    t = rng.normal(0.0, 1.3, size=(B, k + 1, V)).astype(np.float32)
    d = (t[:, :k] + rng.normal(0.0, 0.8, size=(B, k, V))).astype(np.float32)
    T = f32(rng.uniform(0.6, 1.4, size=B))
    K = np.where(rng.random(B) < 0.3, 4, 0).astype(np.int32)
    P = f32(np.where(rng.random(B) < 0.3, 0.85, 1.0))
    drafts = _fresh_drafts(o, d, T, K, P)
    p = [[textbook_topk_topp(t[b, i].astype(np.float64), float(T[b]), int(K[b]), float(P[b])) for i in range(k + 1)]
         for b in range(B)]
    q = [[textbook_topk_topp(d[b, i].astype(np.float64), float(T[b]), int(K[b]), float(P[b])) for i in range(k)]
         for b in range(B)]
    return t, d, drafts, T, K, P, p, q


def _chain(o, seed, offset, b, drafts_b, p_b, q_b, flip=None):
    """Textbook accept chain of one row: (n, per-position distance |u - p/q| of the evaluated tests)."""
    k = len(q_b)
    dist = [math.inf] * k
    for i in range(k):
        x = int(drafts_b[i])
        pt, qd = p_b[i][x], q_b[i][x]
        u = o.accept_uniform(seed, b, i, offset)
        acc = pt > 0 and (qd == 0 or u < pt / qd)
        if flip == i:
            acc = not acc
        if pt > 0 and qd > 0:
            dist[i] = abs(u - pt / qd)
        if not acc:
            return i, dist
    return k, dist


def _race(o, seed, offset, b, n, w):
    """Gumbel race of one row in numpy: keys ln w(x) - ln(-ln U) on the draw stream, sorted descending:
    [(key, x), ...] over w(x) > 0."""
    keys = []
    for x in np.flatnonzero(w > 0):
        U = o.gumbel_uniform(seed, 1, b, n, int(x), offset)
        keys.append((math.log(w[x]) - math.log(-math.log(U)), int(x)))
    return sorted(keys, key=lambda kx: (-kx[0], kx[1]))


def pin_accept_margin(o):
    """accept_margin = min |u_i - p_i(x_i)/q_i(x_i)| over the accept tests the chain evaluates (up to and
    including the first rejection), recomputed from the accept uniforms and textbook distributions; the
    per-position distances are +inf past the first rejection."""
    t, d, drafts, T, K, P, p, q = _diag_case(o, 41)
    seed, off = 3, 5
    r = o.spec_verify(t, d, drafts, T, K, P, seed=seed, offset=off, details=True)
    for b in range(t.shape[0]):
        n, dist = _chain(o, seed, off, b, drafts[b], p[b], q[b])
        assert r.n_accepted[b] == n, (b, r.n_accepted[b], n)
        for i, dv in enumerate(dist):
            assert (math.isinf(dv) and math.isinf(r.accept_pos[b, i])) or abs(r.accept_pos[b, i] - dv) <= 1e-12, \
                (b, i, r.accept_pos[b, i], dv)
        want = min(dist)
        assert (math.isinf(want) and math.isinf(r.accept_margin[b])) or abs(r.accept_margin[b] - want) <= 1e-12, \
            (b, r.accept_margin[b], want)


def pin_gumbel_gap(o):
    """gumbel_gap = top-1 minus top-2 key of the draw (natural-log units) over the residual max(p_n - q_n, 0)
    or the bonus p_k, recomputed from the Gumbel uniforms; the drawn token is the top-1 key."""
    t, d, drafts, T, K, P, p, q = _diag_case(o, 42)
    seed, off = 8, 2
    r = o.spec_verify(t, d, drafts, T, K, P, seed=seed, offset=off)
    k = d.shape[1]
    for b in range(t.shape[0]):
        n = int(r.n_accepted[b])
        w = np.maximum(p[b][n] - q[b][n], 0.0) if n < k else p[b][k]
        keys = _race(o, seed, off, b, n, w)
        assert r.tokens[b, n] == keys[0][1], (b, r.tokens[b, n], keys[0])
        want = keys[0][0] - keys[1][0] if len(keys) > 1 else math.inf
        assert (math.isinf(want) and math.isinf(r.gumbel_gap[b])) or abs(r.gumbel_gap[b] - want) <= 1e-9, \
            (b, r.gumbel_gap[b], want)


def pin_topp_rows(o):
    """Per-row top-p distances inside the verify step equal the hand-worked ones: one batch row whose target
    rows and draft row have cumulative masses 0.5, 0.8, 0.95, 1 (and 0.4, 1 with ties), top-p 0.799999
    (float32), so the distances are |0.8 - P| or |0.5 - P| and the row's margin is their minimum."""
    probs = [np.log([0.5, 0.3, 0.15, 0.05]), np.log([0.3, 0.5, 0.05, 0.15]), np.log([0.4, 0.2, 0.2, 0.2])]
    t = np.stack([probs[0], probs[1]])[None].astype(np.float32)
    d = probs[2][None, None].astype(np.float32)
    P = f32([0.799999])
    r = o.spec_verify(t, d, np.array([[0]], np.int32), f32([1.0]), np.zeros(1, np.int32), P, details=True)
    Pd = float(P[0])
    for row, (at, prev) in enumerate([(0.8, 0.5), (0.8, 0.5), (1.0, 0.4)]):
        lg = (t[0, row] if row < 2 else d[0, 0]).astype(np.float64)
        e = np.exp(lg - lg.max())
        cum = np.cumsum(np.sort(e)[::-1]) / e.sum()   # masses of the upper sets, tie-free except row 2
        if row == 2:
            cum = np.array([cum[0], cum[-1]])
        j = int(np.searchsorted(cum, Pd, side="left"))
        want_at, want_prev = abs(cum[j] - Pd), abs(cum[j - 1] - Pd)
        assert abs(cum[j] - at) < 1e-6 and abs(cum[j - 1] - prev) < 1e-6
        np.testing.assert_allclose(r.topp_rows[0, row], [want_at, want_prev], rtol=0, atol=1e-12)
    assert abs(r.topp_margin[0] - r.topp_rows[0].min()) <= 1e-15


def pin_alternative_resolutions(o):
    """The alternatives the parity check may accept for a margin row are the textbook outcomes of the other
    resolution: the Gumbel runner-up is the second key of the race; a flipped accept test changes the
    chain there; a top-p threshold one distinct value lower or higher keeps one value more or fewer."""
    t, d, drafts, T, K, P, p, q = _diag_case(o, 43)
    seed, off = 6, 4
    B, k = d.shape[0], d.shape[1]
    base = o.spec_verify(t, d, drafts, T, K, P, seed=seed, offset=off)
    # the runner-up of every row's race
    alt = np.zeros((B, 4), np.int32)
    alt[:, 2] = 1 << 16
    alt[:, 3] = 1
    r = o.spec_verify(t, d, drafts, T, K, P, seed=seed, offset=off, alt=alt)
    for b in range(B):
        n = int(base.n_accepted[b])
        w = np.maximum(p[b][n] - q[b][n], 0.0) if n < k else p[b][k]
        keys = _race(o, seed, off, b, n, w)
        assert r.tokens[b, n] == (keys[1][1] if len(keys) > 1 else keys[0][1]), b
        assert r.accept_len[b] == base.accept_len[b]
    # the first accept test decided the other way
    alt[:, 2] = 1
    r = o.spec_verify(t, d, drafts, T, K, P, seed=seed, offset=off, alt=alt)
    for b in range(B):
        n, _ = _chain(o, seed, off, b, drafts[b], p[b], q[b], flip=0)
        assert r.n_accepted[b] == n and r.accept_len[b] == n + 1, b
        np.testing.assert_array_equal(r.tokens[b, :n], drafts[b, :n])
    # target row 0's top-p threshold one value lower / higher: alpha_0 and the logprob follow the textbook
    # kept set of one more / one fewer value (rows are tie-free)
    rows = [b for b in range(B) if P[b] < 1.0]
    for mask_col, extra in ((0, 1), (1, -1)):
        alt = np.zeros((B, 4), np.int32)
        alt[rows, mask_col] = 1
        alt[rows, 3] = 1
        r = o.spec_verify(t, d, drafts, T, K, P, seed=seed, offset=off, alt=alt)
        for b in rows:
            lg = t[b, 0].astype(np.float64)
            kept = int((p[b][0] > 0).sum())
            Kb = int(K[b]) if 0 < K[b] < lg.size else lg.size
            m = min(max(kept + extra, 1), Kb)
            order = np.argsort(-lg, kind="stable")
            pa = np.zeros_like(lg)
            pa[order[:m]] = softmax_T(lg[order[:m]], float(T[b]))
            np.testing.assert_allclose(r.alpha[b, 0], np.minimum(pa, q[b][0]).sum(), rtol=0, atol=1e-12)


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_") and callable(v)]
