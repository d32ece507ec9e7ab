"""Pins for the oracle's truncation, sampling and accept rule.

What fixes the expected values here (never the oracle itself):
* the worked example of "What is Speculative Decoding and How Does a Draft Model Work?",
  section "#2" (tests/golden/worked_example_dogs.json);
* the closed form of rejection sampling ("Qwen3.5 and Qwen3.6 MTP head reaches 1.4x on
  Apple Silicon after three fixes", "The verify was wrong under sampling"):
  P(accept) = sum_x min(p, q) and P(emit x) = p(x), checked exactly with Fractions on dyadic
  distributions by integrating over the uniforms interval by interval;
* special cases: top_k = 1 and top_p -> 0 give the argmax; top_k = V with top_p = 1 gives
  scipy's softmax; q == p always accepts; disjoint supports always reject;
* a Monte-Carlo chi-square test with Philox uniforms, and planted mistakes (negative
  controls) that the same test must reject.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import special, stats

from oracle import philox, sampling
from oracle.sampling import TokenList, accept, sample, truncate

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tl(ids, probs):
    ids = np.asarray(ids, dtype=np.int64)
    o = np.argsort(ids)
    return TokenList(ids[o], np.asarray(probs, dtype=F32)[o])


# ---------------------------------------------------------------- worked example
def test_worked_example_greedy():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_dogs.json")))
    vocab = g["vocab"]
    tid = {w: i for i, w in enumerate(vocab)}
    drafts = [tid[w] for w in g["drafts"]]
    # target rows: one-hot logits at the target's choice at each of the K+1 positions
    ps = []
    for w in g["target_choice"]:
        logits = np.full(len(vocab), -1.0, dtype=F32)
        logits[tid[w]] = 3.0
        ps.append(truncate(logits, 0.0, 20, 0.95))
    qs = [TokenList(np.array([d]), np.array([1.0], dtype=F32)) for d in drafts]
    r = accept(drafts, qs, ps, greedy=True)
    assert r.n == g["expected_n_accepted"]
    assert [vocab[t] for t in r.tokens] == g["expected_emitted"]
    assert len(r.tokens) >= 1          # at least one token per target pass


# ---------------------------------------------------------------- truncation
def brute_truncate(z, k, top_p):
    """Independent restatement with Python floats and a full sort of (value, id) pairs."""
    pairs = sorted(((-float(v), i) for i, v in enumerate(z)))
    kept = [i for _, i in pairs[:k]]
    m = max(float(z[i]) for i in kept)
    e = [np.exp(float(z[i]) - m) for i in kept]
    s = sum(e)
    p = [x / s for x in e]
    out, run = [], 0.0
    for i, pi in zip(kept, p):
        if out and run >= top_p:
            break
        out.append(i)
        run += pi
    return sorted(out)


def test_truncate_matches_brute_force_sets():
    rng = np.random.default_rng(0)
    for trial in range(200):
        V = int(rng.integers(2, 60))
        z = (rng.normal(0, 2, V)).astype(F32)
        k = int(rng.integers(1, V + 1))
        top_p = float(rng.uniform(0.05, 1.0))
        t = truncate(z, 1.0, k, top_p)
        if t.margin < 1e-5:
            continue          # boundary too close to decide in float64 vs float32
        assert list(t.ids) == brute_truncate(z, k, top_p), trial
        assert abs(float(t.probs.sum()) - 1.0) < 1e-5


def test_truncate_special_cases():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 3, 300).astype(F32)
    a = int(np.argmax(z))
    t1 = truncate(z, 1.0, 1, 0.95)
    assert list(t1.ids) == [a] and t1.probs[0] == 1.0
    t2 = truncate(z, 1.0, 300, 1e-9)
    assert list(t2.ids) == [a]
    t3 = truncate(z, 1.0, 0, 1.0)      # top_k disabled, top_p disabled: full softmax
    assert list(t3.ids) == list(range(300))
    np.testing.assert_allclose(t3.probs, special.softmax(z.astype(np.float64)), rtol=2e-6)
    g = truncate(z, 0.0, 20, 0.95)    # temperature 0: greedy
    assert list(g.ids) == [a]


def test_truncate_temperature_is_division():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 1, 100).astype(F32)
    t = truncate(z, 0.5, 10, 0.9)
    t_ref = truncate((z / F32(0.5)).astype(F32), 1.0, 10, 0.9)
    assert list(t.ids) == list(t_ref.ids)
    assert np.array_equal(t.probs, t_ref.probs)


def test_ties_break_on_lower_id_and_signed_zero():
    z = np.zeros(10, dtype=F32)
    z[7] = -0.0
    t = truncate(z, 1.0, 3, 1.0)
    assert list(t.ids) == [0, 1, 2]
    np.testing.assert_allclose(t.probs, [1 / 3] * 3, rtol=1e-6)
    z2 = np.array([1.0, 3.0, 3.0, 2.0], dtype=F32)
    assert list(truncate(z2, 0.0, 0, 1.0).ids) == [1]
    z3 = np.array([-0.0, 0.0, -1.0], dtype=F32)
    assert list(truncate(z3, 0.0, 0, 1.0).ids) == [0]
    assert list(truncate(z3, 1.0, 1, 1.0).ids) == [0]


def test_truncate_invalid_inputs():
    with pytest.raises(ValueError):
        truncate(np.array([0.0, np.nan], dtype=F32), 1.0, 2, 1.0)
    with pytest.raises(ValueError):
        truncate(np.array([0.0, np.inf], dtype=F32), 1.0, 2, 1.0)
    with pytest.raises(ValueError):
        truncate(np.array([-np.inf, -np.inf], dtype=F32), 1.0, 2, 1.0)
    # -inf entries are never kept
    t = truncate(np.array([-np.inf, 1.0, -np.inf], dtype=F32), 1.0, 3, 1.0)
    assert list(t.ids) == [1]


# ---------------------------------------------------------------- sampling from a list
def test_sample_inverse_cdf_by_hand():
    ids = np.array([3, 5, 9])
    w = np.array([0.25, 0.25, 0.5], dtype=F32)
    assert sample(ids, w, F32(0.0))[0] == 3
    assert sample(ids, w, F32(0.2))[0] == 3
    assert sample(ids, w, F32(0.25))[0] == 5     # c = 0.25 is not > 0.25
    assert sample(ids, w, F32(0.3))[0] == 5
    assert sample(ids, w, F32(0.5))[0] == 9
    assert sample(ids, w, F32(0.999))[0] == 9
    # unnormalized weights: threshold u * Z
    assert sample(ids, w * 4, F32(0.3))[0] == 5
    # zero-weight entries are never drawn
    assert sample(ids, np.array([0.0, 1.0, 0.0], dtype=F32), F32(0.999))[0] == 5


# ---------------------------------------------------------------- accept: exact integration
def dyadic_dist(rng, V, denom=16):
    """Random distribution over V ids with probabilities in (1/denom)Z, some zero."""
    while True:
        c = rng.integers(0, 5, V)
        if c.sum() > 0:
            break
    # scale to sum to denom with a remainder on the largest entry
    tot = int(c.sum())
    w = [Fraction(int(x), tot) for x in c]
    # round to multiples of 1/denom keeping the sum at 1
    q = [Fraction(int(x * denom), denom) for x in w]
    q[int(np.argmax(c))] += 1 - sum(q)
    return q


def as_list(fr):
    ids = [i for i, f in enumerate(fr) if f > 0]
    return TokenList(np.array(ids, dtype=np.int64), np.array([float(fr[i]) for i in ids], dtype=F32))


def intervals(cuts):
    """Split [0,1) at the given cut points -> list of (lo, hi) with hi > lo."""
    pts = sorted(set([Fraction(0), Fraction(1)] + [c for c in cuts if 0 < c < 1]))
    return [(a, b) for a, b in zip(pts[:-1], pts[1:])]


def exact_accept_distribution(ps, qs):
    """Distribution of (n, emitted tokens) for the oracle's accept() when drafts are drawn
    from q and the uniforms are continuous U[0,1): call accept() once per cell of the
    partition of the uniforms on which its outcome is constant, weight by the cell volume."""
    K = len(qs)
    V = len(ps[0])
    Lp = [as_list(p) for p in ps]
    Lq = [as_list(q) for q in qs]
    dist = {}
    for drafts in itertools.product(range(V), repeat=K):
        w = Fraction(1)
        for j, d in enumerate(drafts):
            w *= qs[j][d]
        if w == 0:
            continue
        # cut points: accept ratios p_{j}(d_{j+1}) / q_{j+1}(d_{j+1}); residual CDF steps
        acc_cuts = [[qs[j][drafts[j]] and ps[j][drafts[j]] / qs[j][drafts[j]]] for j in range(K)]
        res_cuts = set()
        for j in range(K + 1):
            p = ps[j]
            rows = [p]
            if j < K:
                r = [max(Fraction(0), p[x] - qs[j][x]) for x in range(V)]
                if sum(r) > 0:
                    rows.append([x / sum(r) for x in r])
            for row in rows:
                c = Fraction(0)
                for x in range(V):
                    c += row[x]
                    res_cuts.add(c)
        res_iv = intervals(res_cuts)
        acc_iv = [intervals(c) for c in acc_cuts]
        for cells in itertools.product(*acc_iv):
            vol = Fraction(1)
            for a, b in cells:
                vol *= (b - a)
            u_acc = [F32(float((a + b) / 2)) for a, b in cells]
            for a, b in res_iv:
                u_res = F32(float((a + b) / 2))
                r = accept(list(drafts), Lq, Lp, False, u_acc, u_res)
                key = (r.n, tuple(r.tokens))
                dist[key] = dist.get(key, Fraction(0)) + w * vol * (b - a)
    return dist


@pytest.mark.parametrize("V,K,seed", [(3, 1, 0), (4, 1, 1), (3, 2, 2), (4, 2, 3), (3, 3, 4)])
def test_accept_exact_distribution(V, K, seed):
    rng = np.random.default_rng(seed)
    ps = [dyadic_dist(rng, V) for _ in range(K + 1)]
    qs = [dyadic_dist(rng, V) for _ in range(K)]
    dist = exact_accept_distribution(ps, qs)
    assert sum(dist.values()) == 1
    # first emitted token ~ p_0 exactly
    for x in range(V):
        assert sum(pr for (n, t), pr in dist.items() if t[0] == x) == ps[0][x]
    # P(n >= j) = prod_{i<j} beta_i, beta_i = sum_x min(p_i, q_{i+1})
    betas = [sum(min(ps[i][x], qs[i][x]) for x in range(V)) for i in range(K)]
    for j in range(1, K + 1):
        want = Fraction(1)
        for i in range(j):
            want *= betas[i]
        assert sum(pr for (n, t), pr in dist.items() if n >= j) == want
    # given n >= 1, the second emitted token ~ p_1 exactly
    if K >= 1:
        tot = sum(pr for (n, t), pr in dist.items() if n >= 1)
        if tot > 0:
            for x in range(V):
                got = sum(pr for (n, t), pr in dist.items() if n >= 1 and t[1] == x)
                assert got / tot == ps[1][x]


# ---------------------------------------------------------------- accept: special cases
def test_accept_q_equals_p_always_accepts():
    rng = np.random.default_rng(3)
    for _ in range(50):
        z = rng.normal(0, 2, 50).astype(F32)
        p = truncate(z, 1.0, 20, 0.95)
        K = 4
        drafts = list(rng.choice(p.ids, size=K))
        u = philox.uniforms_np(9, np.arange(1, K + 1), 0, 0, 1)
        r = accept(drafts, [p] * K, [p] * (K + 1), False, u, F32(0.5))
        assert r.n == K and r.tokens[:K] == [int(d) for d in drafts]


def test_accept_disjoint_support_rejects_and_emits_p():
    p = tl([0, 1], [0.5, 0.5])
    q = tl([2, 3], [0.25, 0.75])
    for d in (2, 3):
        for u in (0.0, 0.5, 0.99):
            r = accept([d], [q], [p, p], False, [F32(u)], F32(0.7))
            assert r.n == 0 and r.tokens == [1]      # residual = p, u_res = 0.7 -> id 1


def test_accept_one_hot_q_accepts_with_prob_p():
    p = tl([0, 1, 2], [0.125, 0.375, 0.5])
    q = tl([1], [1.0])
    assert accept([1], [q], [p, p], False, [F32(0.374)], F32(0.1)).n == 1
    r = accept([1], [q], [p, p], False, [F32(0.376)], F32(0.1))
    assert r.n == 0
    # residual = p with the draft removed, renormalized: {0: 0.2, 2: 0.8}
    assert r.tokens == [0]
    assert accept([1], [q], [p, p], False, [F32(0.376)], F32(0.25)).tokens == [2]


def test_greedy_equals_sampled_rule_on_one_hot_lists():
    rng = np.random.default_rng(4)
    for _ in range(100):
        K = int(rng.integers(1, 6))
        V = 7
        p_rows = [rng.normal(0, 1, V).astype(F32) for _ in range(K + 1)]
        ps = [truncate(z, 0.0, 20, 0.95) for z in p_rows]
        drafts = [int(x) for x in rng.integers(0, V, K)]
        qs = [TokenList(np.array([d]), np.array([1.0], dtype=F32)) for d in drafts]
        u = rng.uniform(0, 1, K).astype(F32)
        g = accept(drafts, qs, ps, True)
        s = accept(drafts, qs, ps, False, u, F32(rng.uniform()))
        assert (g.n, g.tokens) == (s.n, s.tokens)


# ---------------------------------------------------------------- Monte-Carlo with power
def mc_first_token(p_logits, q_logits, trunc_p, trunc_q, trials, seed):
    V = len(p_logits)
    p = truncate(p_logits, 1.0, *trunc_p)
    q = truncate(q_logits, 1.0, *trunc_q)
    counts = np.zeros(V, dtype=np.int64)
    acc = 0
    idx = np.arange(trials)
    ud = philox.uniforms_np(seed, 1, idx, 0, philox.STREAM_DRAFT)
    ua = philox.uniforms_np(seed, 1, idx, 0, philox.STREAM_ACCEPT)
    ur = philox.uniforms_np(seed, 0, idx, 0, philox.STREAM_RESIDUAL)
    # draws from q by inverse CDF over q's ascending ids (vectorized form of sample())
    qc = np.cumsum(q.probs, dtype=F32)
    qd = q.ids[np.minimum(np.searchsorted(qc, (ud * qc[-1]).astype(F32), side="right"), len(qc) - 1)]
    for t in range(trials):
        d = int(qd[t])
        r = accept([d], [q], [p, p], False, [ua[t]], ur[t])
        counts[r.tokens[0]] += 1
        acc += r.n
    return counts, acc / trials, p


def chi2_p(counts, p, V):
    exp = np.zeros(V)
    exp[p.ids] = p.probs.astype(np.float64)
    m = exp > 0
    if counts[~m].sum() > 0:       # a token outside p's support was emitted
        return 0.0
    return stats.chisquare(counts[m], exp[m] / exp[m].sum() * counts.sum()).pvalue


TRIALS = 1 << 17


def test_mc_emitted_follows_target_untruncated_and_truncated():
    rng = np.random.default_rng(11)
    V = 8
    pl = rng.normal(0, 1.5, V).astype(F32)
    ql = (pl + rng.normal(0, 1.0, V)).astype(F32)
    for trunc in [(0, 1.0), (5, 0.9)]:
        counts, beta, p = mc_first_token(pl, ql, trunc, trunc, TRIALS, 1)
        assert chi2_p(counts, p, V) > 1e-6
        q = truncate(ql, 1.0, *trunc)
        want = sum(min(float(p.prob(x)), float(q.prob(x))) for x in range(V))
        assert abs(beta - want) < 5 * np.sqrt(want * (1 - want) / TRIALS) + 1e-3


def test_mc_negative_control_resample_from_p(monkeypatch):
    """Planted mistake: resampling from p instead of the residual must fail the same test."""
    rng = np.random.default_rng(11)
    V = 8
    pl = rng.normal(0, 1.5, V).astype(F32)
    ql = (pl + rng.normal(0, 1.0, V)).astype(F32)
    monkeypatch.setattr(sampling, "residual", lambda p, q: p.probs.copy())
    counts, _, p = mc_first_token(pl, ql, (0, 1.0), (0, 1.0), TRIALS, 1)
    assert chi2_p(counts, p, V) < 1e-6


def test_acceptance_beats_naive_and_untruncated_controls():
    """Acceptance of the rule, sum min(p, q), exceeds the naive independent-sample compare
    (sum p*q) and an untruncated verify against a truncated draft."""
    rng = np.random.default_rng(12)
    V = 64
    pl = rng.normal(0, 2.0, V).astype(F32)
    ql = (pl + rng.normal(0, 0.7, V)).astype(F32)
    p = truncate(pl, 1.0, 20, 0.95)
    q = truncate(ql, 1.0, 20, 0.95)
    p_full = truncate(pl, 1.0, 0, 1.0)
    rule = sum(min(float(p.prob(x)), float(q.prob(x))) for x in range(V))
    naive = sum(float(p.prob(x)) * float(q.prob(x)) for x in range(V))
    untrunc = sum(min(float(p_full.prob(x)), float(q.prob(x))) for x in range(V))
    assert rule > naive
    assert rule > untrunc
