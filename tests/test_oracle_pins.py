"""Pins of the CPU oracle to what the pages and the mathematics fix, independent of the oracle's own code.

- library routines for the building blocks (scipy softmax / log-softmax, numpy searchsorted, brute-force loops);
- the exact output law of one verification cycle, found by probing the oracle as a black box (bisection on its
  uniforms) and compared with the closed form that Leviathan et al.'s argument gives (Uno, "What 'lossless' actually
  has to mean"): P(n = m, prefix a, next b) = prod_{j<m} min(p_j, q_j)(a_j) * max(p_m - q_m, 0)(b), and
  prod_{j<gamma} min(p_j, q_j)(a_j) * p_gamma(b) for the bonus;
- Monte Carlo: the emitted law equals p, also across cycles of a context-dependent (Markov) toy model; acceptance
  rate = sum min(p, q) = 1 - TV(p, q) (Uno, "Numbers that don't quite agree with each other"); E[n] closed form;
- special cases: q = p accepts everything; one-hot == dense with -inf draft logits; sparse with full supports ==
  dense; window round 0 == dense; hand-derived golden cases (tests/golden/rule_cases.json).
"""
import fractions
import itertools
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle import verify as ov

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rule_cases.json")


# ----------------------------------------------------------------------------------------------------------------------
# Building blocks against library routines and brute force
# ----------------------------------------------------------------------------------------------------------------------

def test_softmax_and_log_softmax_match_scipy():
    rng = np.random.default_rng(1)
    a = rng.normal(0, 5, (7, 33))
    a[0, 3] = -np.inf
    a[2, :5] = -np.inf
    np.testing.assert_allclose(oracle.softmax(a), special.softmax(a, axis=-1), rtol=1e-13, atol=0)
    x = rng.integers(5, 33, 7)
    ref = special.log_softmax(a, axis=-1)[np.arange(7), x]
    np.testing.assert_allclose(oracle.log_softmax_at(a, x), ref, rtol=1e-12, atol=1e-13)


def _brute_draw(r, t):
    c = 0.0
    for i, ri in enumerate(r):
        c += ri
        if c > t:
            return i
    pos = [i for i, ri in enumerate(r) if ri > 0]
    return pos[-1] if pos else -1


def test_inverse_cdf_matches_brute_force_and_searchsorted():
    rng = np.random.default_rng(2)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        r = rng.random(n) * (rng.random(n) < 0.6)
        if r.sum() == 0:
            r[rng.integers(0, n)] = 0.3
        u = rng.random()
        t = u * r.sum()
        idx, margin = oracle.inverse_cdf(r, t)
        assert idx[0] == _brute_draw(r, t)
        assert idx[0] == min(np.searchsorted(np.cumsum(r), t, side="right"), n - 1) or idx[0] == _brute_draw(r, t)
        assert r[idx[0]] > 0          # zero-mass entries are never chosen
        assert margin[0] >= 0


def test_inverse_cdf_boundaries_and_clamp():
    r = np.array([0.0, 0.25, 0.0, 0.25, 0.5])
    assert oracle.inverse_cdf(r, 0.0)[0][0] == 1           # C_1 = 0.25 > 0
    assert oracle.inverse_cdf(r, 0.25)[0][0] == 3          # C_1 = 0.25 is not > 0.25
    assert oracle.inverse_cdf(r, 0.999)[0][0] == 4
    idx, margin = oracle.inverse_cdf(r, 1.0)               # t at the total: clamp to the last positive entry
    assert idx[0] == 4 and margin[0] == 0
    r2 = np.array([0.2, 0.3, 0.0, 0.0])
    assert oracle.inverse_cdf(r2, 0.5)[0][0] == 1


def test_residual_mass_is_total_variation():
    rng = np.random.default_rng(3)
    for _ in range(50):
        V = int(rng.integers(2, 60))
        p = special.softmax(rng.normal(0, 2, V))
        q = special.softmax(rng.normal(0, 2, V))
        r = oracle.residual(p, q)
        tv = 0.5 * np.abs(p - q).sum()
        assert abs(r.sum() - tv) < 1e-14
        assert abs(r.sum() - (1.0 - np.minimum(p, q).sum())) < 1e-14
        assert np.all(r >= 0)
        assert abs((r / r.sum()).sum() - 1.0) < 1e-14


# ----------------------------------------------------------------------------------------------------------------------
# Exact output law by black-box probing of the oracle
# ----------------------------------------------------------------------------------------------------------------------

def _bisect(pred, shape, iters=64):
    """Threshold of a predicate that is True below it and False above it, on [0, 1]."""
    lo = np.zeros(shape)
    hi = np.ones(shape)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        below = pred(mid)
        lo = np.where(below, mid, lo)
        hi = np.where(below, hi, mid)
    return 0.5 * (lo + hi)


def _probe_law(run, B, G, V_out, token_of):
    """Law of (n, out_token) per batch row by probing ``run(u_accept, u_sample) -> result`` on exact u-intervals.

    ``token_of(result, m)`` maps the emitted token to its position in the CDF used for a draw at slot m (the inverse
    CDF is monotone in that position). Returns alpha [B, G] (acceptance thresholds) and lens[m][B, V_out] (probability
    of each CDF position when the first rejection is at slot m; m = G is the bonus draw)."""
    alpha = _bisect(lambda u: run(u, np.zeros((B, G + 1)))["accept"].astype(bool), (B, G))
    lens = []
    for m in range(G + 1):
        ua = np.zeros((B, G))
        if m < G:
            ua[:, m] = 1.0                                     # u = 1 rejects whatever the ratio
        col = m

        def tok(s, ua=ua, col=col, m=m):
            us = np.zeros((B, G + 1))
            us[:, col] = s
            return token_of(run(ua, us), m)

        cum = np.zeros((B, V_out + 1))
        cum[:, V_out] = 1.0
        for i in range(V_out - 1):
            cum[:, i + 1] = _bisect(lambda s, i=i: tok(s) <= i, (B,))
        lens.append(np.diff(cum, axis=1))
    return alpha, lens


def _law_from_probe(alpha, lens, weights, prefix_of, G, label_of=lambda m, b: b):
    """Combine probed pieces into {(m, prefix, token): prob}."""
    law = {}
    B = alpha.shape[0]
    for m in range(G + 1):
        for bi in range(B):
            w = weights[bi] * np.prod(alpha[bi, :m]) * ((1.0 - alpha[bi, m]) if m < G else 1.0)
            if w == 0:
                continue
            for b, l in enumerate(lens[m][bi]):
                if l > 0:
                    key = (m, prefix_of(bi, m), label_of(m, b))
                    law[key] = law.get(key, 0.0) + w * l
    return law


@pytest.mark.parametrize("T,seed", [(1.0, 0), (0.7, 1), (1.7, 2)])
def test_exact_law_dense_matches_leviathan_closed_form(T, seed):
    rng = np.random.default_rng(seed)
    V, G = 4, 3
    zt = rng.normal(0, 1.5, (G + 1, V)).astype(np.float32)
    zd = (zt[:G] + rng.normal(0, 1.0, (G, V))).astype(np.float32)
    Tf = np.float64(np.float32(T))
    p = special.softmax(zt.astype(np.float64) / Tf, axis=-1)
    q = special.softmax(zd.astype(np.float64) / Tf, axis=-1)
    tuples = np.array(list(itertools.product(range(V), repeat=G)), dtype=np.int32)
    B = len(tuples)
    tgt = np.broadcast_to(zt, (B, G + 1, V))
    dft = np.broadcast_to(zd, (B, G, V))

    def run(ua, us):
        return oracle.verify_dense(tgt, dft, tuples, ua, us, T)

    alpha, lens = _probe_law(run, B, G, V, lambda r, m: r["out_token"])
    weights = np.prod(q[np.arange(G), tuples], axis=1)
    law = _law_from_probe(alpha, lens, weights, lambda bi, m: tuple(tuples[bi, :m]), G)

    closed = {}
    for m in range(G + 1):
        for prefix in itertools.product(range(V), repeat=m):
            base = np.prod([min(p[j, a], q[j, a]) for j, a in enumerate(prefix)])
            nxt = np.maximum(p[m] - q[m], 0) if m < G else p[G]
            for b in range(V):
                if base * nxt[b] > 0:
                    closed[(m, prefix, b)] = base * nxt[b]
    assert abs(sum(law.values()) - 1.0) < 1e-12
    assert abs(sum(closed.values()) - 1.0) < 1e-12
    for key in set(law) | set(closed):
        assert abs(law.get(key, 0.0) - closed.get(key, 0.0)) < 1e-12, key
    # marginal of the first emitted token is p_0 (the lossless property)
    first = np.zeros(V)
    for (m, prefix, b), v in law.items():
        first[prefix[0] if m > 0 else b] += v
    np.testing.assert_allclose(first, p[0], atol=1e-12)


def test_exact_law_onehot_matches_closed_form():
    rng = np.random.default_rng(5)
    V, G = 5, 3
    zt = rng.normal(0, 1.5, (G + 1, V)).astype(np.float32)
    T = 0.7
    p = special.softmax(zt.astype(np.float64) / np.float64(np.float32(T)), axis=-1)
    d = np.array([[1, 0, 3]], dtype=np.int32)

    def run(ua, us):
        return oracle.verify_onehot(zt[None], d, ua, us, T)

    alpha, lens = _probe_law(run, 1, G, V, lambda r, m: r["out_token"])
    law = _law_from_probe(alpha, lens, [1.0], lambda bi, m: tuple(d[0, :m]), G)
    for m in range(G + 1):
        base = np.prod([p[j, d[0, j]] for j in range(m)])
        for b in range(V):
            want = base * (p[m, b] * (b != d[0, m]) if m < G else p[G, b])
            assert abs(law.get((m, tuple(d[0, :m]), b), 0.0) - want) < 1e-12
    first = np.zeros(V)
    for (m, prefix, b), v in law.items():
        first[prefix[0] if m > 0 else b] += v
    np.testing.assert_allclose(first, p[0], atol=1e-12)


def test_exact_law_sparse_matches_closed_form():
    rng = np.random.default_rng(6)
    Vtot, k, G, mass = 9, 4, 2, 0.9375
    p_ids = np.stack([rng.choice(Vtot, k, replace=False) for _ in range(G + 1)]).astype(np.int32)
    q_ids = []
    for j in range(G):
        shared = rng.choice(p_ids[j], 2, replace=False)
        rest = rng.choice(np.setdiff1d(np.arange(Vtot), p_ids[j]), k - 2, replace=False)
        q_ids.append(rng.permutation(np.concatenate([shared, rest])))
    q_ids = np.array(q_ids, dtype=np.int32)
    # probabilities that are exact in float32 and sum to the same mass on both sides
    p_probs = np.array([rng.permutation([0.5, 0.25, 0.125, 0.0625]) for _ in range(G + 1)], np.float32)
    q_probs = np.array([rng.permutation([0.375, 0.3125, 0.1875, 0.0625]) for _ in range(G)], np.float32)
    assert np.allclose(p_probs.sum(-1), mass) and np.allclose(q_probs.sum(-1), mass)
    tuples = np.array(list(itertools.product(range(k), repeat=G)))
    B = len(tuples)
    spec = q_ids[np.arange(G), tuples].astype(np.int32)

    def run(ua, us):
        return oracle.verify_sparse(np.broadcast_to(p_ids, (B, G + 1, k)), np.broadcast_to(p_probs, (B, G + 1, k)),
                                    np.broadcast_to(q_ids, (B, G, k)), np.broadcast_to(q_probs, (B, G, k)),
                                    spec, ua, us)

    def slot_of(r, m):
        tok = r["out_token"]
        return np.argmax(p_ids[m][None, :] == tok[:, None], axis=1)

    alpha, lens = _probe_law(run, B, G, k, slot_of)
    weights = np.prod(q_probs[np.arange(G), tuples].astype(np.float64) / mass, axis=1)
    law = _law_from_probe(alpha, lens, weights, lambda bi, m: tuple(spec[bi, :m]), G,
                          label_of=lambda m, s: int(p_ids[m][s]))

    def dist(ids, probs):
        v = np.zeros(Vtot)
        v[ids] = probs.astype(np.float64) / mass
        return v
    P = [dist(p_ids[j], p_probs[j]) for j in range(G + 1)]
    Q = [dist(q_ids[j], q_probs[j]) for j in range(G)]
    closed = {}
    for m in range(G + 1):
        for prefix in itertools.product(range(Vtot), repeat=m):
            base = np.prod([min(P[j][a], Q[j][a]) for j, a in enumerate(prefix)])
            nxt = np.maximum(P[m] - Q[m], 0) if m < G else P[G]
            for b in range(Vtot):
                if base * nxt[b] > 0:
                    closed[(m, prefix, b)] = base * nxt[b]
    assert abs(sum(law.values()) - 1.0) < 1e-12
    for key in set(law) | set(closed):
        assert abs(law.get(key, 0.0) - closed.get(key, 0.0)) < 1e-12, key


# ----------------------------------------------------------------------------------------------------------------------
# Monte Carlo
# ----------------------------------------------------------------------------------------------------------------------

def _draw(rng, probs, n):
    """n draws from each row of probs (independent), by inverse CDF in the test (not the oracle's)."""
    c = np.cumsum(probs, axis=-1)
    u = rng.random((n,) + probs.shape[:-1])
    return (u[..., None] >= c).sum(-1).clip(max=probs.shape[-1] - 1)


def _chi2_ok(counts, probs):
    keep = probs > 0
    assert counts[~keep].sum() == 0
    res = stats.chisquare(counts[keep], probs[keep] / probs[keep].sum() * counts.sum())
    return res.pvalue > 1e-6


def test_monte_carlo_emitted_law_acceptance_and_length():
    rng = np.random.default_rng(11)
    V, G, N = 8, 3, 200_000
    zt = rng.normal(0, 1.5, (G + 1, V)).astype(np.float32)
    zd = (zt[:G] + rng.normal(0, 1.0, (G, V))).astype(np.float32)
    p = special.softmax(zt.astype(np.float64), axis=-1)
    q = special.softmax(zd.astype(np.float64), axis=-1)
    ids = _draw(rng, q, N).astype(np.int32)                         # [N, G]
    res = oracle.verify_dense(np.broadcast_to(zt, (N, G + 1, V)), np.broadcast_to(zd, (N, G, V)), ids,
                              rng.random((N, G)), rng.random((N, G + 1)), 1.0)
    n, tok, acc = res["n_accepted"], res["out_token"], res["accept"].astype(bool)
    beta = np.minimum(p[:G], q).sum(-1)
    # raw per-position acceptance rate = sum min(p, q) = 1 - TV(p, q)
    for j in range(G):
        sd = np.sqrt(beta[j] * (1 - beta[j]) / N)
        assert abs(acc[:, j].mean() - beta[j]) < 5 * sd
    # E[n] = sum_k prod_{j<=k} beta_j
    en = sum(np.prod(beta[:k + 1]) for k in range(G))
    assert abs(n.mean() - en) < 5 * n.std() / np.sqrt(N)
    assert n.min() >= 0 and n.max() <= G
    # k-th emitted token (k = 0..G) among trials with n >= k has law p_k
    for kk in range(G + 1):
        sel = n >= kk
        emitted = np.where(n[sel] > kk, ids[sel, min(kk, G - 1)], tok[sel])
        counts = np.bincount(emitted, minlength=V)
        assert _chi2_ok(counts, p[kk]), kk


def test_monte_carlo_q_equals_p_accepts_everything():
    rng = np.random.default_rng(12)
    V, G, N = 6, 4, 100_000
    zt = rng.normal(0, 2, (G + 1, V)).astype(np.float32)
    p = special.softmax(zt.astype(np.float64), axis=-1)
    ids = _draw(rng, p[:G], N).astype(np.int32)
    res = oracle.verify_dense(np.broadcast_to(zt, (N, G + 1, V)), np.broadcast_to(zt[:G], (N, G, V)), ids,
                              rng.random((N, G)), rng.random((N, G + 1)), 1.0)
    assert np.all(res["accept"] == 1) and np.all(res["n_accepted"] == G)
    assert _chi2_ok(np.bincount(res["out_token"], minlength=V), p[G])


def test_monte_carlo_markov_decode_is_lossless():
    """Full speculative decoding with context: target and drafter are Markov chains over V tokens (next-token law
    depends on the previous token). Cycles of gamma drafts + one verification must emit sequences whose law is the
    target chain's, whatever the drafter (Uno, 'What lossless actually has to mean')."""
    rng = np.random.default_rng(13)
    V, G, L, N = 3, 2, 3, 150_000
    P = special.softmax(rng.normal(0, 1.2, (V, V)), axis=-1)
    Q = special.softmax(rng.normal(0, 1.2, (V, V)), axis=-1)
    lP, lQ = np.log(P).astype(np.float32), np.log(Q).astype(np.float32)
    start_tok = 0
    seqs = np.full((N, L + G + 1), -1, np.int64)
    length = np.zeros(N, np.int64)
    last = np.full(N, start_tok)
    while (length < L).any():
        act = np.flatnonzero(length < L)
        na = act.size
        drafts = np.empty((na, G), np.int64)
        prev = last[act]
        for j in range(G):
            c = np.cumsum(Q[prev], axis=-1)
            drafts[:, j] = (rng.random(na)[:, None] >= c).sum(-1).clip(max=V - 1)
            prev = drafts[:, j]
        ctx = np.concatenate([last[act][:, None], drafts], axis=1)      # context of each verified position
        tgt = lP[ctx]                                                   # [na, G+1, V]
        dft = lQ[ctx[:, :G]]
        res = oracle.verify_dense(tgt, dft, drafts.astype(np.int32), rng.random((na, G)), rng.random((na, G + 1)), 1.0)
        n, tok = res["n_accepted"], res["out_token"]
        for i, s in enumerate(act):
            emit = list(drafts[i, :n[i]]) + [tok[i]]
            seqs[s, length[s]:length[s] + len(emit)] = emit
            length[s] += len(emit)
            last[s] = emit[-1]
    outcomes = seqs[:, :L]
    code = (outcomes * V ** np.arange(L)).sum(-1)
    counts = np.bincount(code, minlength=V ** L)
    law = np.zeros(V ** L)
    for seq in itertools.product(range(V), repeat=L):
        pr, prev = 1.0, start_tok
        for tkn in seq:
            pr *= P[prev, tkn]
            prev = tkn
        law[sum(t * V ** i for i, t in enumerate(seq))] = pr
    assert _chi2_ok(counts, law)


# ----------------------------------------------------------------------------------------------------------------------
# Special cases and equivalences
# ----------------------------------------------------------------------------------------------------------------------

def test_onehot_equals_dense_with_minus_inf_draft_logits():
    rng = np.random.default_rng(21)
    B, G, V = 40, 4, 50
    zt = rng.normal(0, 2, (B, G + 1, V)).astype(np.float32)
    d = rng.integers(0, V, (B, G)).astype(np.int32)
    zd = np.full((B, G, V), -np.inf, np.float32)
    np.put_along_axis(zd, d[..., None].astype(np.int64), 0.0, axis=-1)
    ua, us = rng.random((B, G)).astype(np.float32), rng.random((B, G + 1)).astype(np.float32)
    a = oracle.verify_onehot(zt, d, ua, us, 0.8)
    b = oracle.verify_dense(zt, zd, d, ua, us, 0.8)
    for key in ("accept", "n_accepted", "out_token"):
        np.testing.assert_array_equal(a[key], b[key])
    np.testing.assert_allclose(a["p_draft"], b["p_draft"], rtol=1e-14)


def test_sparse_with_full_support_equals_dense():
    rng = np.random.default_rng(22)
    B, G, V = 30, 3, 24
    zt = rng.normal(0, 2, (B, G + 1, V))
    zd = zt[:, :G] + rng.normal(0, 1, (B, G, V))
    p = special.softmax(zt, axis=-1).astype(np.float32)
    q = special.softmax(zd, axis=-1).astype(np.float32)
    ids = np.stack([_draw(rng, q[b].astype(np.float64), 1)[0] for b in range(B)]).astype(np.int32)
    ua, us = rng.random((B, G)).astype(np.float32), rng.random((B, G + 1)).astype(np.float32)
    full = np.broadcast_to(np.arange(V, dtype=np.int32), (B, G + 1, V))
    s = oracle.verify_sparse(full, p, full[:, :G], q, ids, ua, us)
    # the dense rule on the same probabilities: logits log p, log q at T = 1
    d = oracle.verify_dense(np.log(p.astype(np.float64)), np.log(q.astype(np.float64)), ids, ua, us, 1.0)
    ok = (s["margin_accept"] > 1e-6).all(-1) & (s["margin_cdf"] > 1e-6)
    assert ok.mean() > 0.9
    for key in ("accept", "n_accepted", "out_token"):
        np.testing.assert_array_equal(s[key][ok], d[key][ok])


def test_window_round_zero_equals_dense_and_start_chains():
    rng = np.random.default_rng(23)
    B, W, V = 12, 6, 40
    zd = rng.normal(0, 2, (B, W, V)).astype(np.float32)
    zt = (zd + rng.normal(0, 0.7, (B, W, V))).astype(np.float32)
    order = np.stack([rng.permutation(W) for _ in range(B)]).astype(np.int32)
    ids = rng.integers(0, V, (B, W)).astype(np.int32)
    ua = rng.random((4, B, W)).astype(np.float32)
    us = rng.random((4, B, W + 1)).astype(np.float32)
    res = oracle.verify_windows(zt, zd, ids, ua, us, 1.0, order=order)
    # round 0 with order sigma == dense on rows permuted into slot order
    bi = np.arange(B)[:, None]
    perm = oracle.verify_dense(zt[bi, order], zd[bi, order], ids[bi, order], ua[0][bi, order],
                               np.concatenate([us[0][bi, order], us[0][:, W:]], axis=1), 1.0, bonus=0)
    np.testing.assert_array_equal(res[0]["n_accepted"], perm["n_accepted"])
    np.testing.assert_array_equal(res[0]["out_token"], perm["out_token"])
    np.testing.assert_array_equal(res[0]["accept"][bi, order], perm["accept"])
    prev = np.zeros(B)
    for r in res:
        assert np.all(r["start_out"] >= prev) and np.all(r["start_out"] <= W)
        prev = r["start_out"]
    # a finished window does nothing
    done = oracle.verify_dense(zt, zd, ids, ua[0], us[0], 1.0, bonus=0, start=np.full(B, W), order=order)
    assert np.all(done["n_accepted"] == 0) and np.all(done["out_token"] == -1) and np.all(done["accept"] == 0)


def test_sparse_accept_is_the_exact_rational_comparison():
    rng = np.random.default_rng(24)
    B, G, k = 200, 4, 8
    p_ids = np.stack([np.stack([rng.choice(50, k, replace=False) for _ in range(G + 1)]) for _ in range(B)])
    q_ids = np.stack([np.stack([rng.choice(50, k, replace=False) for _ in range(G)]) for _ in range(B)])
    pp = rng.random((B, G + 1, k)).astype(np.float32)
    qp = rng.random((B, G, k)).astype(np.float32)
    spec = q_ids[..., 0].astype(np.int32)
    ua = rng.random((B, G)).astype(np.float32)
    res = oracle.verify_sparse(p_ids.astype(np.int32), pp, q_ids.astype(np.int32), qp, spec, ua,
                               np.zeros((B, G + 1), np.float32))
    for b in range(B):
        for j in range(G):
            F = fractions.Fraction
            ps = sum((F(float(v)) for i, v in zip(p_ids[b, j], pp[b, j]) if i == spec[b, j]), F(0))
            qs = sum((F(float(v)) for i, v in zip(q_ids[b, j], qp[b, j]) if i == spec[b, j]), F(0))
            want = qs > 0 and F(float(ua[b, j])) < min(F(1), ps / qs)
            assert bool(res["accept"][b, j]) == want


def test_data_faults_and_flags():
    rng = np.random.default_rng(25)
    B, G, V = 6, 3, 16
    zt = rng.normal(0, 1, (B, G + 1, V)).astype(np.float32)
    zd = rng.normal(0, 1, (B, G, V)).astype(np.float32)
    ids = rng.integers(0, V, (B, G)).astype(np.int32)
    zt[0, 1, 4] = np.nan                 # NaN in a verified target row
    zd[1, 2, :] = -np.inf                # an all -inf draft row
    ids[2, 0] = V                        # id out of range
    zd[3, 0, ids[3, 0]] = -np.inf        # q(x) = 0 at the draft
    zt[4, G, 0] = np.inf                 # bad bonus row (only matters if the bonus is drawn)
    ua = np.zeros((B, G), np.float32)
    ua[3, 0] = 0.5
    us = np.full((B, G + 1), 0.5, np.float32)
    zd[4] = zt[4, :G]                    # q = p on sequence 4 so that it reaches the bonus
    res = oracle.verify_dense(zt, zd, ids, ua, us, 1.0)
    f = res["flags"]
    assert f[0] & oracle.FLAG_NONFINITE and res["n_accepted"][0] == -1 and res["out_token"][0] == -1
    assert np.isnan(res["p_draft"][0]).all() and not res["accept"][0].any()
    assert f[1] & oracle.FLAG_NONFINITE and res["n_accepted"][1] == -1
    assert f[2] & oracle.FLAG_ID_RANGE and res["n_accepted"][2] == -1
    assert f[3] == oracle.FLAG_Q_ZERO and res["accept"][3, 0] == 0 and res["n_accepted"][3] == 0
    assert f[4] == oracle.FLAG_NONFINITE and res["n_accepted"][4] == G and res["out_token"][4] == -1
    assert f[5] == 0
    # bad start / bad order
    r2 = oracle.verify_dense(zt[5:], zd[5:], ids[5:], ua[5:], us[5:], 1.0, start=np.array([G + 1]))
    assert r2["flags"][0] & oracle.FLAG_ID_RANGE and r2["n_accepted"][0] == -1
    r3 = oracle.verify_dense(zt[5:], zd[5:], ids[5:], ua[5:], us[5:], 1.0, order=np.array([[0, 0, 1]]))
    assert r3["flags"][0] & oracle.FLAG_ID_RANGE


def test_sparse_empty_residual_falls_back_to_p():
    p_ids = np.array([[[1, 2], [3, 4]]], np.int32)
    p_probs = np.array([[[0.25, 0.25], [0.5, 0.5]]], np.float32)
    q_ids = np.array([[[1, 2]]], np.int32)
    q_probs = np.array([[[0.5, 0.5]]], np.float32)            # q >= p on p's whole support
    res = oracle.verify_sparse(p_ids, p_probs, q_ids, q_probs, np.array([[2]], np.int32),
                               np.array([[0.9]], np.float32), np.array([[0.75, 0.0]], np.float32))
    assert res["accept"][0, 0] == 0
    assert res["flags"][0] == oracle.FLAG_EMPTY_RESIDUAL
    assert res["out_token"][0] == 2                            # p fallback: CDF (0.25, 0.5), t = 0.375 -> slot 1
    np.testing.assert_allclose(res["correction_probs"][0, 0], [0.5, 0.5])


# ----------------------------------------------------------------------------------------------------------------------
# Hand-derived golden cases
# ----------------------------------------------------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["dense"], ids=lambda c: c["name"])
def test_golden_dense(case):
    scale = case.get("logit_scale", 1.0)
    zt = (scale * np.log(np.array(case["p"]))).astype(np.float32)[None]
    zd = (scale * np.log(np.array(case["q"]))).astype(np.float32)[None]
    res = oracle.verify_dense(zt, zd, np.array([case["draft_ids"]], np.int32), np.array([case["u_accept"]], np.float32),
                              np.array([case["u_sample"]], np.float32), case["T"])
    np.testing.assert_array_equal(res["accept"][0], case["accept"])
    assert res["n_accepted"][0] == case["n_accepted"] and res["out_token"][0] == case["out_token"]
    if "p_draft" in case:
        np.testing.assert_allclose(res["p_draft"][0], case["p_draft"], rtol=1e-6)
        np.testing.assert_allclose(res["q_draft"][0], case["q_draft"], rtol=1e-6)


@pytest.mark.parametrize("case", _golden()["onehot"], ids=lambda c: c["name"])
def test_golden_onehot(case):
    zt = np.log(np.array(case["p"])).astype(np.float32)[None]
    res = oracle.verify_onehot(zt, np.array([case["draft_ids"]], np.int32), np.array([case["u_accept"]], np.float32),
                               np.array([case["u_sample"]], np.float32), case["T"])
    np.testing.assert_array_equal(res["accept"][0], case["accept"])
    assert res["n_accepted"][0] == case["n_accepted"] and res["out_token"][0] == case["out_token"]


@pytest.mark.parametrize("case", _golden()["sparse"], ids=lambda c: c["name"])
def test_golden_sparse(case):
    res = oracle.verify_sparse(np.array([case["p_ids"]], np.int32), np.array([case["p_probs"]], np.float32),
                               np.array([case["q_ids"]], np.int32), np.array([case["q_probs"]], np.float32),
                               np.array([case["spec_ids"]], np.int32), np.array([case["u_accept"]], np.float32),
                               np.array([case["u_sample"]], np.float32))
    np.testing.assert_array_equal(res["accept"][0], case["accept"])
    assert res["n_accepted"][0] == case["n_accepted"] and res["out_token"][0] == case["out_token"]
    if "flags" in case:
        assert res["flags"][0] == case["flags"]
    if "p_spec" in case:
        np.testing.assert_array_equal(res["p_spec"][0], case["p_spec"])
        np.testing.assert_array_equal(res["q_spec"][0], case["q_spec"])
    if "correction_probs" in case:
        np.testing.assert_allclose(res["correction_probs"][0], case["correction_probs"], rtol=1e-15)


def window_golden_inputs(case):
    zt = np.log(np.array(case["p"])).astype(np.float32)[None]
    zd = np.log(np.array(case["q"])).astype(np.float32)[None]
    ua = np.array([[r["u_accept"]] for r in case["rounds"]], np.float32)
    us = np.array([[r["u_sample"]] for r in case["rounds"]], np.float32)
    return zt, zd, np.array([case["draft_ids"]], np.int32), ua, us, np.array([case["order"]], np.int32)


@pytest.mark.parametrize("case", _golden()["window"], ids=lambda c: c["name"][:40])
def test_golden_window_rounds(case):
    zt, zd, ids, ua, us, order = window_golden_inputs(case)
    res = oracle.verify_windows(zt, zd, ids, ua, us, case["T"], order=order)
    assert len(res) == len(case["rounds"])
    for r, (got, want) in enumerate(zip(res, case["rounds"])):
        np.testing.assert_array_equal(got["accept"][0], want["accept"], err_msg=f"round {r}")
        assert got["n_accepted"][0] == want["n_accepted"], f"round {r}"
        assert got["out_token"][0] == want["out_token"], f"round {r}"
        assert got["start_out"][0] == want["start_out"], f"round {r}"
        np.testing.assert_allclose(got["p_draft"][0], want["p_draft"], rtol=1e-6, atol=1e-12)
        np.testing.assert_allclose(got["q_draft"][0], want["q_draft"], rtol=1e-6, atol=1e-12)


# ----------------------------------------------------------------------------------------------------------------------
# The pins catch plausible mistakes (planted in the oracle, on the CPU)
# ----------------------------------------------------------------------------------------------------------------------

def _run_pins():
    """Run the law pin and the golden pins; return how many of them fail."""
    failures = 0
    checks = [lambda: test_exact_law_dense_matches_leviathan_closed_form(1.0, 0),
              lambda: test_exact_law_onehot_matches_closed_form()]
    checks += [lambda c=c: test_golden_dense(c) for c in _golden()["dense"]]
    checks += [lambda c=c: test_golden_onehot(c) for c in _golden()["onehot"]]
    for chk in checks:
        try:
            chk()
        except AssertionError:
            failures += 1
    return failures


@pytest.mark.parametrize("mutation", ["swapped_residual", "ratio_inverted", "reversed_cdf_order", "non_strict_test",
                                      "draw_distribution_reversed"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    assert _run_pins() == 0
    if mutation == "swapped_residual":
        monkeypatch.setattr(ov, "residual", lambda p, q: np.maximum(q - p, 0.0))
    elif mutation == "ratio_inverted":
        real = ov.accept_test
        monkeypatch.setattr(ov, "accept_test", lambda u, ratio: real(u, np.where(ratio > 0, 1.0 / ratio, 0.0)))
    elif mutation == "reversed_cdf_order":
        real_icdf = ov.inverse_cdf

        def rev(r, t):
            idx, m = real_icdf(np.atleast_2d(r)[:, ::-1], t)
            return np.atleast_2d(r).shape[-1] - 1 - idx, m
        monkeypatch.setattr(ov, "inverse_cdf", rev)
    elif mutation == "non_strict_test":
        monkeypatch.setattr(ov, "accept_test", lambda u, ratio: u <= np.minimum(1.0, ratio))
        monkeypatch.setattr(ov, "accept_test_exact", lambda u, p, q: (q > 0) & (u * q <= p))
    elif mutation == "draw_distribution_reversed":
        real_softmax = ov.softmax

        def sm(a):
            return real_softmax(a[..., ::-1]) if a.ndim == 2 else real_softmax(a)
        monkeypatch.setattr(ov, "softmax", sm)
    failures = _run_pins()
    if mutation == "non_strict_test":
        # a tie u == ratio has probability zero, so only an exact tie case can see it: the sparse golden tie
        with pytest.raises(AssertionError):
            test_golden_sparse(_golden()["sparse"][1])
    else:
        assert failures > 0
