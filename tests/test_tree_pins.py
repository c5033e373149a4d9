"""Pins of the tree-verification oracle (oracle/tree.py) to what the rule and the mathematics fix.

- exact output law: the oracle is probed as a black box (each test's uniform and the final draw's uniform are bisected
  to their decision thresholds, and every branch of the walk is explored with its exact probability); the law of the
  emitted token sequence must equal the target's own autoregressive law, stopped after the first token that is not a
  drafted child of the node reached (the losslessness of speculative sampling, Leviathan et al., as the Uno page
  restates it in "What 'lossless' actually has to mean"), to 1e-12;
- a chain tree (one child per node) is the one-hot draft rule of the dense oracle, whose law is pinned elsewhere;
- Monte Carlo: the first emitted token of a star tree follows p_root (chi-square);
- hand-derived golden cases (tests/golden/tree_cases.json) and the fault flags.
"""
import itertools
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_cases.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _run(zt, parent, token, ua, us, T):
    return oracle.verify_tree(zt[None], parent[None], token[None], ua[None], us[None], T)


def _bisect(pred, iters=60):
    lo, hi = 0.0, 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if pred(mid):
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def probed_law(zt, parent, token, T):
    """{(accepted path, emitted final token): probability} by exploring the oracle's decisions as a black box."""
    N, V = zt.shape
    law = {}

    def uniforms(dec):
        ua = np.ones(N)                       # an undecided test gets u = 1: it fails whatever p'(x) is
        for c, u in dec.items():
            ua[c] = u
        return ua

    def walk(dec, w):
        r = _run(zt, parent, token, uniforms(dec), np.zeros(N), T)
        assert r["flags"][0] == 0
        new = [c for c in np.flatnonzero(r["tested"][0]) if c not in dec]
        if new:
            c = int(min(new))
            alpha = _bisect(lambda u: r_accept(dec, c, u))
            if alpha > 1e-15:
                walk({**dec, c: alpha / 2}, w * alpha)
            if alpha < 1 - 1e-15:
                walk({**dec, c: 1.0}, w * (1 - alpha))
            return
        stop = int(r["stop_node"][0])
        path = tuple(int(x) for x in r["path"][0][:r["n_accepted"][0]])
        ua = uniforms(dec)
        cuts = [0.0]
        for i in range(V - 1):
            def below(s, i=i):
                us = np.zeros(N)
                us[stop] = s
                return _run(zt, parent, token, ua, us, T)["out_token"][0] <= i
            cuts.append(_bisect(below))
        cuts.append(1.0)
        for tok, length in enumerate(np.diff(cuts)):
            if length > 1e-15:
                law[(path, tok)] = law.get((path, tok), 0.0) + w * length

    def r_accept(dec, c, u):
        return bool(_run(zt, parent, token, uniforms({**dec, c: u}), np.zeros(N), T)["accept"][0, c])

    walk({}, 1.0)
    return law


def closed_law(zt, parent, token, T):
    """The target's autoregressive law with the tree's stopping rule: from node u, token y has probability p_u(y);
    if y is a child token of u (its first child holding y) the sequence continues there, else it ends with y."""
    N, V = zt.shape
    p = special.softmax(zt.astype(np.float64) / np.float64(np.float32(T)), axis=-1)
    kids = [[c for c in range(1, N) if parent[c] == u] for u in range(N)]
    law = {}

    def go(u, path, w):
        first = {}
        for c in kids[u]:
            first.setdefault(int(token[c]), c)
        for y in range(V):
            if p[u, y] == 0:
                continue
            if y in first:
                go(first[y], path + (first[y],), w * p[u, y])
            else:
                law[(path, y)] = law.get((path, y), 0.0) + w * p[u, y]

    go(0, (), 1.0)
    return law


TREES = [
    # parent, token, V (token[0] unused)
    ([-1, 0, 0, 1], [0, 1, 2, 0], 3),
    ([-1, 0, 0, 0, 2, 2], [0, 3, 1, 0, 2, 1], 4),
    ([-1, 0, 1, 2, 0, 4], [0, 2, 2, 0, 1, 3], 4),             # two branches, one deep
    ([-1, 0, 0, 0, 1, 1, 4], [0, 1, 1, 2, 0, 1, 2], 3),       # a repeated sibling token
]


@pytest.mark.parametrize("idx", range(len(TREES)))
@pytest.mark.parametrize("T", [1.0, 0.6])
def test_exact_law_matches_the_target_autoregressive_law(idx, T):
    parent, token, V = TREES[idx]
    parent, token = np.array(parent), np.array(token)
    rng = np.random.default_rng(10 + idx)
    zt = rng.normal(0, 1.3, (len(parent), V)).astype(np.float32)
    law = probed_law(zt, parent, token, T)
    closed = closed_law(zt, parent, token, T)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    assert abs(sum(closed.values()) - 1.0) < 1e-12
    for key in set(law) | set(closed):
        assert abs(law.get(key, 0.0) - closed.get(key, 0.0)) < 1e-12, key


def test_chain_tree_is_the_onehot_rule():
    rng = np.random.default_rng(3)
    B, G, V = 40, 5, 12
    zt = rng.normal(0, 1.5, (B, G + 1, V)).astype(np.float32)
    d = rng.integers(0, V, (B, G)).astype(np.int32)
    d[: B // 2] = np.argmax(zt[: B // 2, :G], axis=-1)          # likely candidates: long accepted chains
    ua = rng.random((B, G)).astype(np.float32)
    us = rng.random((B, G + 1)).astype(np.float32)
    parent = np.tile(np.arange(-1, G), (B, 1))
    token = np.concatenate([np.zeros((B, 1), np.int32), d], axis=1)
    ua_t = np.concatenate([np.zeros((B, 1), np.float32), ua], axis=1)
    t = oracle.verify_tree(zt, parent, token, ua_t, us, 0.9)
    o = oracle.verify_onehot(zt, d, ua, us, 0.9)
    np.testing.assert_array_equal(t["n_accepted"], o["n_accepted"])
    np.testing.assert_array_equal(t["out_token"], o["out_token"])
    for b in range(B):
        n = o["n_accepted"][b]
        assert list(t["path"][b, :n]) == list(range(1, n + 1))
        tested = list(range(1, min(n + 1, G) + 1))
        assert list(np.flatnonzero(t["tested"][b])) == tested
        np.testing.assert_allclose(t["p_test"][b, tested], o["p_draft"][b, [s - 1 for s in tested]], rtol=1e-12)
    assert (o["n_accepted"] > 0).mean() > 0.2 and (o["n_accepted"] < G).any()


def test_monte_carlo_first_token_of_a_star_tree_follows_the_root():
    rng = np.random.default_rng(4)
    V, m, n = 6, 3, 200_000
    zt = rng.normal(0, 1.0, (m + 1, V)).astype(np.float32)
    parent = np.array([-1] + [0] * m)
    token = np.array([0, 4, 1, 4])                              # a repeated candidate among the siblings
    p0 = special.softmax(zt[0].astype(np.float64))
    B = n
    r = oracle.verify_tree(np.broadcast_to(zt, (B, m + 1, V)), np.broadcast_to(parent, (B, m + 1)),
                           np.broadcast_to(token, (B, m + 1)), rng.random((B, m + 1)), rng.random((B, m + 1)), 1.0)
    first = np.where(r["n_accepted"] > 0, token[np.maximum(r["path"][:, 0], 0)], r["out_token"])
    counts = np.bincount(first, minlength=V)
    chi2, pval = stats.chisquare(counts, p0 * B)
    assert pval > 1e-6, (counts, p0 * B)


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"][:40])
def test_golden_trees(case):
    zt = np.log(np.array(case["p"])).astype(np.float32)
    r = _run(zt, np.array(case["parent"]), np.array(case["token"]), np.array(case["u_accept"], np.float32),
             np.array(case["u_sample"], np.float32), case["T"])
    assert list(r["accept"][0]) == case["accept"]
    assert list(r["tested"][0]) == case["tested"]
    assert r["n_accepted"][0] == case["n_accepted"]
    assert list(r["path"][0][:r["n_accepted"][0]]) == case["path"]
    assert r["out_token"][0] == case["out_token"] and r["stop_node"][0] == case["stop_node"]
    want = np.array([np.nan if v is None else v for v in case["p_test"]])
    np.testing.assert_allclose(r["p_test"][0], want, rtol=1e-6, atol=1e-12)


def test_faults():
    rng = np.random.default_rng(6)
    B, N, V = 5, 4, 7
    zt = rng.normal(0, 1, (B, N, V)).astype(np.float32)
    parent = np.tile([-1, 0, 1, 1], (B, 1))
    token = rng.integers(0, V, (B, N)).astype(np.int32)
    ua = np.zeros((B, N), np.float32)             # every test passes (p'(x) > 0): the walk goes 0 -> 1 -> 2
    us = np.full((B, N), 0.5, np.float32)
    parent[1, 3] = 3                              # not an earlier node
    token[2, 2] = V                               # out of the vocabulary
    zt[3, 1, 2] = np.nan                          # a row on the walk
    zt[4, 3, :] = np.nan                          # a row off the walk (node 3 is never reached)
    r = oracle.verify_tree(zt, parent, token, ua, us, 1.0)
    assert r["flags"][0] == 0 and r["n_accepted"][0] == 2
    assert r["flags"][1] == oracle.FLAG_ID_RANGE and r["n_accepted"][1] == -1 and r["out_token"][1] == -1
    assert r["flags"][2] == oracle.FLAG_ID_RANGE
    assert r["flags"][3] == oracle.FLAG_NONFINITE and r["n_accepted"][3] == -1 and r["out_token"][3] == -1
    assert not r["accept"][3].any() and np.isnan(r["p_test"][3]).all()
    assert r["flags"][4] == 0 and r["n_accepted"][4] == 2
