"""Pins of the greedy (T = 0) verification oracle to what the pages and the mathematics fix, independent of the
oracle's own code.

- hand-derived cases (tests/golden/greedy_cases.json): ties, start, order, bonus on and off, faults in verified,
  unverified and bonus rows, signed zeros;
- the zero-temperature limit of the sampled rule: with a greedy drafter (q one-hot at the draft) and a target whose
  maximum leads the runner-up by a wide margin, the sampled one-hot oracle at a tiny temperature has p exactly
  one-hot, so its accept test and its residual and bonus draws become deterministic and must equal greedy
  verification for any uniforms;
- constructed chains: drafts that copy the target argmax (found by a sort, not by argmax) for the first m slots and
  then differ must give n = m and the argmax of slot m;
- first_argmax against a stable sort on data full of ties.
"""
import json
import os

import numpy as np
import pytest

from oracle import greedy as og
from oracle import verify as ov
from oracle.verify import FLAG_ID_RANGE, FLAG_NONFINITE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "greedy_cases.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _sort_argmax(z):
    """Lowest index among the maxima of each row, by a stable sort on the negated values (a different mechanism
    from numpy's argmax)."""
    z = np.asarray(z, np.float64)
    flat = z.reshape(-1, z.shape[-1])
    out = np.array([np.argsort(-r, kind="stable")[0] for r in flat])
    return out.reshape(z.shape[:-1])


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_golden_greedy(case):
    g = _golden()
    tgt = [list(r) for r in g["target"]]
    for i, row in case.get("rows", {}).items():
        tgt[int(i)] = row
    target = np.asarray([[float(v) for v in r] for r in tgt], np.float32)[None]      # [1, 4, 4]
    kw = dict(bonus=case["bonus"], dtype="f32")
    if "start" in case:
        kw["start"] = np.array([case["start"]])
    if "order" in case:
        kw["order"] = np.array([case["order"]])
    if not case["bonus"]:
        target = target[:, :3]
    out = og.verify_greedy(target, np.array([case["draft"]]), **kw)
    e = case["expect"]
    assert out["accept"][0].tolist() == e["accept"]
    assert int(out["n_accepted"][0]) == e["n"]
    assert int(out["out_token"][0]) == e["token"]
    assert int(out["start_out"][0]) == e["start_out"]
    assert int(out["first_reject"][0]) == e["k"]
    assert int(out["flags"][0]) == e["flags"]
    assert int(out["resampled"][0]) == e["kind"]


def _separated(rng, B, R, V, gap=2.0):
    """Logits whose maximum exceeds every other entry by at least ``gap``."""
    z = rng.normal(0.0, 1.0, size=(B, R, V))
    am = rng.integers(0, V, size=(B, R))
    z[np.arange(B)[:, None], np.arange(R)[None, :], am] = z.max(-1) + gap
    return z.astype(np.float32), am


@pytest.mark.parametrize("bonus", [0, 1])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_zero_temperature_limit_of_sampled_rule(seed, bonus):
    rng = np.random.default_rng(seed)
    B, G, V = 40, 6, 37
    z, am = _separated(rng, B, G + bonus, V)
    # drafts: the argmax with probability 0.8, otherwise another id
    draft = np.where(rng.random((B, G)) < 0.8, am[:, :G], (am[:, :G] + rng.integers(1, V, (B, G))) % V)
    start = rng.integers(0, G + 1, size=B)
    order = np.array([rng.permutation(G) for _ in range(B)])
    ua = rng.random((B, G)).astype(np.float32)
    us = rng.random((B, G + 1)).astype(np.float32)
    ref = ov.verify_onehot(z, draft, ua, us, 1e-3, bonus=bonus, start=start, order=order, dtype="f32")
    got = og.verify_greedy(z, draft, bonus=bonus, start=start, order=order, dtype="f32")
    for key in ("accept", "n_accepted", "out_token", "first_reject", "start_out", "flags", "resampled"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)


def test_zero_temperature_limit_bf16():
    rng = np.random.default_rng(7)
    B, G, V = 30, 5, 29
    z, am = _separated(rng, B, G + 1, V, gap=4.0)
    bits = (z.view(np.uint32) >> 16).astype(np.uint16)         # truncation keeps the 4.0 gap at these magnitudes
    zb = (bits.astype(np.uint32) << 16).view(np.float32)
    assert (_sort_argmax(zb) == am).all()
    draft = np.where(rng.random((B, G)) < 0.7, am[:, :G], (am[:, :G] + 1) % V)
    ua = rng.random((B, G)).astype(np.float32)
    us = rng.random((B, G + 1)).astype(np.float32)
    ref = ov.verify_onehot(bits, draft, ua, us, 1e-3, dtype="bf16")
    got = og.verify_greedy(bits, draft, dtype="bf16")
    for key in ("accept", "n_accepted", "out_token", "first_reject", "start_out", "flags", "resampled"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)


@pytest.mark.parametrize("seed", range(4))
def test_constructed_chains(seed):
    rng = np.random.default_rng(100 + seed)
    B, G, V = 64, 9, 50
    # integer-valued logits: many ties, broken towards the lowest id
    z = rng.integers(-3, 4, size=(B, G + 1, V)).astype(np.float32)
    am = _sort_argmax(z)
    m = rng.integers(0, G + 1, size=B)                        # drafts copy the argmax for slots < m
    draft = am[:, :G].copy()
    for b in range(B):
        if m[b] < G:
            draft[b, m[b]] = (am[b, m[b]] + 1 + rng.integers(0, V - 1)) % V
    got = og.verify_greedy(z, draft, dtype="f32")
    np.testing.assert_array_equal(got["n_accepted"], m)
    exp_tok = np.where(m < G, am[np.arange(B), np.minimum(m, G - 1)], am[:, G])
    np.testing.assert_array_equal(got["out_token"], exp_tok)
    np.testing.assert_array_equal(got["resampled"], np.where(m < G, 1, 2))
    np.testing.assert_array_equal(got["start_out"], np.minimum(G, m + 1))
    np.testing.assert_array_equal(got["argmax"], am[:, :G])
    # the accepted prefix plus the emitted token is what greedy decoding of the target gives there
    for b in range(B):
        seq = list(draft[b, :m[b]]) + [got["out_token"][b]]
        assert seq == list(am[b, :m[b] + 1]) if m[b] < G else seq == list(am[b, :G + 1])


def test_first_argmax_matches_stable_sort_on_ties():
    rng = np.random.default_rng(5)
    z = rng.integers(0, 3, size=(200, 17)).astype(np.float64)
    np.testing.assert_array_equal(og.first_argmax(z), _sort_argmax(z))
    z[:, :] = 1.0
    assert (og.first_argmax(z) == 0).all()


def test_fault_flags_are_fatal_only_on_examined_rows():
    rng = np.random.default_rng(9)
    B, G, V = 8, 4, 16
    z, am = _separated(rng, B, G + 1, V)
    draft = am[:, :G].copy()
    draft[:, 1] = (draft[:, 1] + 1) % V                       # every sequence rejects at slot 1
    z[0, 3, 2] = np.nan                                      # verified row after the rejection: fatal
    z[1, 4, 0] = np.nan                                      # bonus row, not taken: no flag
    z[2, 0, :] = -np.inf                                     # slot 0 unverified with start = 1: not examined
    draft[3, 2] = V                                          # id out of range in a verified slot: fatal
    start = np.zeros(B, np.int64)
    start[2] = 1
    got = og.verify_greedy(z, draft, start=start, dtype="f32")
    assert got["flags"][0] == FLAG_NONFINITE and got["n_accepted"][0] == -1
    assert got["flags"][1] == 0 and got["n_accepted"][1] == 1 and got["out_token"][1] == am[1, 1]
    assert got["flags"][2] == 0 and got["n_accepted"][2] == 0 and got["out_token"][2] == am[2, 1]
    assert got["flags"][3] == FLAG_ID_RANGE and got["out_token"][3] == -1
