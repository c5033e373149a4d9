"""Pins of the top-k / top-p support oracle to what the mathematics and library routines fix, independent of the
oracle's own code.

- hand-derived cases (tests/golden/support_cases.json), chosen so that a dropped renormalisation, an off-by-one at
  the threshold, a missing temperature or a wrong tie order fails one of them;
- library routines: numpy's stable argsort for the top-k order, scipy's softmax for the probabilities, numpy's
  argmax (first maximum) for k = 1 or a vanishing top_p; k = V with top_p = 1 keeps the whole softmax;
- invariants on random rows: the count is the shortest prefix whose top-k mass reaches top_p, recomputed with
  scipy; the count never decreases as the temperature rises or top_p grows; the kept renormalised probabilities
  sum to 1 and their ratios are exp((z_i - z_j) / T).
"""
import json
import os

import numpy as np
import pytest
from scipy import special

from oracle import support as osup
from oracle.verify import FLAG_NONFINITE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "support_cases.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _row(case):
    if "log_weights" in case:
        return np.log(np.asarray(case["log_weights"], np.float64)).astype(np.float32)
    return np.asarray([float(v) for v in case["logits"]], np.float32)


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
@pytest.mark.parametrize("renorm", [True, False])
def test_golden_supports(case, renorm):
    z = _row(case)[None, :]
    out = osup.build_support(z, "f32", case["k"], case["top_p"], case["T"], renorm=renorm)
    assert out["flags"][0] == 0
    assert out["ids"][0].tolist() == case["ids"]
    assert int(out["count"][0]) == case["count"]
    exp = np.asarray(case["probs_renorm" if renorm else "probs_full"])
    np.testing.assert_allclose(out["probs"][0], exp, rtol=1e-6, atol=0)


@pytest.mark.parametrize("case", _golden()["faults"], ids=lambda c: c["name"])
def test_golden_faults(case):
    z = _row(case)[None, :]
    out = osup.build_support(z, "f32", case["k"], 0.9, 1.0)
    assert out["flags"][0] == FLAG_NONFINITE
    assert int(out["count"][0]) == 0
    assert (out["ids"][0] == -1).all() and np.isnan(out["probs"][0]).all()


def _random_rows(seed, n, V, scale=3.0, dtype="f32"):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, scale, (n, V)).astype(np.float32)
    z += (-1.1 * np.log1p(np.arange(V))).astype(np.float32)       # a Zipf-like bias over the id
    if dtype == "bf16":
        return (z.view(np.uint32) >> 16).astype(np.uint16)
    return z


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk_order_matches_stable_argsort(dtype):
    z = _random_rows(3, 6, 4099, dtype=dtype)
    if dtype == "bf16":
        zf = (z.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        zf = z.astype(np.float64)
    out = osup.build_support(z, dtype, 50, 1.0, 1.0)     # bf16 rows hold many exact ties
    for r in range(z.shape[0]):
        ref = np.argsort(-zf[r], kind="stable")[:50]
        assert out["ids"][r].tolist() == ref.tolist()


def test_ties_broken_towards_lower_id():
    V = 300
    z = np.zeros((1, V), np.float32)
    z[0, [7, 100, 250]] = 1.0
    out = osup.build_support(z, "f32", 10, 1.0, 1.0)
    assert out["ids"][0].tolist() == [7, 100, 250, 0, 1, 2, 3, 4, 5, 6]


def test_full_support_is_the_softmax():
    z = _random_rows(5, 4, 37)
    for T in (0.7, 1.0, 1.6):
        out = osup.build_support(z, "f32", 37, 1.0, T)
        T32 = float(np.float32(T))                 # the temperature is a float32 argument
        for r in range(4):
            ids = out["ids"][r]
            assert int(out["count"][r]) == 37
            ref = special.softmax(z[r].astype(np.float64) / T32)[ids]
            np.testing.assert_allclose(out["probs"][r], ref, rtol=2e-7, atol=1e-30)
            full = osup.build_support(z[r:r + 1], "f32", 37, 1.0, T, renorm=False)
            np.testing.assert_allclose(full["probs"][0], ref, rtol=2e-7, atol=1e-30)


def test_k1_and_vanishing_top_p_give_the_argmax():
    z = _random_rows(9, 8, 1000)
    z[2, 5] = z[2, 9] = z[2].max() + 1.0          # a tie at the maximum: the first one is the argmax
    for k, p in ((1, 0.95), (50, 1e-9)):
        out = osup.build_support(z, "f32", k, p, 1.0)
        assert out["count"].tolist() == [1] * 8
        assert out["ids"][:, 0].tolist() == np.argmax(z, axis=1).tolist()
        np.testing.assert_array_equal(out["probs"][:, 0], np.ones(8, np.float32))


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
@pytest.mark.parametrize("top_p", [0.3, 0.9, 0.95, 0.999])
def test_count_is_the_shortest_prefix_reaching_top_p(T, top_p):
    z = _random_rows(11, 16, 2048, scale=2.0)
    k = 64
    out = osup.build_support(z, "f32", k, top_p, T)
    p32 = float(np.float32(top_p))
    for r in range(16):
        ids = out["ids"][r]
        pk = special.softmax(z[r, ids].astype(np.float64) / T)
        C = np.cumsum(pk)
        m = int(out["count"][r])
        assert 1 <= m <= k
        if m < k:
            assert C[m - 1] >= p32 - 1e-12
        if m > 1:
            assert C[m - 2] < p32 + 1e-12
        kept = out["probs"][r, :m].astype(np.float64)
        np.testing.assert_allclose(kept.sum(), 1.0, rtol=1e-6)
        np.testing.assert_allclose(kept, pk[:m] / pk[:m].sum(), rtol=2e-7, atol=1e-30)
        assert (out["probs"][r, m:] == 0).all()


def test_count_monotone_in_temperature_and_top_p():
    z = _random_rows(13, 12, 3000)
    counts = [osup.build_support(z, "f32", 50, 0.9, T)["count"] for T in (0.25, 0.5, 1.0, 2.0, 4.0)]
    for a, b in zip(counts, counts[1:]):
        assert (a <= b).all()
    counts = [osup.build_support(z, "f32", 50, p, 1.0)["count"] for p in (0.1, 0.5, 0.9, 0.99, 1.0)]
    for a, b in zip(counts, counts[1:]):
        assert (a <= b).all()


def test_full_probs_are_the_softmax_mass():
    z = _random_rows(17, 6, 5000)
    out = osup.build_support(z, "f32", 50, 0.95, 1.0, renorm=False)
    for r in range(6):
        m = int(out["count"][r])
        ref = special.softmax(z[r].astype(np.float64))[out["ids"][r, :m]]
        np.testing.assert_allclose(out["probs"][r, :m], ref, rtol=2e-7, atol=1e-30)


def test_argument_checks():
    z = np.zeros((1, 8), np.float32)
    with pytest.raises(ValueError):
        osup.build_support(z, "f32", 9, 0.9)
    with pytest.raises(ValueError):
        osup.build_support(z, "f32", 4, 0.0)
    with pytest.raises(ValueError):
        osup.build_support(z, "f32", 4, 1.5)
    with pytest.raises(ValueError):
        osup.build_support(z, "f32", 4, 0.9, temperature=0.0)
