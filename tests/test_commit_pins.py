"""Pins of the confidence-threshold commit oracle to what the page and the mathematics fix, independent of the
oracle's own code.

- hand-derived cases: slot probabilities set through log-weights, so that each slot's confidence is a known fraction
  (0.8, 0.6, 0.5 exactly, ...); the threshold, the forced commit of the most confident slot when none reaches it,
  ties at the threshold (reached) and between slots (the lower slot), masks, faults;
- library routines: scipy's softmax for the confidence, numpy's argmax for the token;
- invariants on random blocks: the commit set is the masked slots at or above tau, or else the single most confident
  one; raising tau never adds a slot beyond that forced one.
"""
import numpy as np
import pytest
from scipy import special

from oracle import commit as oc
from oracle.verify import FLAG_NONFINITE


def _logw(rows):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(rows, np.float64)).astype(np.float32)


# slot confidences 0.8, 0.4, 0.6, 0.25 (weights out of 10, 10, 10, 4); argmax ids 0, 3, 1, 2
BLOCK = [[8, 1, 1, 0], [3, 2, 1, 4], [2, 6, 1, 1], [1, 1, 1, 1]]


@pytest.mark.parametrize("tau,commit,n", [
    (0.5, [1, 0, 1, 0], 2),            # 0.8 and 0.6 reach 0.5
    (0.55, [1, 0, 1, 0], 2),
    (0.7, [1, 0, 0, 0], 1),
    (0.9, [1, 0, 0, 0], 1),            # none reaches: the most confident slot is forced
    (0.0, [1, 1, 1, 1], 4),
    (0.25, [1, 1, 1, 1], 4),           # 1/4 is exact in float32 and float64
])
def test_hand_block(tau, commit, n):
    z = _logw(BLOCK)[None]
    out = oc.confidence_commit(z, "f32", tau)
    assert out["commit"][0].tolist() == commit
    assert int(out["n_commit"][0]) == n
    assert out["token"][0].tolist() == [t if c else -1 for t, c in zip([0, 3, 1, 0], commit)]
    np.testing.assert_allclose(out["confidence"][0], [0.8, 0.4, 0.6, 0.25], rtol=1e-6)


def test_forced_commit_ties_go_to_the_lower_slot_and_masks_are_respected():
    z = _logw([[1, 1, 0, 0], [1, 1, 0, 0], [9, 1, 0, 0], [1, 3, 0, 0]])[None]   # conf 0.5, 0.5, 0.9, 0.75
    masked = np.array([[True, True, False, True]])
    out = oc.confidence_commit(z, "f32", 0.95, masked)
    assert out["commit"][0].tolist() == [0, 0, 0, 1]                              # 0.75 is the best masked slot
    out = oc.confidence_commit(z, "f32", 0.95, np.array([[True, True, False, False]]))
    assert out["commit"][0].tolist() == [1, 0, 0, 0] and out["token"][0, 0] == 0  # equal 0.5: the lower slot
    out = oc.confidence_commit(z, "f32", 0.5, np.array([[True, True, False, False]]))
    assert out["commit"][0].tolist() == [1, 1, 0, 0]                              # 0.5 reaches 0.5 exactly
    out = oc.confidence_commit(z, "f32", 0.5, np.zeros((1, 4), bool))
    assert out["n_commit"][0] == 0 and (out["token"][0] == -1).all()


def test_faults_only_in_masked_slots():
    z = _logw(BLOCK)[None].repeat(3, 0)
    z[0, 1, 2] = np.nan                     # masked: fault
    z[1, 2, :] = -np.inf                    # masked, all -inf: fault
    z[2, 3, 0] = np.inf                     # not masked: ignored
    masked = np.ones((3, 4), bool)
    masked[2, 3] = False
    out = oc.confidence_commit(z, "f32", 0.5, masked)
    assert out["flags"].tolist() == [FLAG_NONFINITE, FLAG_NONFINITE, 0]
    assert out["n_commit"].tolist() == [-1, -1, 2]
    assert (out["commit"][:2] == 0).all()


@pytest.mark.parametrize("seed", range(3))
def test_library_and_invariants(seed):
    rng = np.random.default_rng(seed)
    B, W, V = 30, 8, 200
    z = rng.normal(0, 1.0 + 2.0 * rng.random((B, W, 1)), size=(B, W, V)).astype(np.float32)
    z[:, :, :3] = np.round(z[:, :, :3])      # some exact ties at the top
    masked = rng.random((B, W)) < 0.7
    p = special.softmax(z.astype(np.float64), axis=-1)
    conf = p.max(-1)
    tok = np.argmax(z, axis=-1)
    prev = None
    for tau in (0.0, 0.05, 0.1, 0.2, 0.4, 0.8, 1.0):
        out = oc.confidence_commit(z, "f32", tau, masked)
        tau32 = float(np.float32(tau))
        for b in range(B):
            js = np.flatnonzero(masked[b])
            if js.size == 0:
                assert out["n_commit"][b] == 0
                continue
            np.testing.assert_allclose(out["confidence"][b, js], conf[b, js], rtol=1e-12)
            want = masked[b] & (conf[b] >= tau32)
            if not want.any():
                want = np.zeros(W, bool)
                want[js[np.argmax(conf[b, js])]] = True
            assert out["commit"][b].astype(bool).tolist() == want.tolist()
            assert out["token"][b].tolist() == np.where(want, tok[b], -1).tolist()
        if prev is not None:
            grew = (out["commit"] > prev) & ~(out["n_commit"] == 1)[:, None]
            assert not grew.any()
        prev = out["commit"]
