"""Plain float64 CPU oracle of the confidence-threshold commit of block diffusion.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg import this module.
The HIP library never calls it, and it imports nothing from the HIP package: the two share no code.

What it follows (pages cited by title and section): the SDAR-style block diffusion page, section 5 "Decoding
timeline": every denoising pass gives a full distribution over the vocabulary at each masked slot of the block; the
slots whose confidence reaches a threshold tau are committed, and at least the most confident proposal is always
committed so that every pass makes progress; the committed token of a slot is its most likely one; section 2 states
the same rule in words (the most confident proposals are kept, the rest stay masked).

Readings where the page leaves a step open (each is repeated in the design notes):
- confidence = the largest probability of the slot's softmax (temperature 1: the page names none), its token the
  argmax, equal maxima going to the lowest id;
- "reaches the threshold": confidence >= tau, decided in float64;
- when no masked slot reaches tau, the single most confident masked slot is committed (equal confidences: the lowest
  slot index);
- slots that are not masked are neither read nor committed; a block with no masked slot commits nothing;
- a NaN or +inf logit, or a row that is all -inf, in a masked slot is a data fault of the block: flag NONFINITE,
  nothing committed, count -1.
The commit decisions compare float64 confidences with tau and with each other; ``margin`` gives, per block, the
distance of the nearest confidence to tau and the gap between the two most confident masked slots, so that a
comparison can tell near-ties from real differences.
"""
from __future__ import annotations

import numpy as np

from .verify import FLAG_NONFINITE, _bad_rows, widen


def slot_confidence(z: np.ndarray):
    """(argmax, confidence) of each row of logits z [..., V] (float64): the lowest id among the maxima and the
    largest softmax probability, 1 / sum(exp(z - max))."""
    a = np.argmax(z, axis=-1)
    m = np.take_along_axis(z, a[..., None], axis=-1)
    with np.errstate(invalid="ignore"):
        s = np.exp(z - m).sum(-1)
    return a, 1.0 / s


def confidence_commit(logits, dtype: str, tau: float, masked=None):
    """Confidence-threshold commit over B blocks of W slots.

    logits [B, W, V] (float32 values or bfloat16 bit patterns); masked [B, W] bool (default all); tau in [0, 1].
    Returns a dict: commit [B, W] uint8, token [B, W] int32 (-1 where not committed), confidence [B, W] float64 (NaN
    where not read), n_commit [B] int32, flags [B] uint32, margin [B] float64.
    """
    z_all = widen(logits, dtype)
    B, W, V = z_all.shape
    tau = float(np.float32(tau))                 # the C call receives tau as a float32 value
    masked = np.ones((B, W), bool) if masked is None else np.asarray(masked, bool)
    out = dict(commit=np.zeros((B, W), np.uint8), token=np.full((B, W), -1, np.int32),
               confidence=np.full((B, W), np.nan), n_commit=np.zeros(B, np.int32), flags=np.zeros(B, np.uint32),
               margin=np.full(B, np.inf))
    for b in range(B):
        js = np.flatnonzero(masked[b])
        if js.size == 0:
            continue
        z = z_all[b, js]
        if _bad_rows(z).any():
            out["flags"][b] = FLAG_NONFINITE
            out["n_commit"][b] = -1
            continue
        a, conf = slot_confidence(z)
        out["confidence"][b, js] = conf
        keep = conf >= tau
        if not keep.any():
            keep[int(np.argmax(conf))] = True     # the most confident slot, lowest index on ties
        out["commit"][b, js] = keep.astype(np.uint8)
        out["token"][b, js] = np.where(keep, a, -1)
        out["n_commit"][b] = int(keep.sum())
        srt = np.sort(conf)[::-1]
        gap = srt[0] - srt[1] if srt.size > 1 else np.inf
        out["margin"][b] = min(float(np.min(np.abs(conf - tau))), float(gap))
    return out
