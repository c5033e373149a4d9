"""Plain float64 CPU oracle of greedy (T = 0) verification.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg import this module.
The HIP library never calls it, and it imports nothing from the HIP package: the two share no code.

What it follows (pages cited by title and section):
- DFlash/DFlash2 guide, section 4.4 "Mathematical Losslessness Guarantee": under greedy decoding (T = 0) a drafted
  token is accepted exactly when it is the target's most likely token at its position (the formula itself is lost
  in the page's text; the prose around it and the serving example of section 7, whose sampling parameters set
  temperature 0 and call it the greedy verification mode, leave this as the only reading). The block is truncated
  at the first rejected position, as in the sampled case.
- DFlash/DFlash2 guide, section 2 "Speculative Decoding Speedup Formulation": a cycle yields between 1 and gamma + 1
  tokens, the last one from the target.

Readings where the pages leave a step open (each is repeated in the design notes):
- "most likely" is the argmax of the target logits (the order by probability is the order by logit); equal maxima go
  to the lowest token id;
- the token emitted at the first mismatch is the target's argmax there (the T -> 0 limit of the residual draw, whose
  distribution collapses onto that argmax); when every verified draft matches, the bonus token is the argmax of
  target row gamma;
- start, order, bonus, the flags and the fault rules are those of the sampled dense verifier: every verified row is
  examined, a NaN or +inf logit or a row that is all -inf in a verified row is a data fault of the sequence, and the
  bonus row is examined only when the bonus token is taken from it. No uniforms and no temperature are involved.
"""
from __future__ import annotations

import numpy as np

from .verify import FLAG_ID_RANGE, FLAG_NONFINITE, _bad_rows, widen


def first_argmax(z: np.ndarray) -> np.ndarray:
    """Index of the largest entry along the last axis; equal maxima go to the lowest index (numpy's rule)."""
    return np.argmax(z, axis=-1)


def verify_greedy(target, draft_ids, *, bonus=1, start=None, order=None, dtype="f32"):
    """Greedy verification of B blocks of gamma drafted ids against target logits.

    target    [B, gamma + bonus, V] logits (float32 values or bfloat16 bit patterns); row gamma only for the bonus
    draft_ids [B, gamma] int (by storage row); start [B] first slot to verify (default 0);
    order     [B, gamma] slot -> storage row (default identity)

    Returns a dict of numpy arrays: accept (uint8, by storage row), n_accepted, out_token, flags, start_out,
    first_reject (slot k, or gamma), resampled (1: argmax at the first mismatch, 2: bonus argmax), argmax (int64,
    by storage row, -1 where the row was not verified).
    """
    draft_ids = np.asarray(draft_ids)
    B, G = draft_ids.shape
    start = np.zeros(B, np.int64) if start is None else np.asarray(start, dtype=np.int64)
    order = np.tile(np.arange(G), (B, 1)) if order is None else np.asarray(order, dtype=np.int64)
    tgt = np.asarray(target)
    V = tgt.shape[-1]

    out = dict(accept=np.zeros((B, G), np.uint8), n_accepted=np.zeros(B, np.int32),
               out_token=np.full(B, -1, np.int32), flags=np.zeros(B, np.uint32), start_out=np.zeros(B, np.int32),
               first_reject=np.full(B, G, np.int32), resampled=np.zeros(B, np.int8),
               argmax=np.full((B, G), -1, np.int64))
    for b in range(B):
        st = int(start[b])
        od = order[b]
        bad = False
        if st < 0 or st > G:
            bad = True
        if ((od < 0) | (od >= G)).any() or len(set(od.tolist())) != G:
            bad = True
        if bad:
            out["flags"][b] = FLAG_ID_RANGE
            out["n_accepted"][b] = -1
            out["start_out"][b] = st
            continue
        if st == G:                                   # finished: nothing verified, nothing emitted
            out["start_out"][b] = st
            continue
        slots = np.arange(st, G)
        rows = od[slots]
        x = draft_ids[b, rows].astype(np.int64)
        z = widen(tgt[b, rows], dtype)                # [n_verified, V], slot order
        flags = 0
        if ((x < 0) | (x >= V)).any():
            flags |= FLAG_ID_RANGE
        if _bad_rows(z).any():
            flags |= FLAG_NONFINITE
        if flags:
            out["flags"][b] = flags
            out["n_accepted"][b] = -1
            out["start_out"][b] = st
            continue
        am = first_argmax(z)
        acc = am == x
        out["argmax"][b, rows] = am
        out["accept"][b, rows] = acc.astype(np.uint8)
        miss = np.flatnonzero(~acc)
        k = st + (int(miss[0]) if miss.size else G - st)
        out["first_reject"][b] = k
        out["n_accepted"][b] = k - st
        out["start_out"][b] = min(G, k + 1)
        if k < G:
            out["out_token"][b] = am[k - st]
            out["resampled"][b] = 1
        elif bonus:
            zb = widen(tgt[b, G], dtype)
            if _bad_rows(zb[None])[0]:
                out["flags"][b] = FLAG_NONFINITE
                out["out_token"][b] = -1
            else:
                out["out_token"][b] = int(first_argmax(zb))
                out["resampled"][b] = 2
    return out
