"""Plain float64 CPU oracle of the top-k / top-p support builder: dense logit rows become sparse (ids, probs)
supports, the input of the sparse verifier.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg import this module.
The HIP library never calls it, and it imports nothing from the HIP package: the two share no code.

What it follows (pages cited by title and section):
- "Uno: the draft model was already inside the target model", section "The speedup, without the 'up to'": the
  throughput test samples at temperature 1 with top-p 0.95 and top-k 50. Section "What 'lossless' actually has to
  mean" of the same page prints the engine's sparse verify routine, which takes p and q as (ids, probs) supports.
- DFlash/DFlash2 guide, section 9, Q3: under temperature, top-p or top-k sampling the logits are divided by the
  temperature before the probabilities are formed.

Readings where the pages leave the procedure open (they name the parameters only; each is repeated in the design
notes):
- the usual sampler order: temperature, then top-k, then top-p on what top-k left;
- top-k keeps the k largest logits, ties broken towards the lower id; the order by logit is the order by
  probability at any T > 0, so the selection does not depend on T;
- top-p works on the top-k distribution renormalised over its k entries: in descending order (logit, then lower
  id first), slot j is kept when j = 0 or the cumulative probability of slots 0..j-1 is below top_p, i.e. the
  shortest prefix whose mass reaches top_p, the token that crosses the threshold included;
- output: the k ids in that order, always (top-p only zeroes probabilities); probs of the kept slots, zero beyond
  them; with ``renorm`` the kept probabilities are renormalised to sum to 1, without it they are the full-vocabulary
  softmax probabilities (their sum is the kept mass, below 1);
- a row with a NaN or +inf logit, or with every logit -inf, is a data fault: flag NONFINITE, ids -1, probs NaN,
  count 0. Rows with fewer than k finite logits keep -inf entries (probability 0) among their k ids.
The count is an integer that float64 arithmetic decides (cumulative sums compared with top_p); the oracle and the
GPU both take that decision in float64, and ``margin`` gives the distance of the nearest cumulative sum to top_p so
that a comparison can tell near-ties from real differences.
"""
from __future__ import annotations

import numpy as np

from .verify import FLAG_NONFINITE, widen


def topk_order(z: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest entries of one row: descending value, equal values by ascending id."""
    V = z.shape[0]
    ids = np.arange(V)
    # lexsort sorts by its last key first: -z ascending (z descending), then the id ascending
    return np.lexsort((ids, -z))[:k]


def build_support(logits, dtype: str, k: int, top_p: float, temperature: float = 1.0, renorm: bool = True):
    """Top-k / top-p supports of every row of ``logits`` ([..., V], float32 values or bfloat16 bit patterns).

    Returns a dict: ``ids`` [..., k] int32, ``probs`` [..., k] float32, ``count`` [...] int32 (kept slots),
    ``flags`` [...] uint32, ``margin`` [...] float64 (min over slots 0..k-2 of |C_j - top_p|, C the cumulative
    top-k probabilities; inf when k = 1).
    """
    z_all = widen(logits, dtype)
    lead = z_all.shape[:-1]
    V = z_all.shape[-1]
    if not (1 <= k <= V):
        raise ValueError("k must lie in [1, V]")
    if not (0.0 < top_p <= 1.0):
        raise ValueError("top_p must lie in (0, 1]")
    if not (np.isfinite(temperature) and temperature > 0):
        raise ValueError("temperature must be finite and positive")
    T = float(np.float32(temperature))         # both arrive as float32 values (the C call's argument types)
    p_cut = float(np.float32(top_p))
    rows = z_all.reshape(-1, V)
    n = rows.shape[0]
    ids = np.full((n, k), -1, np.int32)
    probs = np.full((n, k), np.nan, np.float32)
    count = np.zeros(n, np.int32)
    flags = np.zeros(n, np.uint32)
    margin = np.full(n, np.inf)
    for r in range(n):
        z = rows[r]
        if np.isnan(z).any() or (z == np.inf).any() or (z == -np.inf).all():
            flags[r] = FLAG_NONFINITE
            continue
        order = topk_order(z, k)
        a = z[order] / T                       # descending; a[0] is the row's maximum and finite
        e = np.exp(a - a[0])                   # unnormalised top-k probabilities (0 for -inf logits)
        cum = np.cumsum(e)                     # sequential sums in slot order
        C = cum / cum[-1]                      # cumulative top-k probabilities
        m = 1 + int(np.count_nonzero(C[:-1] < p_cut))
        if k > 1:
            margin[r] = float(np.min(np.abs(C[:-1] - p_cut)))
        out = np.zeros(k, np.float64)
        if renorm:
            out[:m] = e[:m] / cum[m - 1]
        else:
            full = np.exp(z / T - a[0])        # the full-vocabulary softmax, normalised by the whole row
            out[:m] = full[order[:m]] / full.sum()
        ids[r] = order.astype(np.int32)
        probs[r] = out.astype(np.float32)
        count[r] = m
    return dict(ids=ids.reshape(*lead, k), probs=probs.reshape(*lead, k), count=count.reshape(lead),
                flags=flags.reshape(lead), margin=margin.reshape(lead))
