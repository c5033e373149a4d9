"""Plain float64 CPU oracle of tree (multi-candidate) verification.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg import this module.
The HIP library never calls it, and it imports nothing from the HIP package: the two share no code.

What the pages give and what they leave open. They verify trees of drafted tokens: the Uno page's B = 16 tree sampler
("One backbone, two pathways", Table 2), EAGLE-2's dynamic draft trees (DFlash/DFlash2 guide, section 3) and DFlash2's
top-m candidates per position, submitted as a path or a dense verification tree (same guide, section 5.2, "Dynamic
Candidate Path Selector"). They state the acceptance rule for one candidate per position only (Uno, "What 'lossless'
actually has to mean"), including its closing remark that a greedy drafter makes q one-hot and that the rule must be
applied to that one-hot q. For several candidates this module takes the published multi-step speculative sampling of
SpecInfer (Miao et al., "SpecInfer: Accelerating Large Language Model Serving with Tree-based Speculative Inference and
Verification", ASPLOS 2024) with q one-hot at each candidate, the case of candidates chosen deterministically (top-m):

- at node u, with p = softmax(z_u / T) (the target's distribution after the path to u) and an excluded set E, empty
  when u is reached, the children of u are tested in increasing node index;
- child c with token x passes when u_accept[c] < min(1, p'(x)), p' = p with the tokens of E removed and renormalised
  (one-hot q: the ratio p'(x)/q(x) is p'(x)); a token already in E has p'(x) = 0 and fails;
- a passing child is accepted and the walk continues at it (E emptied); a failing child's token joins E
  (the residual max(p' - e_x, 0) renormalised is p' without x);
- when every child of u fails, or u has no children, one token is drawn from p' (p without E, renormalised) by inverse
  CDF at t = u_sample[u] * (its mass), in vocabulary order, and the walk ends. At a leaf E is empty and this is the
  tree's bonus token.

With distinct candidates each candidate x is emitted first with probability p(x) and every other token y with
probability p(y): the emitted sequence follows the target exactly (the Leviathan guarantee). Readings where the pages
are silent (each is repeated in the design notes):
- row i of the target logits is the target's distribution after the path to node i; node 0 is the root;
- parent[b][0] is ignored; for i >= 1 parent[b][i] must lie in [0, i) (nodes in topological order) and token[b][i] in
  [0, V), else the sequence is flagged ID_RANGE and not verified;
- a NaN or +inf logit, or a row of -inf only, in a row the walk reads (every node it visits, the stop node included)
  is flagged NONFINITE and the sequence is not verified; rows off the walk are not checked;
- p'(x) is formed as p(x) over the mass of p outside E, that mass summed directly over the complement (no 1 - sum);
- the draw follows the dense verifier's rule: smallest index whose running sum exceeds t, the last index with
  positive weight if rounding leaves none, and p itself (flag EMPTY_RESIDUAL) if the excluded tokens held all of p.
"""
from __future__ import annotations

import numpy as np

from .verify import FLAG_EMPTY_RESIDUAL, FLAG_ID_RANGE, FLAG_NONFINITE, _bad_rows, inverse_cdf, softmax, widen


def tree_children(parent: np.ndarray) -> list:
    """Children of every node of one tree, each list in increasing node index (node 0 is the root)."""
    N = len(parent)
    kids = [[] for _ in range(N)]
    for i in range(1, N):
        kids[int(parent[i])].append(i)
    return kids


def tree_is_valid(parent: np.ndarray, token: np.ndarray, V: int) -> bool:
    """parent[i] in [0, i) and token[i] in [0, V) for every node i >= 1."""
    i = np.arange(1, len(parent))
    return bool(np.all((parent[1:] >= 0) & (parent[1:] < i)) and np.all((token[1:] >= 0) & (token[1:] < V)))


def verify_tree(target, parent, token, u_accept, u_sample, temperature, *, dtype="f32"):
    """Verify B token trees of N nodes against the target's logits.

    target [B, N, V] logits (row i: the target's distribution after the path to node i); parent [B, N] int; token
    [B, N] int (token[b][i] is the drafted token of node i >= 1); u_accept [B, N] (test of node i); u_sample [B, N]
    (the draw at stop node i); temperature T > 0.

    Returns a dict of numpy arrays: accept [B, N] uint8 (1 for accepted nodes), tested [B, N] uint8, p_test [B, N]
    (p'(x) of each tested node, NaN elsewhere), n_accepted [B], path [B, N] (accepted nodes in walk order, -1 after),
    out_token [B], stop_node [B], flags [B], margin_accept [B, N] (|u - min(1, p'(x))|, inf where not tested),
    margin_cdf [B] (the draw's distance to the nearer CDF boundary over its mass, inf where none).
    """
    parent = np.asarray(parent, dtype=np.int64)
    token = np.asarray(token, dtype=np.int64)
    B, N = parent.shape
    V = np.shape(target)[-1]
    T = np.float64(np.float32(temperature))
    ua = np.asarray(u_accept, dtype=np.float64)
    us = np.asarray(u_sample, dtype=np.float64)
    out = dict(accept=np.zeros((B, N), np.uint8), tested=np.zeros((B, N), np.uint8), p_test=np.full((B, N), np.nan),
               n_accepted=np.zeros(B, np.int32), path=np.full((B, N), -1, np.int32),
               out_token=np.full(B, -1, np.int32), stop_node=np.full(B, -1, np.int32), flags=np.zeros(B, np.uint32),
               margin_accept=np.full((B, N), np.inf), margin_cdf=np.full(B, np.inf))
    for b in range(B):
        if not tree_is_valid(parent[b], token[b], V):
            out["flags"][b] = FLAG_ID_RANGE
            out["n_accepted"][b] = -1
            continue
        kids = tree_children(parent[b])
        rows = {}

        def row_p(i):
            if i not in rows:
                z = widen(np.asarray(target)[b, i], dtype) / T
                rows[i] = None if _bad_rows(z[None])[0] else softmax(z)
            return rows[i]

        cur, path, fault = 0, [], False
        while True:
            p = row_p(cur)
            if p is None:
                fault = True
                break
            excluded = np.zeros(V, bool)
            nxt = -1
            for c in kids[cur]:
                x = token[b, c]
                if excluded[x]:
                    P = 0.0
                else:
                    P = p[x] / np.sum(p[~excluded])          # p'(x): p renormalised outside the excluded tokens
                out["tested"][b, c] = 1
                out["p_test"][b, c] = P
                out["margin_accept"][b, c] = abs(ua[b, c] - min(1.0, P))
                if ua[b, c] < min(1.0, P):                   # the strict test with one-hot q
                    nxt = c
                    break
                excluded[x] = True                           # residual max(p' - e_x, 0): p' without x
            if nxt < 0:
                break
            out["accept"][b, nxt] = 1
            path.append(nxt)
            cur = nxt
        if fault:
            out["flags"][b] = FLAG_NONFINITE
            out["n_accepted"][b] = -1
            out["accept"][b] = 0
            out["tested"][b] = 0
            out["p_test"][b] = np.nan
            out["margin_accept"][b] = np.inf
            continue
        r = np.where(excluded, 0.0, p)
        if r.sum() == 0:                                     # the excluded tokens held all of p
            r = p
            out["flags"][b] |= FLAG_EMPTY_RESIDUAL
        idx, mg = inverse_cdf(r, us[b, cur] * r.sum())
        out["out_token"][b] = int(idx[0])
        out["margin_cdf"][b] = float(mg[0])
        out["stop_node"][b] = cur
        out["n_accepted"][b] = len(path)
        out["path"][b, :len(path)] = path
    return out
