"""Plain float64 CPU oracle of the speculative-sampling verifier.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg import this module.
The HIP library never calls it, and it imports nothing from the HIP package: the two share no code.

What it follows (pages cited by title and section):
- "Uno: the draft model was already inside the target model", section "What 'lossless' actually has to mean":
  the Leviathan et al. rule. A draft token x drawn from q is kept with probability min(1, p(x)/q(x)); on rejection a
  replacement is drawn from max(p - q, 0) renormalised. The same section prints the engine's sparse top-k verify
  routine; its observable semantics (id-equality gathers of p and q at the drafted id, ratio 0 when q is 0, the strict
  test u < min(1, ratio), a correction distribution clamp(p - q_on_p, 0) renormalised on p's support) define
  ``verify_sparse``. The last paragraph of that section says that greedy drafting makes q one-hot and that the rule
  must then be applied to that q: ``onehot=True``.
- DFlash/DFlash2 guide, section 4.4 "Mathematical Losslessness Guarantee": the block is truncated at the first
  rejected position k and the replacement is drawn from the normalised residual there. Section 9, Q3: temperature
  scales both the draft and the target logits before the ratio. Section 2, "Speculative Decoding Speedup
  Formulation": the tokens per cycle lie in [1, gamma + 1], counting the target's bonus token drawn when every draft
  is accepted.
- "Self-Speculative Masked Diffusions", 关键设计 2: verification walks the generation order sigma from the first
  unknown slot, stops at the first rejection and resamples there, with no bonus; 关键设计 4: several verification
  rounds reuse one draft, each starting after the previous round's resampled slot (``verify_windows``).

Readings where the pages leave a step open (each is repeated in the design notes):
- tie u == min(1, ratio) rejects (the printed routine uses a strict less-than);
- p = softmax(z_t / T), q = softmax(z_d / T), the same T > 0 on both sides;
- ratio = 0 when q(x) is exactly 0 (draft logit -inf at x): the draft is rejected and the Q_ZERO flag is set;
- an empty residual (zero total mass) falls back to drawing from p and sets EMPTY_RESIDUAL;
- the inverse CDF runs over vocabulary order (dense) or the given slot order (sparse): the chosen index is the
  smallest i whose inclusive prefix sum exceeds t = u * (total mass); if rounding leaves none, the last index with
  positive mass is taken;
- u_accept is indexed by storage row; u_sample by the storage row of the slot where the draw happens, and by
  column gamma for the bonus draw.
"""
from __future__ import annotations

import numpy as np

FLAG_NONFINITE = 1        # NaN or +inf logit / probability, negative probability, or a row that is all -inf
FLAG_ID_RANGE = 2         # a draft/spec/support id out of range, a bad order permutation, or start outside [0, gamma]
FLAG_EMPTY_RESIDUAL = 4   # the residual had zero mass; the draw used p instead
FLAG_Q_ZERO = 8           # q was exactly 0 at the drafted id

FATAL = FLAG_NONFINITE | FLAG_ID_RANGE


# ----------------------------------------------------------------------------------------------------------------------
# Input decoding (exact widening to float64)
# ----------------------------------------------------------------------------------------------------------------------

def widen(x, dtype: str) -> np.ndarray:
    """Return the float64 values of a logit tensor given as float32 (or float64) or as bfloat16 bit patterns."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------------------------------------------------
# Building blocks, each a plain definition
# ----------------------------------------------------------------------------------------------------------------------

def softmax(a: np.ndarray) -> np.ndarray:
    """softmax over the last axis: exp(a - max a) / sum exp(a - max a). Entries at -inf get probability 0."""
    with np.errstate(invalid="ignore", over="ignore"):
        m = np.max(a, axis=-1, keepdims=True)
        e = np.exp(a - m)
        return e / np.sum(e, axis=-1, keepdims=True)


def log_softmax_at(a: np.ndarray, x: np.ndarray) -> np.ndarray:
    """log softmax(a)[x] = a[x] - (max a + log sum exp(a - max a)), over the last axis, at index x (one per row)."""
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        m = np.max(a, axis=-1)
        lse = m + np.log(np.sum(np.exp(a - m[..., None]), axis=-1))
        ax = np.take_along_axis(a, x[..., None], axis=-1)[..., 0]
        return ax - lse


def residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """The leftover mass max(p - q, 0) (unnormalised)."""
    return np.maximum(p - q, 0.0)


def inverse_cdf(r: np.ndarray, t: np.ndarray):
    """Draw by inverse CDF from unnormalised weights r (rows on the last axis) at thresholds t (one per row).

    Returns (index, margin). The index is the smallest i with C_i > t, where C is the inclusive running sum of r in
    index order; when rounding leaves no such i, the last index with r_i > 0 (margin 0). The margin is the distance of
    t to the nearer boundary of the chosen interval, min(t - C_{i-1}, C_i - t), divided by the total mass C_last."""
    r = np.atleast_2d(r)
    t = np.atleast_1d(np.asarray(t, dtype=np.float64))
    C = np.cumsum(r, axis=-1)
    hit = C > t[:, None]
    any_hit = hit.any(axis=-1)
    idx = np.argmax(hit, axis=-1)
    pos = r > 0
    last_pos = np.where(pos.any(axis=-1), r.shape[-1] - 1 - np.argmax(pos[:, ::-1], axis=-1), -1)
    idx = np.where(any_hit, idx, last_pos)
    rows = np.arange(r.shape[0])
    hi = C[rows, np.maximum(idx, 0)]
    lo = np.where(idx > 0, C[rows, np.maximum(idx - 1, 0)], 0.0)
    total = C[:, -1]
    with np.errstate(invalid="ignore", divide="ignore"):
        margin = np.where(any_hit, np.minimum(t - lo, hi - t) / total, 0.0)
    return idx.astype(np.int64), margin


def accept_test(u: np.ndarray, ratio: np.ndarray) -> np.ndarray:
    """Strict test u < min(1, ratio)."""
    return u < np.minimum(1.0, ratio)


def accept_test_exact(u: np.ndarray, p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """The strict test u < min(1, p/q) with ratio 0 when q is 0, evaluated without a division.

    For u in [0, 1) and q > 0, u < min(1, p/q) holds iff u*q < p. When u, p and q are float32 values their products
    are exact in float64, so this is the exact comparison of the real numbers."""
    return (q > 0) & (u * q < p)


# ----------------------------------------------------------------------------------------------------------------------
# Dense and one-hot verification
# ----------------------------------------------------------------------------------------------------------------------

def _bad_rows(a: np.ndarray) -> np.ndarray:
    """Rows (last axis) holding a NaN or +inf, or only -inf."""
    return np.isnan(a).any(-1) | np.isposinf(a).any(-1) | np.isneginf(a).all(-1)


def verify_dense(target, draft, draft_ids, u_accept, u_sample, temperature, *, bonus=1, start=None, order=None,
                 dtype="f32", onehot=False, chunk_elems=1 << 23):
    """Verify B blocks of gamma drafted tokens against dense logits.

    target    [B, gamma + bonus, V] logits of the target model (row gamma is only read for a bonus draw)
    draft     [B, gamma, V] logits of the drafter, or None with ``onehot=True`` (q is one-hot at the draft id)
    draft_ids [B, gamma] int, u_accept [B, gamma], u_sample [B, gamma + 1] (all indexed by storage row)
    start     [B] first slot to verify (default 0); order [B, gamma] slot -> storage row (default identity)

    Returns a dict of numpy arrays: accept (uint8, by row), n_accepted, out_token, p_draft, q_draft (by row),
    flags, start_out, first_reject (slot k, or gamma), margin_accept (by row; inf where not verified),
    margin_cdf (per sequence; inf where no draw happened), resampled (1 for a residual draw, 2 for a bonus draw).
    """
    draft_ids = np.asarray(draft_ids)
    B, G = draft_ids.shape
    V = np.shape(target)[-1]
    T = np.float64(np.float32(temperature))
    start = np.zeros(B, np.int64) if start is None else np.asarray(start, dtype=np.int64)
    order = np.tile(np.arange(G), (B, 1)) if order is None else np.asarray(order, dtype=np.int64)
    ua = np.asarray(u_accept, dtype=np.float64)      # float32 inputs widen exactly
    us = np.asarray(u_sample, dtype=np.float64)

    out = dict(accept=np.zeros((B, G), np.uint8), n_accepted=np.zeros(B, np.int32), out_token=np.full(B, -1, np.int32),
               p_draft=np.zeros((B, G)), q_draft=np.zeros((B, G)), flags=np.zeros(B, np.uint32),
               start_out=start.astype(np.int32).copy(), first_reject=np.full(B, G, np.int32),
               margin_accept=np.full((B, G), np.inf), margin_cdf=np.full(B, np.inf), resampled=np.zeros(B, np.int8))

    per_seq = max(1, (G + 1) * V * 2)
    step = max(1, chunk_elems // per_seq)
    for b0 in range(0, B, step):
        b1 = min(B, b0 + step)
        _dense_chunk(out, slice(b0, b1), target, draft, draft_ids, ua, us, T, bonus, start, order, dtype, onehot, G, V)
    return out


def _dense_chunk(out, sl, target, draft, draft_ids, ua, us, T, bonus, start, order, dtype, onehot, G, V):
    nb = sl.stop - sl.start
    bi = np.arange(nb)[:, None]
    st = start[sl]
    od = order[sl]

    # Argument checks that make a sequence unverifiable.
    bad_order = ((od < 0) | (od >= G)).any(-1)
    od_safe = np.where((od >= 0) & (od < G), od, 0)
    bad_order |= np.array([len(set(r.tolist())) != G for r in od_safe])
    od_safe = np.where(bad_order[:, None], np.arange(G)[None, :], od_safe)
    bad_start = (st < 0) | (st > G)
    done = (st >= G) & ~bad_start
    slot = np.arange(G)[None, :]
    verified = (slot >= st[:, None]) & ~bad_start[:, None] & ~bad_order[:, None]

    # Temperature on both sides before the ratio (DFlash guide, section 9 Q3).
    a = widen(np.asarray(target)[sl], dtype)[bi, od_safe] / T                      # [nb, G, V], slot order
    x = np.asarray(draft_ids)[sl][bi, od_safe].astype(np.int64)                    # drafted id per slot
    bad_id = ((x < 0) | (x >= V)) & verified
    xs = np.clip(x, 0, V - 1)
    bad_row = _bad_rows(a) & verified
    if onehot:
        c = None
    else:
        c = widen(np.asarray(draft)[sl], dtype)[bi, od_safe] / T
        bad_row |= _bad_rows(c) & verified
    fatal_id = bad_order | bad_start | bad_id.any(-1)
    fatal_nf = bad_row.any(-1)
    fatal = fatal_id | fatal_nf

    # p(x), q(x) and the acceptance ratio p(x)/q(x) (Uno, "What 'lossless' actually has to mean").
    lp = log_softmax_at(a, xs)
    if onehot:
        lq = np.zeros_like(lp)                       # q = e_x: q(x) = 1
        q_zero = np.zeros_like(lp, dtype=bool)
    else:
        lq = log_softmax_at(c, xs)
        q_zero = np.isneginf(np.take_along_axis(c, xs[..., None], axis=-1)[..., 0])
    with np.errstate(invalid="ignore", over="ignore"):
        ratio = np.where(q_zero, 0.0, np.exp(lp - lq))
    ratio = np.where(np.isnan(ratio), 0.0, ratio)
    u_slot = ua[sl][bi, od_safe]
    acc = accept_test(u_slot, ratio) & verified
    m_acc = np.where(verified, np.abs(u_slot - np.minimum(1.0, ratio)), np.inf)

    # First rejection at or after start (slots before start count as already settled).
    settled = acc | ~verified
    k = np.where(settled.all(-1), G, np.argmin(settled, axis=-1))
    n = k - np.minimum(st, G)

    flags = np.zeros(nb, np.uint32)
    flags |= np.where(fatal_id, FLAG_ID_RANGE, 0).astype(np.uint32)
    flags |= np.where(fatal_nf, FLAG_NONFINITE, 0).astype(np.uint32)
    flags |= np.where(~fatal & (q_zero & verified).any(-1), FLAG_Q_ZERO, 0).astype(np.uint32)

    token = np.full(nb, -1, np.int64)
    m_cdf = np.full(nb, np.inf)
    kind = np.zeros(nb, np.int8)
    live = ~fatal & ~done

    # Residual draw at the first rejected slot (DFlash guide 4.4; Uno, "What 'lossless' actually has to mean").
    rej = np.flatnonzero(live & (k < G))
    if rej.size:
        kr = k[rej]
        rho = od_safe[rej, kr]
        p = softmax(a[rej, kr])
        if onehot:
            q = np.zeros_like(p)
            q[np.arange(rej.size), xs[rej, kr]] = 1.0
        else:
            q = softmax(c[rej, kr])
        r = residual(p, q)
        S_r = r.sum(-1)
        empty = S_r == 0
        r = np.where(empty[:, None], p, r)
        flags[rej[empty]] |= FLAG_EMPTY_RESIDUAL
        t = us[sl][rej, rho] * r.sum(-1)
        idx, mg = inverse_cdf(r, t)
        token[rej], m_cdf[rej], kind[rej] = idx, mg, 1

    # Bonus draw from p of target row gamma when every draft was accepted (DFlash guide, section 2).
    if bonus:
        bon = np.flatnonzero(live & (k == G))
        if bon.size:
            ab = widen(np.asarray(target)[sl][bon, G], dtype) / T
            badb = _bad_rows(ab)
            flags[bon[badb]] |= FLAG_NONFINITE
            good = bon[~badb]
            if good.size:
                p = softmax(ab[~badb])
                t = us[sl][good, G] * p.sum(-1)
                idx, mg = inverse_cdf(p, t)
                token[good], m_cdf[good], kind[good] = idx, mg, 2

    # Scatter slot-ordered results back to storage rows.
    acc_row = np.zeros((nb, G), np.uint8)
    p_row = np.zeros((nb, G))
    q_row = np.zeros((nb, G))
    ma_row = np.full((nb, G), np.inf)
    acc_row[bi, od_safe] = acc
    with np.errstate(over="ignore"):
        p_row[bi, od_safe] = np.where(verified, np.exp(lp), 0.0)
        q_row[bi, od_safe] = np.where(verified, np.exp(lq), 0.0)
    ma_row[bi, od_safe] = m_acc
    acc_row[fatal] = 0
    p_row[fatal] = np.nan
    q_row[fatal] = np.nan
    ma_row[fatal] = np.inf

    out["accept"][sl] = acc_row
    out["p_draft"][sl] = p_row
    out["q_draft"][sl] = q_row
    out["margin_accept"][sl] = ma_row
    out["n_accepted"][sl] = np.where(fatal, -1, np.where(done, 0, n))
    out["out_token"][sl] = np.where(fatal, -1, token)
    out["flags"][sl] = flags
    out["first_reject"][sl] = np.where(live, k, G)
    out["margin_cdf"][sl] = m_cdf
    out["resampled"][sl] = kind
    out["start_out"][sl] = np.where(live, np.minimum(G, k + 1), st)


def verify_onehot(target, draft_ids, u_accept, u_sample, temperature, **kw):
    """Greedy drafting: q is one-hot at the draft id, so the test is u < p(d) and the residual is p with d removed."""
    return verify_dense(target, None, draft_ids, u_accept, u_sample, temperature, onehot=True, **kw)


def verify_windows(target, draft, draft_ids, u_accept_rounds, u_sample_rounds, temperature, *, order, start=None,
                   dtype="f32"):
    """Several verification rounds over one window of drafts (Self-Speculative Masked Diffusions, 关键设计 2 and 4).

    Round r verifies slots start_r .. W-1 in the given order with no bonus; the next round starts after the
    resampled slot: start_{r+1} = min(W, first_reject_r + 1). Returns one result dict per round."""
    B, W = np.asarray(draft_ids).shape
    st = np.zeros(B, np.int64) if start is None else np.asarray(start, dtype=np.int64).copy()
    results = []
    for r in range(len(u_accept_rounds)):
        res = verify_dense(target, draft, draft_ids, u_accept_rounds[r], u_sample_rounds[r], temperature, bonus=0,
                           start=st, order=order, dtype=dtype)
        results.append(res)
        st = res["start_out"].astype(np.int64)
    return results


# ----------------------------------------------------------------------------------------------------------------------
# Sparse (top-k support) verification
# ----------------------------------------------------------------------------------------------------------------------

def _slot_order_sum(v: np.ndarray) -> np.ndarray:
    """Sum over the last axis strictly left to right (the running sum's final value)."""
    if v.shape[-1] == 0:
        return np.zeros(v.shape[:-1])
    return np.cumsum(v, axis=-1)[..., -1]


def verify_sparse(p_ids, p_probs, q_ids, q_probs, spec_ids, u_accept, u_sample, *, bonus=1, vocab_size=0,
                  chunk_elems=1 << 24):
    """Verify drafts against top-k supports (Uno, the sparse verify routine in "What 'lossless' actually has to mean").

    p_ids/p_probs [B, gamma + bonus, kp] target support; q_ids/q_probs [B, gamma, kq] drafter support;
    spec_ids [B, gamma] drafted ids; u_accept [B, gamma]; u_sample [B, gamma + 1].

    Per position: p_spec and q_spec are the probabilities on the slots whose id equals the drafted id (summed in
    slot order); accept iff q_spec > 0 and u < min(1, p_spec / q_spec); the correction distribution on p's support is
    max(p_i - q_on_p_i, 0) renormalised, with q_on_p_i the q probability of p's i-th id. Probabilities are used as
    given (no renormalisation of p or q). Returns accept, n_accepted, out_token, correction_probs, p_spec, q_spec,
    flags, first_reject, margin_accept, margin_cdf, resampled.
    """
    B = np.shape(spec_ids)[0]
    per_seq = max(1, int(np.prod(np.shape(q_ids)[1:])) * np.shape(p_ids)[-1])
    step = max(1, chunk_elems // per_seq)
    if B > step:
        parts = [verify_sparse(p_ids[b:b + step], p_probs[b:b + step], q_ids[b:b + step], q_probs[b:b + step],
                               spec_ids[b:b + step], u_accept[b:b + step], u_sample[b:b + step], bonus=bonus,
                               vocab_size=vocab_size, chunk_elems=chunk_elems) for b in range(0, B, step)]
        return {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}
    p_ids = np.asarray(p_ids, dtype=np.int64)
    q_ids = np.asarray(q_ids, dtype=np.int64)
    pp = np.asarray(p_probs, dtype=np.float32).astype(np.float64)
    qp = np.asarray(q_probs, dtype=np.float32).astype(np.float64)
    x = np.asarray(spec_ids, dtype=np.int64)
    ua = np.asarray(u_accept, dtype=np.float64)      # float32 inputs widen exactly
    us = np.asarray(u_sample, dtype=np.float64)
    B, G = x.shape
    kp = p_ids.shape[-1]

    pr, qr, prb, qrb = p_ids[:, :G], q_ids, pp[:, :G], qp
    p_spec = _slot_order_sum(np.where(pr == x[..., None], prb, 0.0))
    q_spec = _slot_order_sum(np.where(qr == x[..., None], qrb, 0.0))

    q_zero = q_spec == 0
    with np.errstate(invalid="ignore"):
        acc = accept_test_exact(ua, p_spec, q_spec)
        ratio = np.where(q_zero, 0.0, p_spec / np.where(q_zero, 1.0, q_spec))
    m_acc = np.abs(ua - np.minimum(1.0, ratio))

    # Correction distribution on p's support.
    q_on_p = _slot_order_sum(np.where(pr[..., :, None] == qr[..., None, :], qrb[..., None, :], 0.0))
    corr = residual(prb, q_on_p)
    S_c = _slot_order_sum(corr)
    empty_pos = S_c == 0
    corr_used = np.where(empty_pos[..., None], prb, corr)
    S_used = _slot_order_sum(corr_used)
    with np.errstate(invalid="ignore", divide="ignore"):
        correction = corr_used / S_used[..., None]

    flags = np.zeros(B, np.uint32)
    fatal_nf = (~np.isfinite(prb) | (prb < 0)).any((-1, -2)) | (~np.isfinite(qrb) | (qrb < 0)).any((-1, -2))
    if vocab_size:
        fatal_id = ((x < 0) | (x >= vocab_size)).any(-1) | ((pr < 0) | (pr >= vocab_size)).any((-1, -2)) \
            | ((qr < 0) | (qr >= vocab_size)).any((-1, -2))
    else:
        fatal_id = np.zeros(B, bool)
    fatal = fatal_nf | fatal_id
    flags |= np.where(fatal_id, FLAG_ID_RANGE, 0).astype(np.uint32)
    flags |= np.where(fatal_nf, FLAG_NONFINITE, 0).astype(np.uint32)
    flags |= np.where(~fatal & q_zero.any(-1), FLAG_Q_ZERO, 0).astype(np.uint32)

    k = np.where(acc.all(-1), G, np.argmin(acc, axis=-1))
    token = np.full(B, -1, np.int64)
    m_cdf = np.full(B, np.inf)
    kind = np.zeros(B, np.int8)

    rej = np.flatnonzero(~fatal & (k < G))
    if rej.size:
        kr = k[rej]
        w = corr_used[rej, kr]
        flags[rej[empty_pos[rej, kr]]] |= FLAG_EMPTY_RESIDUAL
        t = us[rej, kr] * S_used[rej, kr]
        idx, mg = _slot_draw(w, t)
        token[rej] = np.where(idx >= 0, p_ids[rej, kr, np.maximum(idx, 0)], -1)
        m_cdf[rej], kind[rej] = mg, 1
    if bonus:
        bon = np.flatnonzero(~fatal & (k == G))
        if bon.size:
            wb = pp[bon, G]
            badb = (~np.isfinite(wb) | (wb < 0)).any(-1)
            if vocab_size:
                badb_id = ((p_ids[bon, G] < 0) | (p_ids[bon, G] >= vocab_size)).any(-1)
            else:
                badb_id = np.zeros(bon.size, bool)
            flags[bon[badb]] |= FLAG_NONFINITE
            flags[bon[badb_id & ~badb]] |= FLAG_ID_RANGE
            good = ~badb & ~badb_id
            g = bon[good]
            if g.size:
                t = us[g, G] * _slot_order_sum(wb[good])
                idx, mg = _slot_draw(wb[good], t)
                token[g] = np.where(idx >= 0, p_ids[g, G, np.maximum(idx, 0)], -1)
                m_cdf[g], kind[g] = mg, 2

    p_spec_o = np.where(fatal[:, None], np.nan, p_spec)
    q_spec_o = np.where(fatal[:, None], np.nan, q_spec)
    corr_o = np.where(fatal[:, None, None], np.nan, correction)
    return dict(accept=np.where(fatal[:, None], 0, acc).astype(np.uint8),
                n_accepted=np.where(fatal, -1, k).astype(np.int32),
                out_token=np.where(fatal, -1, token).astype(np.int32),
                correction_probs=corr_o, p_spec=p_spec_o, q_spec=q_spec_o, flags=flags,
                first_reject=np.where(fatal, G, k).astype(np.int32),
                margin_accept=np.where(fatal[:, None], np.inf, m_acc), margin_cdf=m_cdf, resampled=kind)


def _slot_draw(w: np.ndarray, t: np.ndarray):
    """Inverse CDF over support slots in their given order (no sorting); same rule as ``inverse_cdf``."""
    return inverse_cdf(w, t)
