"""Seeded synthetic inputs for the verifier, shaped like the workloads the pages describe.

This module only draws random inputs. It holds none of the verifier's arithmetic, and both the HIP path and the CPU
oracle consume what it returns (host numpy arrays). It imports numpy only.

Logits stand in for the outputs of the models the pages discuss; the models, datasets and serving systems themselves
are not available, so every tensor here is drawn from the stated distributions with ``numpy.random.Generator(PCG64)``
seeded through ``SeedSequence(seed).spawn(n)``, one independent stream per array.

Conventions
- bf16 tensors are returned as ``uint16`` bit patterns, rounded from float32 to nearest-even.
- Uniforms are float32 multiples of 2**-24 in [0, 1).
- Draft tokens "sampled from softmax(z / T)" use the Gumbel-max construction
  ``argmax(z / T + G)`` with i.i.d. standard Gumbel noise G, which draws from that softmax without forming it.
- Shapes: target logits [B, gamma + bonus, V], draft logits [B, gamma, V], draft ids [B, gamma],
  u_accept [B, gamma], u_sample [B, gamma + 1] (the last column is only read for a bonus draw).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

DTYPE_F32 = "f32"
DTYPE_BF16 = "bf16"

_CHUNK = 1 << 22          # elements per independently seeded chunk (fixed, so results do not depend on threads)
_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))


class _Stream:
    """One named random stream. Large fills are cut into fixed chunks, each with its own child seed, and filled on a
    thread pool; the values depend only on the seed and the shape."""

    def __init__(self, seed_seq: np.random.SeedSequence):
        self.ss = seed_seq
        self.rng = np.random.Generator(np.random.PCG64(seed_seq.spawn(1)[0]))

    def _chunked(self, n: int, fill):
        out = np.empty(n, dtype=np.float32)
        kids = self.ss.spawn((n + _CHUNK - 1) // _CHUNK)

        def run(i):
            g = np.random.Generator(np.random.PCG64(kids[i]))
            fill(g, out[i * _CHUNK:min(n, (i + 1) * _CHUNK)])
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(run, range(len(kids))))
        return out

    def normal(self, shape, sigma: float) -> np.ndarray:
        n = int(np.prod(shape))

        def fill(g, o):
            g.standard_normal(out=o, dtype=np.float32)
            o *= np.float32(sigma)
        return self._chunked(n, fill).reshape(shape)

    def gumbel(self, shape) -> np.ndarray:
        """Standard Gumbel noise -log(-log(U)) in float32."""
        n = int(np.prod(shape))

        def fill(g, o):
            g.random(out=o, dtype=np.float32)
            with np.errstate(divide="ignore"):
                np.log(o, out=o)
                np.negative(o, out=o)
                np.log(o, out=o)
                np.negative(o, out=o)
        return self._chunked(n, fill).reshape(shape)


def _streams(seed: int, n: int):
    return [_Stream(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _pmap(fn, n: int):
    """Run fn(i0, i1) over [0, n) in fixed chunks on the thread pool (numpy releases the GIL in these kernels)."""
    spans = [(i, min(n, i + _CHUNK)) for i in range(0, n, _CHUNK)]
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(lambda s: fn(*s), spans))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the 16-bit patterns as uint16. NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)

    def conv(i0, i1):
        u = flat[i0:i1].view(np.uint32)
        r = (u >> 16) & 1
        r += 0x7FFF
        r += u                      # finite and infinite inputs cannot wrap around 2**32
        r >>= 16
        nan = np.isnan(flat[i0:i1])
        if nan.any():
            r[nan] = (u[nan] >> 16) | 0x40
        out[i0:i1] = r
    _pmap(conv, flat.size)
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    flat = bits.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint32)

    def conv(i0, i1):
        o = out[i0:i1]
        o[...] = flat[i0:i1]
        o <<= 16
    _pmap(conv, flat.size)
    return out.view(np.float32).reshape(bits.shape)


def uniforms(stream: "_Stream", shape) -> np.ndarray:
    """float32 uniforms on the 2**-24 grid of [0, 1)."""
    return (stream.rng.integers(0, 1 << 24, size=shape, dtype=np.int64).astype(np.float64)
            * (2.0 ** -24)).astype(np.float32)


def _gumbel_argmax(stream: "_Stream", scores: np.ndarray, scale: float = 1.0, rows_per_chunk: int = 256) -> np.ndarray:
    """argmax over the last axis of scores * scale + standard Gumbel noise: a draw from softmax(scores * scale)."""
    lead = scores.shape[:-1]
    V = scores.shape[-1]
    flat = scores.reshape(-1, V)
    out = np.empty(flat.shape[0], dtype=np.int32)
    for r0 in range(0, flat.shape[0], rows_per_chunk):
        blk = flat[r0:r0 + rows_per_chunk]
        g = stream.gumbel(blk.shape)
        if scale != 1.0:
            g += blk.astype(np.float32, copy=False) * np.float32(scale)
        else:
            g += blk
        out[r0:r0 + rows_per_chunk] = np.argmax(g, axis=-1)
    return out.reshape(lead)


def _normal_f32(stream: "_Stream", shape, sigma):
    return stream.normal(shape, sigma)


# ----------------------------------------------------------------------------------------------------------------------
# Dense inputs
# ----------------------------------------------------------------------------------------------------------------------

def dense_case(B: int, gamma: int, V: int, *, dtype: str = DTYPE_F32, sigma_t: float = 2.0, sigma_d: float = 0.5,
               zipf: float = 0.0, temperature: float = 1.0, bonus: int = 1, seed: int = 0) -> dict:
    """Target ~ N(0, sigma_t^2) (+ optional -zipf*ln(i+1) bias on token i), draft = target + N(0, sigma_d^2),
    draft ids ~ softmax(draft / T); per-position uniforms. Values are rounded to ``dtype`` after all noise is added."""
    r_t, r_d, r_x, r_a, r_s = _streams(seed, 5)
    rows_t = gamma + bonus
    zt = _normal_f32(r_t, (B, rows_t, V), sigma_t)
    if zipf:
        zt += (-zipf * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
    zd = _normal_f32(r_d, (B, gamma, V), sigma_d)
    zd += zt[:, :gamma]
    if dtype == DTYPE_BF16:
        zt_store, zd_store = f32_to_bf16_bits(zt), f32_to_bf16_bits(zd)
        del zt
        zd = bf16_bits_to_f32(zd_store)
    else:
        zt_store, zd_store = zt, zd
    T = np.float32(temperature)
    ids = _gumbel_argmax(r_x, zd, 1.0 / float(T))
    del zd
    return dict(kind="dense", dtype=dtype, B=B, gamma=gamma, V=V, bonus=bonus, temperature=float(T),
                target=zt_store, draft=zd_store, draft_ids=ids.astype(np.int32),
                u_accept=uniforms(r_a, (B, gamma)), u_sample=uniforms(r_s, (B, gamma + 1)))


def onehot_case(B: int, gamma: int, V: int, *, dtype: str = DTYPE_BF16, sigma_t: float = 2.5, sigma_x: float = 1.5,
                temperature: float = 0.7, bonus: int = 1, seed: int = 0) -> dict:
    """Greedy drafter: target ~ N(0, sigma_t^2); draft id = argmax(target + N(0, sigma_x^2)) (lowest index on ties);
    the draft distribution is one-hot at that id, so no draft logits exist."""
    r_t, r_n, r_a, r_s = _streams(seed, 4)
    rows_t = gamma + bonus
    zt = _normal_f32(r_t, (B, rows_t, V), sigma_t)
    zt_store = f32_to_bf16_bits(zt) if dtype == DTYPE_BF16 else zt
    zt_eff = bf16_bits_to_f32(zt_store) if dtype == DTYPE_BF16 else zt
    noisy = _normal_f32(r_n, (B, gamma, V), sigma_x)
    noisy += zt_eff[:, :gamma]
    ids = np.argmax(noisy, axis=-1).astype(np.int32)
    del noisy
    return dict(kind="onehot", dtype=dtype, B=B, gamma=gamma, V=V, bonus=bonus, temperature=float(np.float32(temperature)),
                target=zt_store, draft=None, draft_ids=ids,
                u_accept=uniforms(r_a, (B, gamma)), u_sample=uniforms(r_s, (B, gamma + 1)))


def greedy_case(B: int, gamma: int, V: int, *, dtype: str = DTYPE_BF16, sigma_t: float = 3.0, zipf: float = 1.1,
                agree: float = 0.85, sigma_x: float = 1.5, bonus: int = 1, seed: int = 0) -> dict:
    """Greedy verification inputs: the target of ``dense_case`` (N(0, sigma_t^2) plus the Zipf bias); each draft id
    is, with probability ``agree``, the largest target logit of its row (lowest index on ties), and otherwise the
    largest of target + N(0, sigma_x^2). No draft logits, uniforms or temperature."""
    r_t, r_n, r_a = _streams(seed, 3)
    zt = _normal_f32(r_t, (B, gamma + bonus, V), sigma_t)
    if zipf:
        zt += (-zipf * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
    zt_store = f32_to_bf16_bits(zt) if dtype == DTYPE_BF16 else zt
    zt_eff = bf16_bits_to_f32(zt_store) if dtype == DTYPE_BF16 else zt
    noisy = _normal_f32(r_n, (B, gamma, V), sigma_x)
    keep = uniforms(r_a, (B, gamma)) < agree
    noisy[keep] = 0.0
    noisy += zt_eff[:, :gamma]
    ids = np.argmax(noisy, axis=-1).astype(np.int32)
    del noisy
    return dict(kind="greedy", dtype=dtype, B=B, gamma=gamma, V=V, bonus=bonus, target=zt_store, draft_ids=ids)


def commit_case(B: int, W: int, V: int, *, dtype: str = DTYPE_BF16, sigma: float = 3.0, zipf: float = 1.1,
                peak: float = 14.0, p_masked: float = 0.75, tau: float = 0.9, seed: int = 0) -> dict:
    """Masked-diffusion block inputs: logits N(0, sigma^2) plus the Zipf bias, plus a spike of height U(0, peak) at one
    uniform id per slot (so that slot confidences spread over (0, 1)); each slot still masked with probability
    ``p_masked``."""
    r_z, r_h, r_i, r_m = _streams(seed, 4)
    z = _normal_f32(r_z, (B, W, V), sigma)
    if zipf:
        z += (-zipf * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
    h = uniforms(r_h, (B, W)) * np.float32(peak)
    at = (uniforms(r_i, (B, W)) * V).astype(np.int64)
    np.put_along_axis(z, at[..., None], np.take_along_axis(z, at[..., None], axis=-1) + h[..., None], axis=-1)
    masked = (uniforms(r_m, (B, W)) < p_masked).astype(np.uint8)
    zs = f32_to_bf16_bits(z) if dtype == DTYPE_BF16 else z
    return dict(kind="commit", dtype=dtype, B=B, W=W, V=V, logits=zs, masked=masked, tau=float(np.float32(tau)))


# ----------------------------------------------------------------------------------------------------------------------
# Sparse (top-k support) inputs
# ----------------------------------------------------------------------------------------------------------------------

def _support_probs(rng, n_rows, k, alpha, mass):
    p = rng.dirichlet(np.full(k, alpha), size=n_rows) * mass
    p = -np.sort(-p, axis=-1)                      # like a top-k output: slots by decreasing probability
    return p.astype(np.float32)


def sparse_case(B: int, gamma: int, k: int, V: int, *, alpha: float = 0.3, mass: float = 0.95, shared: int | None = None,
                bonus: int = 1, seed: int = 0) -> dict:
    """p support: k distinct ids uniform in [0, V) with Dirichlet(alpha) probs scaled to ``mass``; q support: k distinct
    ids of which ``shared`` (default k/2) come from the same row's p ids and the rest from outside p's support, with
    their own Dirichlet(alpha)*mass probs; spec id drawn from q over q's support."""
    r_pid, r_pp, r_qid, r_qp, r_x, r_a, r_s = _streams(seed, 7)
    if shared is None:
        shared = k // 2
    rows_p = gamma + bonus
    p_ids = np.empty((B, rows_p, k), dtype=np.int32)
    q_ids = np.empty((B, gamma, k), dtype=np.int32)
    for b in range(B):
        for j in range(rows_p):
            p_ids[b, j] = r_pid.rng.choice(V, size=k, replace=False)
        for j in range(gamma):
            from_p = r_qid.rng.choice(p_ids[b, j], size=shared, replace=False)
            outside = []
            taken = set(p_ids[b, j].tolist())
            while len(outside) < k - shared:
                c = int(r_qid.rng.integers(0, V))
                if c not in taken:
                    taken.add(c)
                    outside.append(c)
            ids = np.concatenate([from_p, np.asarray(outside, dtype=np.int64)])
            q_ids[b, j] = r_qid.rng.permutation(ids)
    p_probs = _support_probs(r_pp.rng, B * rows_p, k, alpha, mass).reshape(B, rows_p, k)
    q_probs = _support_probs(r_qp.rng, B * gamma, k, alpha, mass).reshape(B, gamma, k)
    with np.errstate(divide="ignore"):
        slot = _gumbel_argmax(r_x, np.log(q_probs))
    spec = np.take_along_axis(q_ids, slot[..., None].astype(np.int64), axis=-1)[..., 0]
    return dict(kind="sparse", B=B, gamma=gamma, k=k, V=V, bonus=bonus,
                p_ids=p_ids, p_probs=p_probs, q_ids=q_ids, q_probs=q_probs, spec_ids=spec.astype(np.int32),
                u_accept=uniforms(r_a, (B, gamma)), u_sample=uniforms(r_s, (B, gamma + 1)))


# ----------------------------------------------------------------------------------------------------------------------
# Masked-diffusion window (several verification rounds over one draft)
# ----------------------------------------------------------------------------------------------------------------------

def window_case(B: int, W: int, V: int, *, rounds: int = 4, sigma_d: float = 2.0, sigma_t: float = 0.7,
                temperature: float = 1.0, seed: int = 0) -> dict:
    """Non-causal draft logits ~ N(0, sigma_d^2) fp32, causal target = draft + N(0, sigma_t^2); a random generation
    order per sequence; draft ids ~ softmax(draft / T) drawn once per window; fresh uniforms per round; no bonus."""
    r_d, r_t, r_o, r_x, r_a, r_s = _streams(seed, 6)
    zd = _normal_f32(r_d, (B, W, V), sigma_d)
    zt = _normal_f32(r_t, (B, W, V), sigma_t)
    zt += zd
    order = np.stack([r_o.rng.permutation(W) for _ in range(B)]).astype(np.int32)
    T = np.float32(temperature)
    ids = _gumbel_argmax(r_x, zd, 1.0 / float(T))
    return dict(kind="window", dtype=DTYPE_F32, B=B, gamma=W, V=V, bonus=0, rounds=rounds, temperature=float(T),
                target=zt, draft=zd, draft_ids=ids.astype(np.int32), order=order,
                u_accept=uniforms(r_a, (rounds, B, W)), u_sample=uniforms(r_s, (rounds, B, W + 1)))


# ----------------------------------------------------------------------------------------------------------------------
# Token trees (several candidates per position)
# ----------------------------------------------------------------------------------------------------------------------

def random_tree_parents(rng, B: int, N: int, p_chain: float = 0.5) -> np.ndarray:
    """parent[b][0] = -1; node i >= 1 hangs under node i - 1 with probability p_chain, else under a uniformly chosen
    earlier node (a random recursive tree: deep main lines with side branches)."""
    parent = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        for i in range(1, N):
            parent[b, i] = i - 1 if rng.random() < p_chain else int(rng.integers(0, i))
    return parent


def tree_case(B: int, N: int, V: int, *, dtype: str = DTYPE_BF16, sigma: float = 2.0, zipf: float = 1.1,
              spike: tuple = (12.0, 24.0), sigma_x: float = 1.5, temperature: float = 1.0, seed: int = 0) -> dict:
    """Token trees of N nodes (node 0 the root): target logits [B, N, V], one row per node (the target's distribution
    after the path to that node): N(0, sigma^2) plus the Zipf bias plus a spike of height U(spike) at one uniform id, so
    that the top candidates carry much of the mass; parents from ``random_tree_parents``; the children of a node, in
    increasing node index, carry the drafter's top candidates in decreasing order: the largest entries of that node's
    row + N(0, sigma_x^2) (distinct tokens, as a top-m drafter proposes them); u_accept [B, N] and u_sample [B, N]."""
    r_z, r_h, r_i, r_p, r_x, r_a, r_s = _streams(seed, 7)
    z = _normal_f32(r_z, (B, N, V), sigma)
    if zipf:
        z += (-zipf * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
    h = np.float32(spike[0]) + uniforms(r_h, (B, N)) * np.float32(spike[1] - spike[0])
    at = (uniforms(r_i, (B, N)) * V).astype(np.int64)
    np.put_along_axis(z, at[..., None], np.take_along_axis(z, at[..., None], axis=-1) + h[..., None], axis=-1)
    zs = f32_to_bf16_bits(z) if dtype == DTYPE_BF16 else z
    z_eff = bf16_bits_to_f32(zs) if dtype == DTYPE_BF16 else z
    parent = random_tree_parents(r_p.rng, B, N)
    token = np.zeros((B, N), dtype=np.int32)
    noisy = _normal_f32(r_x, (B, N, V), sigma_x)
    noisy += z_eff
    for b in range(B):
        nkids = np.bincount(parent[b, 1:], minlength=N)
        for u in range(N):
            k = int(nkids[u])
            if k == 0:
                continue
            top = np.argpartition(-noisy[b, u], k - 1)[:k]
            top = top[np.argsort(-noisy[b, u, top], kind="stable")]
            token[b, np.flatnonzero(parent[b] == u)] = top
    del noisy
    return dict(kind="tree", dtype=dtype, B=B, N=N, V=V, temperature=float(np.float32(temperature)), target=zs,
                parent=parent, token=token, u_accept=uniforms(r_a, (B, N)), u_sample=uniforms(r_s, (B, N)))


# ----------------------------------------------------------------------------------------------------------------------
# The named workloads
# ----------------------------------------------------------------------------------------------------------------------

WORKLOADS = {
    # tiny dense instance, fp32
    "dense_tiny_B1_g4_V1024": lambda seed=0: dense_case(1, 4, 1024, dtype=DTYPE_F32, sigma_t=2.0, sigma_d=0.5,
                                                         temperature=1.0, seed=seed),
    # block-diffusion drafter block: B=64, gamma=16, V=151936, bf16, Zipf(1.1)-biased target
    "dense_block_B64_g16_V151936_bf16": lambda seed=0: dense_case(64, 16, 151936, dtype=DTYPE_BF16, sigma_t=3.0,
                                                                   sigma_d=1.0, zipf=1.1, temperature=1.0, seed=seed),
    # greedy (one-hot) drafter: B=256, gamma=8, V=128256, bf16, T=0.7
    "onehot_B256_g8_V128256_bf16": lambda seed=0: onehot_case(256, 8, 128256, dtype=DTYPE_BF16, sigma_t=2.5,
                                                              sigma_x=1.5, temperature=0.7, seed=seed),
    # sparse top-64 supports: B=1024, gamma=16, V=151936
    "sparse_B1024_g16_k64_V151936": lambda seed=0: sparse_case(1024, 16, 64, 151936, seed=seed),
    # masked-diffusion window: B=32, W=32, V=262144, fp32, 4 rounds
    "window_B32_W32_V262144_r4": lambda seed=0: window_case(32, 32, 262144, rounds=4, seed=seed),
    # token trees: B=64 trees of 17 nodes (root + 16 drafted, the Uno page's B = 16 tree sampler), V=151936, bf16
    "tree_B64_N17_V151936_bf16": lambda seed=0: tree_case(64, 17, 151936, dtype=DTYPE_BF16, seed=seed),
}


def make(name: str, seed: int = 0) -> dict:
    return WORKLOADS[name](seed)
