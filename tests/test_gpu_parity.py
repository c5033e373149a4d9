"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded inputs.

Small cases run the oracle on every sequence and span several tiles of both passes with ragged heads and tails;
the full-size workloads run the exact launch configuration the benchmark times and compare the oracle on every or
on sampled sequences. Decision parity and tolerances are described in gpu_helpers.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from lossless_draft_verification_spec_amd import workloads as W

from gpu_helpers import (compare_decisions, compare_probs, dev, host, oracle_dense, run_dense, run_onehot,
                         run_sparse, t_, t_logits)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rule_cases.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_draft_verification_spec_amd import sv  # noqa: F401  (raises if the library is missing)


def log(msg):
    print(msg, flush=True)


# ----------------------------------------------------------------------------------------------------------------------
# dense
# ----------------------------------------------------------------------------------------------------------------------

def check_dense(case, label, **kw):
    g = run_dense(case, **kw)
    o = oracle_dense(case, **kw)
    s = compare_decisions(g, o, label)
    compare_probs(g, o, "p_draft", case["dtype"], label)
    compare_probs(g, o, "q_draft", case["dtype"], label)
    log(f"{label}: {s}")
    return g, o


def test_dense_tiny_workload():
    case = W.make("dense_tiny_B1_g4_V1024")
    g, o = check_dense(case, "dense tiny")
    assert np.array_equal(g["accept"], o["accept"]) and np.array_equal(g["out_token"], o["out_token"])


DENSE_SHAPES = [
    # B, gamma, V, dtype, T, bonus, sigma_t, sigma_d, zipf
    (3, 5, 50_000, "bf16", 1.0, 1, 3.0, 1.0, 1.1),
    (2, 3, 100_003, "f32", 0.7, 1, 2.0, 0.5, 0.0),
    (5, 1, 4_099, "bf16", 1.3, 1, 2.0, 0.3, 0.0),
    (1, 16, 12_345, "f32", 1.0, 0, 2.5, 1.0, 0.0),
    (7, 4, 1_031, "bf16", 0.5, 1, 1.0, 0.2, 0.0),
    (4, 8, 257, "f32", 2.0, 1, 2.0, 0.1, 0.0),
    (2, 2, 9, "f32", 1.0, 1, 1.0, 1.0, 0.0),
    (33, 2, 3_000, "bf16", 1.0, 1, 2.0, 0.05, 0.0),
]


@pytest.mark.parametrize("idx", range(len(DENSE_SHAPES)),
                         ids=["B{}_g{}_V{}_{}_T{}_b{}".format(*s[:6]) for s in DENSE_SHAPES])
def test_dense_shapes(idx):
    shape = DENSE_SHAPES[idx]
    B, G, V, dt, T, bonus, st, sd, zipf = shape
    case = W.dense_case(B, G, V, dtype=dt, sigma_t=st, sigma_d=sd, zipf=zipf, temperature=T, bonus=bonus,
                        seed=100 + idx)
    check_dense(case, f"dense {shape}")


def test_dense_unaligned_and_strided_rows():
    """Rows that start off 16-byte boundaries and a padded row stride (head/tail peeling of the vector loads)."""
    B, G, V = 3, 4, 20_001
    for dt in ("f32", "bf16"):
        case = W.dense_case(B, G, V, dtype=dt, seed=5)
        pad = 13
        tgt_np = np.zeros((B, G + 1, V + pad), dtype=case["target"].dtype)
        tgt_np[:, :, 1:V + 1] = case["target"]
        dft_np = np.zeros((B, G, V + pad), dtype=case["draft"].dtype)
        dft_np[:, :, 3:V + 3] = case["draft"]
        tgt = t_logits(tgt_np, dt)[:, :, 1:V + 1]
        dft = t_logits(dft_np, dt)[:, :, 3:V + 3]
        g = run_dense(case, target=tgt, draft=dft)
        o = oracle_dense(case)
        log(f"strided {dt}: {compare_decisions(g, o, 'strided ' + dt)}")
        compare_probs(g, o, "p_draft", dt)


def test_dense_q_equals_p_accepts_all():
    case = W.dense_case(6, 7, 30_000, dtype="bf16", sigma_d=0.0, seed=11)
    case["draft"] = np.ascontiguousarray(case["target"][:, :7])
    g = run_dense(case)
    assert np.all(g["accept"] == 1) and np.all(g["n_accepted"] == 7)
    o = oracle_dense(case)
    compare_decisions(g, o, "q=p")
    assert np.array_equal(g["p_draft"], g["q_draft"])


def test_dense_masked_vocab_and_onehot_through_dense():
    B, G, V = 4, 5, 6_000
    case = W.dense_case(B, G, V, dtype="f32", seed=12)
    rng = np.random.default_rng(0)
    mask = rng.random(V) < 0.3
    mask[case["draft_ids"].ravel()] = False
    case["target"][:, :, mask] = -np.inf
    case["draft"][:, :, mask] = -np.inf
    check_dense(case, "masked vocab")
    # one-hot drafts through the dense entry point == the one-hot entry point
    d = case["draft_ids"]
    oh = np.full((B, G, V), -np.inf, np.float32)
    np.put_along_axis(oh, d[..., None].astype(np.int64), 0.0, axis=-1)
    case2 = dict(case, draft=oh)
    g_dense = run_dense(case2)
    g_oh = run_onehot(case)
    o = oracle_dense(case, onehot=True)
    compare_decisions(g_dense, o, "one-hot via dense")
    compare_decisions(g_oh, o, "one-hot")
    assert np.array_equal(g_dense["n_accepted"], g_oh["n_accepted"])


def test_dense_data_faults():
    B, G, V = 8, 3, 700
    case = W.dense_case(B, G, V, dtype="f32", seed=13)
    zt, zd, ids = case["target"], case["draft"], case["draft_ids"]
    zt[0, 1, 4] = np.nan
    zd[1, 2, :] = -np.inf
    ids[2, 0] = V
    ids[3, 1] = -1
    zd[4, 0, ids[4, 0]] = -np.inf
    case["u_accept"][4, 0] = 0.5
    zd[5] = zt[5, :G]
    zt[5, G, 9] = np.inf
    zt[6, 0, 10] = np.inf
    g = run_dense(case)
    o = oracle_dense(case)
    compare_decisions(g, o, "faults")
    compare_probs(g, o, "p_draft", "f32", "faults")
    assert g["flags"][0] & oracle.FLAG_NONFINITE and g["n_accepted"][0] == -1
    assert g["flags"][2] & oracle.FLAG_ID_RANGE and g["flags"][3] & oracle.FLAG_ID_RANGE
    assert g["flags"][4] & oracle.FLAG_Q_ZERO
    assert g["flags"][5] == oracle.FLAG_NONFINITE and g["out_token"][5] == -1 and g["n_accepted"][5] == G
    # start / order faults
    start = np.array([0, G, G + 1, -1, 1, 2, 0, 1], np.int32)
    order = np.tile(np.arange(G, dtype=np.int32), (B, 1))
    order[7] = [0, 0, 1]
    case2 = W.dense_case(B, G, V, dtype="f32", seed=14)
    g = run_dense(case2, start=start, order=order)
    o = oracle_dense(case2, start=start, order=order)
    compare_decisions(g, o, "start/order faults")
    assert g["n_accepted"][1] == 0 and g["out_token"][1] == -1 and g["start_out"][1] == G
    assert g["flags"][2] & oracle.FLAG_ID_RANGE and g["flags"][3] & oracle.FLAG_ID_RANGE
    assert g["flags"][7] & oracle.FLAG_ID_RANGE


def test_dense_faults_inside_later_segments():
    """Rows of 600,001 float32 logits are read as three statistics segments: a NaN in the last segment of a target
    row and a +inf in the middle segment of a draft row make their sequences non-finite once the segments' partials
    are merged; a draft row that is -inf past its first 1000 elements has q = 0 at its drafted id (Q_ZERO, the
    draft rejected) while its finite head still normalises the row."""
    B, G, V = 4, 2, 600_001
    case = W.dense_case(B, G, V, dtype="f32", seed=18)
    zt, zd = case["target"], case["draft"]
    zt[0, 1, V - 5] = np.nan
    zd[1, 0, V // 2] = np.inf
    zd[2, 1, 1000:] = -np.inf
    g = run_dense(case)
    o = oracle_dense(case)
    s = compare_decisions(g, o, "faults in later segments")
    compare_probs(g, o, "p_draft", "f32", "faults in later segments")
    assert g["flags"][0] & oracle.FLAG_NONFINITE and g["n_accepted"][0] == -1
    assert g["flags"][1] & oracle.FLAG_NONFINITE and g["n_accepted"][1] == -1
    assert g["flags"][2] & oracle.FLAG_Q_ZERO and g["n_accepted"][2] == o["n_accepted"][2]
    assert g["flags"][3] == o["flags"][3]
    log(f"faults in later segments: {s}, flags {g['flags'].tolist()}, n {g['n_accepted'].tolist()}")


@pytest.mark.parametrize("V", [30_000, 600_001])
def test_dense_near_equal_distributions(V):
    """Draft = target + tiny noise: the residual's sign is undecided for most elements, so the pick recomputes most
    chunks exactly. Uniforms near 1 force rejections."""
    B, G = 3, 2
    case = W.dense_case(B, G, V, dtype="f32", sigma_t=2.0, sigma_d=2e-5, seed=16)
    case["u_accept"][:] = np.float32(0.99999)
    g = run_dense(case)
    o = oracle_dense(case)
    s = compare_decisions(g, o, f"near-equal V={V}")
    compare_probs(g, o, "p_draft", "f32")
    log(f"near-equal V={V}: {s}, n {g['n_accepted'].tolist()}")
    assert (g["n_accepted"] < G).any()


def test_dense_rows_longer_than_one_pick_tile():
    """V = 1300003: more 1024-element chunks per row than the pick holds at once, so chunk masses go through global
    memory tile by tile. Sequence 0 accepts every draft (bonus draw over the long row); the others reject."""
    B, G, V = 3, 2, 1_300_003
    case = W.dense_case(B, G, V, dtype="f32", sigma_t=2.0, sigma_d=0.5, seed=17)
    case["u_accept"][0] = 0.0
    case["u_accept"][1:] = np.float32(0.99999)
    g = run_dense(case)
    o = oracle_dense(case)
    s = compare_decisions(g, o, "multi-tile")
    compare_probs(g, o, "p_draft", "f32")
    log(f"multi-tile: {s}, n {g['n_accepted'].tolist()}, tokens {g['out_token'].tolist()}")
    assert g["n_accepted"][0] == G and (g["n_accepted"][1:] < G).any()


def _side_by_side(*cases):
    """Cases of one shape and dtype as one batch (sequence order kept)."""
    out = dict(cases[0])
    for key in ("target", "draft", "draft_ids", "u_accept", "u_sample"):
        if out.get(key) is not None:
            out[key] = np.concatenate([c[key] for c in cases])
    out["B"] = sum(c["B"] for c in cases)
    return out


@pytest.mark.parametrize("dt,V", [("f32", 257), ("bf16", 1_031)])
def test_dense_at_the_largest_gamma(dt, V):
    """gamma = SV_MAX_GAMMA = 1024: 2048 statistics items per sequence and a scan over 1024 slots. Sequence 0's draft
    is the target up to a tiny perturbation (a long run of acceptances), sequence 1's differs (an early rejection);
    then the same batch along random orders from starts 0 and 700 (a 1024-slot permutation check)."""
    from lossless_draft_verification_spec_amd import sv
    G = sv.SV_MAX_GAMMA
    case = _side_by_side(W.dense_case(1, G, V, dtype=dt, sigma_t=1.0, sigma_d=1e-3, seed=71),
                         W.dense_case(1, G, V, dtype=dt, sigma_t=1.0, sigma_d=1.0, seed=72))
    g, o = check_dense(case, f"dense gamma={G} {dt}")
    log(f"  n_accepted {g['n_accepted'].tolist()}")
    assert o["n_accepted"][0] > 200 and o["n_accepted"][1] < 50
    rng = np.random.default_rng(73)
    order = np.stack([rng.permutation(G) for _ in range(2)]).astype(np.int32)
    g, o = check_dense(case, f"dense gamma={G} {dt} ordered", start=np.array([0, 700], np.int32), order=order)
    log(f"  n_accepted {g['n_accepted'].tolist()}, starts out {g['start_out'].tolist()}")


def test_onehot_at_the_largest_gamma():
    """One-hot drafts at gamma = 1024 whose drafted ids carry nearly all of the target's mass: sequence 0 accepts
    every slot and draws the bonus after 1024 rows; sequence 1 has one ordinary slot (600) with a uniform near 1, so
    it rejects there and draws from that row's residual."""
    from lossless_draft_verification_spec_amd import sv
    G = sv.SV_MAX_GAMMA
    case = W.onehot_case(2, G, 513, dtype="f32", temperature=0.7, seed=74)
    spike = np.ones((2, G), bool)
    spike[1, 600] = False
    b, j = np.nonzero(spike)
    case["target"][b, j, case["draft_ids"][b, j]] += np.float32(30.0)
    case["u_accept"][1, 600] = np.float32(0.99999)
    g = run_onehot(case)
    o = oracle_dense(case, onehot=True)
    log(f"onehot gamma={G}: {compare_decisions(g, o, f'onehot gamma={G}')}, n {g['n_accepted'].tolist()}")
    compare_probs(g, o, "p_draft", "f32")
    assert o["n_accepted"].tolist() == [G, 600]


def test_dense_is_deterministic():
    case = W.dense_case(4, 6, 40_000, dtype="bf16", seed=15)
    a, b = run_dense(case), run_dense(case)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_workspace_reused_across_shapes_and_kinds():
    """One workspace, zero-filled once, serves dense and one-hot calls of different shapes in a row: every call
    returns the work-queue counters, the draw ticket and the job slots to their start state, so each call matches the
    oracle and a repeated call repeats its outputs bit for bit."""
    from lossless_draft_verification_spec_amd import sv
    a = W.dense_case(5, 4, 50_000, dtype="bf16", sigma_t=3.0, sigma_d=1.0, seed=41)
    b = W.onehot_case(7, 6, 20_011, dtype="bf16", temperature=0.8, seed=42)
    c = W.dense_case(33, 2, 3_000, dtype="f32", sigma_t=2.0, sigma_d=0.3, seed=43)
    need = int(max(sv.sv_workspace_bytes(sv.SV_KIND_DENSE, 5, 4, 50_000),
                   sv.sv_workspace_bytes(sv.SV_KIND_ONEHOT, 7, 6, 20_011),
                   sv.sv_workspace_bytes(sv.SV_KIND_DENSE, 33, 2, 3_000)))
    raw = torch.zeros(need + 256, dtype=torch.uint8, device="cuda")     # zero-filled once, 256-byte aligned view
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + need]
    first = None
    for i, (case, kind) in enumerate([(a, "dense"), (b, "onehot"), (c, "dense"), (a, "dense"), (b, "onehot")]):
        if kind == "dense":
            g = run_dense(case, ws=ws)
            o = oracle_dense(case)
        else:
            g = run_onehot(case, ws=ws)
            o = oracle_dense(case, onehot=True)
        log(f"workspace reuse call {i} ({kind}): {compare_decisions(g, o, f'reuse {i}')}")
        if i == 0:
            first = g
        if i == 3:
            for k in first:
                assert np.array_equal(first[k], g[k], equal_nan=True), k


def test_dense_block_workload_full_size():
    """The dense block workload at its full size (B=64, gamma=16, V=151936, bf16) in the benchmark's launch
    configuration; the oracle runs on every sequence."""
    case = W.make("dense_block_B64_g16_V151936_bf16")
    log("generated dense block workload")
    g = run_dense(case)
    log("gpu done")
    o = oracle_dense(case)
    s = compare_decisions(g, o, "dense block full")
    r = compare_probs(g, o, "p_draft", "bf16")
    compare_probs(g, o, "q_draft", "bf16")
    log(f"dense block full: {s}, max rel err p {r:.3g}, mean n {g['n_accepted'].mean():.3f}")


# ----------------------------------------------------------------------------------------------------------------------
# one-hot (greedy drafter)
# ----------------------------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(4, 8, 30_011, "bf16", 0.7), (3, 3, 5_000, "f32", 1.0), (16, 2, 700, "bf16", 0.4)])
def test_onehot_shapes(shape):
    B, G, V, dt, T = shape
    case = W.onehot_case(B, G, V, dtype=dt, temperature=T, seed=21)
    g = run_onehot(case)
    o = oracle_dense(case, onehot=True)
    log(f"onehot {shape}: {compare_decisions(g, o, f'onehot {shape}')}")
    compare_probs(g, o, "p_draft", dt)


def test_onehot_workload_full_size():
    """Greedy-draft workload at full size (B=256, gamma=8, V=128256, bf16, T=0.7), the benchmark's launch
    configuration; the oracle runs on every sequence."""
    case = W.make("onehot_B256_g8_V128256_bf16")
    log("generated one-hot workload")
    g = run_onehot(case)
    log("gpu done")
    o = oracle_dense(case, onehot=True)
    s = compare_decisions(g, o, "onehot full")
    compare_probs(g, o, "p_draft", "bf16")
    log(f"onehot full: {s}, mean n {g['n_accepted'].mean():.3f}")


# ----------------------------------------------------------------------------------------------------------------------
# sparse
# ----------------------------------------------------------------------------------------------------------------------

def check_sparse_exact(g, o, label):
    for k in ("accept", "n_accepted", "out_token", "flags"):
        assert np.array_equal(g[k].astype(np.int64), o[k].astype(np.int64)), f"{label}: {k}"
    for k in ("p_spec", "q_spec", "correction_probs"):
        want = o[k].astype(np.float32)
        assert np.array_equal(g[k], want, equal_nan=True), f"{label}: {k}"


@pytest.mark.parametrize("shape", [(8, 5, 64, 1000), (3, 16, 17, 200), (5, 2, 256, 100_000), (40, 1, 1, 10),
                                   (3, 30, 64, 5000), (2, 7, 256, 100_000), (2, 70, 128, 3000)])
def test_sparse_shapes_bit_exact(shape):
    B, G, k, V = shape
    case = W.sparse_case(B, G, k, V, shared=max(1, k // 2), seed=31)
    g = run_sparse(case, vocab_size=V)
    o = oracle.verify_sparse(case["p_ids"], case["p_probs"], case["q_ids"], case["q_probs"], case["spec_ids"],
                             case["u_accept"], case["u_sample"], bonus=1, vocab_size=V)
    check_sparse_exact(g, o, f"sparse {shape}")


@pytest.mark.parametrize("k", [16, 256])
def test_sparse_at_the_largest_gamma(k):
    """gamma = SV_MAX_GAMMA = 1024 slots (several batches of correction weights in LDS). Sequence 0's draft support is
    its target support (q = p at every slot: every draft is accepted and the bonus is drawn after 1024 slots);
    sequence 1 is random (an early rejection)."""
    from lossless_draft_verification_spec_amd import sv
    G, V = sv.SV_MAX_GAMMA, 50_000
    case = W.sparse_case(2, G, k, V, shared=max(1, k // 2), seed=75)
    case["q_ids"][0] = case["p_ids"][0, :G]
    case["q_probs"][0] = case["p_probs"][0, :G]
    case["spec_ids"][0] = case["q_ids"][0, :, 0]
    g = run_sparse(case, vocab_size=V)
    o = oracle.verify_sparse(case["p_ids"], case["p_probs"], case["q_ids"], case["q_probs"], case["spec_ids"],
                             case["u_accept"], case["u_sample"], bonus=1, vocab_size=V)
    check_sparse_exact(g, o, f"sparse gamma={G} k={k}")
    assert o["n_accepted"][0] == G and o["n_accepted"][1] < G


def test_sparse_faults_and_fallback():
    case = W.sparse_case(6, 3, 8, 50, seed=32)
    case["p_probs"][0, 1, 2] = np.nan
    case["q_ids"][1, 0, 0] = 50                      # out of the vocabulary
    case["q_probs"][2] = 0.0                          # q_spec = 0 everywhere: rejections with Q_ZERO
    case["q_ids"][3] = case["p_ids"][3, :3]           # q dominates p on p's support: empty residual
    case["q_probs"][3] = 0.95
    g = run_sparse(case, vocab_size=50)
    o = oracle.verify_sparse(case["p_ids"], case["p_probs"], case["q_ids"], case["q_probs"], case["spec_ids"],
                             case["u_accept"], case["u_sample"], bonus=1, vocab_size=50)
    check_sparse_exact(g, o, "sparse faults")


def test_sparse_faults_across_batches():
    """gamma = 1024 slots in batches of correction weights (96 slots a batch at k = 16): a NaN probability and an
    out-of-vocabulary id in late batches, q = 0 at every drafted id, a bad bonus row after 1024 accepted slots, and an
    empty residual at slot 800 after 800 accepted ones; the kernel checks the rows batch by batch here, not all at
    once."""
    from lossless_draft_verification_spec_amd import sv
    G, k, V = sv.SV_MAX_GAMMA, 16, 5000
    case = W.sparse_case(6, G, k, V, seed=33)
    pi, pp, qi, qp, sp, ua = (case[x] for x in ("p_ids", "p_probs", "q_ids", "q_probs", "spec_ids", "u_accept"))
    pp[0, 900, 3] = np.nan
    qi[1, 700, 0] = V
    qp[2] = 0.0
    for b in (3, 4):                                   # q = p: every draft accepted
        qi[b], qp[b] = pi[b, :G], pp[b, :G]
        sp[b] = qi[b, :, 0]
    pp[3, G, 5] = np.nan                               # the bonus row
    qp[4, 800] = 2.0 * pp[4, 800]                      # q dominates p at slot 800, which then rejects
    ua[4, 800] = np.float32(0.9)
    g = run_sparse(case, vocab_size=V)
    o = oracle.verify_sparse(pi, pp, qi, qp, sp, ua, case["u_sample"], bonus=1, vocab_size=V)
    check_sparse_exact(g, o, "sparse faults across batches")
    log(f"sparse faults across batches: flags {g['flags'].tolist()}, n {g['n_accepted'].tolist()}")


def _one_bucket(n, bits, bucket, rng):
    """n distinct ids in [0, 2^24) that the kernel's index of q (2^bits buckets of a multiplicative hash) sends to
    one bucket, so that all but one of a support's entries lose it and take the kernel's slower matching."""
    ids = np.arange(1 << 24, dtype=np.int64)
    h = ((ids * 0x9E3779B1) & 0xFFFFFFFF) >> (32 - bits)
    pool = ids[h == bucket]
    assert pool.size >= n
    return rng.choice(pool, size=n, replace=False).astype(np.int32)


@pytest.mark.parametrize("k,bits", [(64, 8), (50, 8), (128, 9), (256, 10)])
def test_sparse_colliding_repeated_and_unchecked_ids(k, bits):
    """Supports whose ids all share one bucket of the kernel's index of q, q and p supports with repeated ids
    (matches summed in slot order, as the routine's id-equality gathers do), and, with the vocabulary unchecked, ids
    -1, 0 and the most negative int32. Bit-exact against the oracle."""
    rng = np.random.default_rng(k)
    case = W.sparse_case(6, 4, k, 1 << 24, shared=k // 2, seed=40 + k)
    G = case["gamma"]
    for b in range(6):
        for j in range(G + 1):
            ids = _one_bucket(2 * k, bits, (1 << bits) - 1, rng)
            case["p_ids"][b, j] = ids[:k]
            if j < G:
                q = np.concatenate([rng.choice(ids[:k], k // 2, replace=False), ids[k:k + k - k // 2]])
                case["q_ids"][b, j] = rng.permutation(q)
    case["q_ids"][1, :, 1] = case["q_ids"][1, :, 0]   # q repeats an id (shared with p or not)
    case["p_ids"][2, :, 2] = case["p_ids"][2, :, 0]   # p repeats an id
    case["q_ids"][2, 0, 3] = case["p_ids"][2, 0, 0]
    for c, v in ((3, -1), (4, 0), (5, np.iinfo(np.int32).min)):
        case["p_ids"][c, :, 0] = v                    # unchecked ids when vocab_size = 0
        case["q_ids"][c, :, 1] = v
    slot = rng.integers(0, k, size=(6, G))
    case["spec_ids"] = np.take_along_axis(case["q_ids"], slot[..., None], axis=-1)[..., 0].astype(np.int32)
    for vocab in (0, 1 << 24):
        if vocab:
            for key in ("p_ids", "q_ids", "spec_ids"):
                case[key] = np.where(case[key] < 0, 7, case[key]).astype(np.int32)
        g = run_sparse(case, vocab_size=vocab)
        o = oracle.verify_sparse(case["p_ids"], case["p_probs"], case["q_ids"], case["q_probs"], case["spec_ids"],
                                 case["u_accept"], case["u_sample"], bonus=1, vocab_size=vocab)
        check_sparse_exact(g, o, f"colliding ids k={k} vocab={vocab}")


def test_sparse_workload_full_size_bit_exact():
    case = W.make("sparse_B1024_g16_k64_V151936")
    g = run_sparse(case, vocab_size=case["V"])
    o = oracle.verify_sparse(case["p_ids"], case["p_probs"], case["q_ids"], case["q_probs"], case["spec_ids"],
                             case["u_accept"], case["u_sample"], bonus=1, vocab_size=case["V"])
    check_sparse_exact(g, o, "sparse full")
    log(f"sparse full: mean n {g['n_accepted'].mean():.3f}")


# ----------------------------------------------------------------------------------------------------------------------
# golden hand-derived cases through the GPU
# ----------------------------------------------------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_cases_on_gpu():
    gd = _golden()
    for c in gd["dense"]:
        scale = c.get("logit_scale", 1.0)
        zt = (scale * np.log(np.array(c["p"]))).astype(np.float32)[None]
        zd = (scale * np.log(np.array(c["q"]))).astype(np.float32)[None]
        case = dict(dtype="f32", target=zt, draft=zd, draft_ids=np.array([c["draft_ids"]], np.int32),
                    u_accept=np.array([c["u_accept"]], np.float32), u_sample=np.array([c["u_sample"]], np.float32),
                    temperature=c["T"], bonus=1)
        g = run_dense(case)
        assert list(g["accept"][0]) == c["accept"], c["name"]
        assert g["n_accepted"][0] == c["n_accepted"] and g["out_token"][0] == c["out_token"], c["name"]
    for c in gd["onehot"]:
        zt = np.log(np.array(c["p"])).astype(np.float32)[None]
        case = dict(dtype="f32", target=zt, draft_ids=np.array([c["draft_ids"]], np.int32),
                    u_accept=np.array([c["u_accept"]], np.float32), u_sample=np.array([c["u_sample"]], np.float32),
                    temperature=c["T"], bonus=1)
        g = run_onehot(case)
        assert g["n_accepted"][0] == c["n_accepted"] and g["out_token"][0] == c["out_token"], c["name"]
    for c in gd["sparse"]:
        case = dict(p_ids=np.array([c["p_ids"]], np.int32), p_probs=np.array([c["p_probs"]], np.float32),
                    q_ids=np.array([c["q_ids"]], np.int32), q_probs=np.array([c["q_probs"]], np.float32),
                    spec_ids=np.array([c["spec_ids"]], np.int32), u_accept=np.array([c["u_accept"]], np.float32),
                    u_sample=np.array([c["u_sample"]], np.float32), bonus=1)
        g = run_sparse(case)
        assert list(g["accept"][0]) == c["accept"], c["name"]
        assert g["n_accepted"][0] == c["n_accepted"] and g["out_token"][0] == c["out_token"], c["name"]
        if "flags" in c:
            assert g["flags"][0] == c["flags"], c["name"]


# ----------------------------------------------------------------------------------------------------------------------
# windows: several verification rounds chained on the device
# ----------------------------------------------------------------------------------------------------------------------

def run_window_rounds(case, seqs=None):
    """All rounds on the GPU with `start` kept on the device between calls; oracle on the selected sequences."""
    from lossless_draft_verification_spec_amd import sv
    tgt = t_logits(case["target"], "f32")
    dft = t_logits(case["draft"], "f32")
    ids = t_(case["draft_ids"], torch.int32)
    order = t_(case["order"], torch.int32)
    B = case["B"]
    start = torch.zeros(B, dtype=torch.int32, device=dev())
    outs = []
    for r in range(case["rounds"]):
        o = sv.sv_verify_dense(tgt, dft, ids, t_(case["u_accept"][r], torch.float32),
                               t_(case["u_sample"][r], torch.float32), case["temperature"], bonus=0, start=start,
                               order=order)
        res = host(o)
        res["start_out"] = start.cpu().numpy()
        outs.append(res)
    sl = slice(None) if seqs is None else seqs
    ora = oracle.verify_windows(case["target"][sl], case["draft"][sl], case["draft_ids"][sl],
                                case["u_accept"][:, sl], case["u_sample"][:, sl], case["temperature"],
                                order=case["order"][sl])
    for r, (g, o) in enumerate(zip(outs, ora)):
        gs = {k: v[sl] for k, v in g.items()}
        s = compare_decisions(gs, o, f"window round {r}")
        compare_probs(gs, o, "p_draft", "f32")
        log(f"window round {r}: {s}, starts {np.bincount(gs['start_out'], minlength=case['gamma'] + 1)}")
    return outs


def test_window_rounds_small():
    case = W.window_case(6, 12, 9_000, rounds=4, seed=41)
    run_window_rounds(case)


def test_window_workload_full_size():
    """Masked-diffusion window at full size (B=32, W=32, V=262144, fp32, 4 rounds), the benchmark's launch
    configuration; the oracle runs every round on every sequence."""
    case = W.make("window_B32_W32_V262144_r4")
    log("generated window workload")
    run_window_rounds(case)


def test_golden_window_rounds_on_gpu():
    """The hand-derived two-round window (tests/golden/rule_cases.json, "window"): rounds chained on the device
    through `start`, each with its own uniforms."""
    from lossless_draft_verification_spec_amd import sv
    for c in _golden()["window"]:
        zt = np.log(np.array(c["p"])).astype(np.float32)[None]
        zd = np.log(np.array(c["q"])).astype(np.float32)[None]
        start = torch.zeros(1, dtype=torch.int32, device=dev())
        for r, want in enumerate(c["rounds"]):
            out = sv.sv_verify_dense(t_logits(zt, "f32"), t_logits(zd, "f32"), t_(np.array([c["draft_ids"]]), torch.int32),
                                     t_(np.array([want["u_accept"]]), torch.float32),
                                     t_(np.array([want["u_sample"]]), torch.float32), c["T"], bonus=0, start=start,
                                     order=t_(np.array([c["order"]]), torch.int32))
            g = host(out)
            assert list(g["accept"][0]) == want["accept"], (c["name"], r)
            assert g["n_accepted"][0] == want["n_accepted"] and g["out_token"][0] == want["out_token"], (c["name"], r)
            assert int(start.cpu()[0]) == want["start_out"], (c["name"], r)
            np.testing.assert_allclose(g["p_draft"][0], want["p_draft"], rtol=1e-5, atol=1e-30)
