"""GPU parity of tree verification (sv_verify_tree, through the C ABI) against the float64 oracle (oracle/tree.py).

Decision parity: where the walks agree, the accepted nodes, the path and the flags match exactly and the drawn token
matches except where the oracle's CDF margin is below 1e-5; where they differ, the first differing test must sit at an
oracle margin |u - min(1, p'(x))| below 1e-5, and such sequences stay under 1e-4 of the tests made. p'(x) of every
tested node agrees to 1e-5 relative (float32 logits) or 2e-3 (bfloat16 logits).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from lossless_draft_verification_spec_amd import workloads as W

from gpu_helpers import MARGIN, RTOL, t_, t_logits

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_cases.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_draft_verification_spec_amd import sv  # noqa: F401  (raises if the library is missing)


def run_tree(case, target=None, ws=None):
    from lossless_draft_verification_spec_amd import sv
    tgt = t_logits(case["target"], case["dtype"]) if target is None else target
    out = sv.sv_verify_tree(tgt, t_(case["parent"], torch.int32), t_(case["token"], torch.int32),
                            t_(case["u_accept"], torch.float32), t_(case["u_sample"], torch.float32),
                            case["temperature"], ws=ws)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["flags"] = res["flags"].astype(np.uint32)
    return res


def run_oracle(case):
    return oracle.verify_tree(case["target"], case["parent"], case["token"], case["u_accept"], case["u_sample"],
                              case["temperature"], dtype=case["dtype"])


def compare_tree(g, o, dtype, label):
    B = o["n_accepted"].shape[0]
    tested_o = o["tested"].astype(bool)
    tested_g = ~np.isnan(g["p_test"])
    n_tests = int(tested_o.sum())
    bad, near_cdf = 0, 0
    for b in range(B):
        same_walk = (g["n_accepted"][b] == o["n_accepted"][b] and np.array_equal(g["path"][b], o["path"][b])
                     and np.array_equal(tested_g[b], tested_o[b]))
        if same_walk:
            assert np.array_equal(g["accept"][b], o["accept"][b]), (label, b)
            if g["out_token"][b] != o["out_token"][b]:
                assert o["margin_cdf"][b] < MARGIN, (label, b, g["out_token"][b], o["out_token"][b],
                                                     o["margin_cdf"][b])
                bad += 1
            else:
                assert g["flags"][b] == o["flags"][b], (label, b, g["flags"][b], o["flags"][b])
            t = tested_o[b]
            if t.any():
                np.testing.assert_allclose(g["p_test"][b, t], o["p_test"][b, t], rtol=RTOL[dtype], atol=1e-30,
                                           err_msg=f"{label} b={b}")
        else:
            both = tested_o[b] & tested_g[b]
            differ = both & (g["accept"][b] != o["accept"][b])
            assert differ.any(), (label, b, "walks differ without a differing test")
            first = int(np.flatnonzero(differ)[0])
            assert o["margin_accept"][b, first] < MARGIN, (label, b, first, o["margin_accept"][b, first])
            bad += 1
        near_cdf += int(o["margin_cdf"][b] < MARGIN)
    assert bad <= max(1e-4 * n_tests, 0), f"{label}: {bad} disagreeing sequences over {n_tests} tests"
    return dict(sequences=B, tests=n_tests, disagreements=bad, near_ties_cdf=near_cdf,
                mean_accepted=float(np.mean(np.maximum(o["n_accepted"], 0))))


SHAPES = [
    # B, N, V, dtype, T, parent chain probability
    (16, 17, 50_000, "bf16", 1.0, 0.5),
    (8, 9, 12_345, "f32", 0.7, 0.5),
    (5, 40, 4_099, "bf16", 1.3, 0.2),
    (3, 1, 2_000, "f32", 1.0, 0.5),             # the root alone: a bonus draw
    (12, 6, 257, "f32", 0.5, 0.8),
    (2, 200, 31_000, "bf16", 1.0, 0.9),         # deep trees
]


@pytest.mark.parametrize("idx", range(len(SHAPES)), ids=["B{}_N{}_V{}_{}_T{}".format(*s[:5]) for s in SHAPES])
def test_tree_shapes(idx):
    B, N, V, dt, T, pc = SHAPES[idx]
    print(f"tree shape {SHAPES[idx]}", flush=True)
    case = W.tree_case(B, N, V, dtype=dt, temperature=T, seed=200 + idx)
    if pc != 0.5:
        case["parent"] = W.random_tree_parents(np.random.default_rng(idx), B, N, p_chain=pc)
        case = _retoken(case)
    g = run_tree(case)
    print(f"  {compare_tree(g, run_oracle(case), dt, f'tree {SHAPES[idx]}')}", flush=True)


@pytest.mark.parametrize("N", [63, 64, 65])
def test_tree_sizes_at_the_walk_boundary(N):
    """Trees of 63, 64 and 65 nodes: up to 64 nodes the walk evaluates every node's test at once (one lane per node,
    the 64th lane included), from 65 on it walks level by level; deep and bushy trees of each size, both dtypes, and
    a root with all the other nodes as children (sibling masks of 63 and 64 bits)."""
    for dt, pc, seed in (("bf16", 0.3, 301), ("f32", 0.8, 302)):
        case = W.tree_case(9, N, 20_000, dtype=dt, seed=seed + N)
        case["parent"] = W.random_tree_parents(np.random.default_rng(seed + N), 9, N, p_chain=pc)
        case = _retoken(case)
        print(f"tree N={N} {dt}: {compare_tree(run_tree(case), run_oracle(case), dt, f'N={N} {dt}')}", flush=True)
    case = W.tree_case(4, N, 9_000, dtype="f32", seed=303 + N)
    case["parent"][:] = 0
    case["parent"][:, 0] = -1
    case = _retoken(case)
    case["token"][:, 1:] = case["token"][:, 1:][:, ::-1]     # the root's top candidate on its last child
    case["u_accept"][:] = np.float32(0.97)                  # long sibling walks at the root
    r = compare_tree(run_tree(case), run_oracle(case), 'f32', f'star N={N}')
    print(f"star N={N}: {r}", flush=True)
    assert r["tests"] > 4 * (N - 1) // 2                      # most siblings were tested


@pytest.mark.parametrize("B,N,dt", [(2, 9, "bf16"), (2, 5, "f32")])
def test_tree_rows_cut_into_many_pieces(B, N, dt):
    """A few rows of V = 600,001: the launch cuts every row into as many pieces as fill a resident round (56 pieces
    of the 18 bf16 rows, the most the merge takes, 64, of the 10 float32 rows), merged one lane per piece."""
    case = W.tree_case(B, N, 600_001, dtype=dt, seed=321 + N)
    r = compare_tree(run_tree(case), run_oracle(case), dt, f"pieces B={B} N={N} {dt}")
    print(f"tree pieces B={B} N={N} {dt}: {r}", flush=True)


def test_tree_faults_inside_pieces():
    """Rows of 600,001 float32 logits cut into pieces: a NaN in the root row's last piece and a +inf in a middle
    piece of a row on the walk's path make those sequences non-finite once the pieces are merged; the third tree
    is clean."""
    case = W.tree_case(3, 5, 600_001, dtype="f32", seed=331)
    case["target"][0, 0, 600_001 - 3] = np.nan
    case["target"][1, 1, 300_000] = np.inf
    g, o = run_tree(case), run_oracle(case)
    r = compare_tree(g, o, "f32", "faults inside pieces")
    assert (g["flags"][:2] & oracle.FLAG_NONFINITE).all() and (g["n_accepted"][:2] == -1).all()
    assert g["flags"][2] == o["flags"][2] == 0
    print(f"tree faults inside pieces: {r}, flags {g['flags'].tolist()}", flush=True)


@pytest.mark.parametrize("shape", ["chain", "random", "star"])
def test_tree_at_the_largest_size(shape):
    """Trees of SV_MAX_TREE_NODES = 1024 nodes: a single chain (the walk descends up to 1023 levels), a random
    recursive tree, and a root with 1023 children (1023 masked tokens in the root's row, siblings tested in chunks of
    64 with first-holder checks across chunks)."""
    from lossless_draft_verification_spec_amd import sv
    N = sv.SV_MAX_TREE_NODES
    case = W.tree_case(2, N, 3_000, dtype="bf16", seed=311)
    if shape == "chain":
        case["parent"] = W.random_tree_parents(np.random.default_rng(312), 2, N, p_chain=1.0)
        case["u_accept"][0] = np.float32(0.0)                  # every test passes: down to the leaf
    elif shape == "random":
        case["parent"] = W.random_tree_parents(np.random.default_rng(313), 2, N, p_chain=0.0)
    else:
        case["parent"][:] = 0
        case["parent"][:, 0] = -1
    case = _retoken(case)
    if shape == "star":
        case["token"][:, 1:] = case["token"][:, 1:][:, ::-1]   # the root's top candidate on its last child
        case["u_accept"][:] = np.float32(0.97)
    o = run_oracle(case)
    r = compare_tree(run_tree(case), o, "bf16", f"N={N} {shape}")
    print(f"tree N={N} {shape}: {r}", flush=True)
    if shape == "chain":
        assert o["n_accepted"][0] == N - 1
    if shape == "star":
        assert r["tests"] == 2 * (N - 1)


def _retoken(case):
    """Children tokens for a new parent array: the top candidates of each node's row, in decreasing order."""
    z = oracle.widen(case["target"], case["dtype"])
    for b in range(case["B"]):
        for u in range(case["N"]):
            kids = np.flatnonzero(case["parent"][b] == u)
            if kids.size:
                case["token"][b, kids] = np.argsort(-z[b, u], kind="stable")[:kids.size]
    return case


def test_tree_unaligned_and_strided_rows():
    for dt in ("f32", "bf16"):
        case = W.tree_case(6, 9, 20_001, dtype=dt, seed=211)
        B, N, V = case["B"], case["N"], case["V"]
        big = np.zeros((B, N, V + 13), dtype=case["target"].dtype)
        big[:, :, 3:V + 3] = case["target"]
        g = run_tree(case, target=t_logits(big, dt)[:, :, 3:V + 3])
        print(f"strided {dt}: {compare_tree(g, run_oracle(case), dt, 'strided ' + dt)}", flush=True)


def test_many_children_in_one_thread_share():
    """A root with 150 children whose tokens fall in one thread's share of the row stream (multiples of 2048 for
    bf16 and 1024 for float32): more masked elements than a thread lists, so the row takes the exact slow path; the
    walk lists children over several 64-node chunks."""
    for dt, step in (("bf16", 2048), ("f32", 1024)):
        B, N, V = 3, 151, 400_000
        case = W.tree_case(B, N, V, dtype=dt, seed=212)
        case["parent"][:] = 0
        case["parent"][:, 0] = -1
        case["token"][:, 1:] = (np.arange(1, N) * step) % V
        case["u_accept"][:] = np.float32(0.999)                 # most children rejected: long sibling walks
        case["u_accept"][1, 100] = 0.0                           # sequence 1 accepts child 100
        g = run_tree(case)
        print(f"many children {dt}: {compare_tree(g, run_oracle(case), dt, 'many children ' + dt)}", flush=True)


def test_chain_trees_equal_the_onehot_entry_point():
    from lossless_draft_verification_spec_amd import sv
    case = W.onehot_case(16, 7, 30_011, dtype="bf16", temperature=0.8, seed=213)
    B, G = case["B"], case["gamma"]
    tree = dict(dtype="bf16", temperature=case["temperature"], target=case["target"],
                parent=np.tile(np.arange(-1, G, dtype=np.int32), (B, 1)),
                token=np.concatenate([np.zeros((B, 1), np.int32), case["draft_ids"]], axis=1),
                u_accept=np.concatenate([np.zeros((B, 1), np.float32), case["u_accept"]], axis=1),
                u_sample=case["u_sample"])
    g = run_tree(tree)
    oh = sv.sv_verify_onehot_draft(t_logits(case["target"], "bf16"), t_(case["draft_ids"], torch.int32),
                                   t_(case["u_accept"], torch.float32), t_(case["u_sample"], torch.float32),
                                   case["temperature"], bonus=1)
    torch.cuda.synchronize()
    o = run_oracle(tree)
    print(f"chains: {compare_tree(g, o, 'bf16', 'chains')}", flush=True)
    n_oh = oh["n_accepted"].cpu().numpy()
    agree = (g["n_accepted"] == n_oh)
    assert agree.mean() > 0.9
    assert np.array_equal(g["out_token"][agree & (o["margin_cdf"] > MARGIN)],
                          oh["out_token"].cpu().numpy()[agree & (o["margin_cdf"] > MARGIN)])


def test_golden_trees_on_gpu():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        zt = np.log(np.array(c["p"])).astype(np.float32)[None]
        case = dict(dtype="f32", temperature=c["T"], target=zt, parent=np.array([c["parent"]], np.int32),
                    token=np.array([c["token"]], np.int32), u_accept=np.array([c["u_accept"]], np.float32),
                    u_sample=np.array([c["u_sample"]], np.float32))
        g = run_tree(case)
        assert list(g["accept"][0]) == c["accept"], c["name"]
        assert g["n_accepted"][0] == c["n_accepted"] and g["out_token"][0] == c["out_token"], c["name"]
        assert list(g["path"][0][:c["n_accepted"]]) == c["path"], c["name"]
        want = np.array([np.nan if v is None else v for v in c["p_test"]])
        np.testing.assert_allclose(g["p_test"][0], want, rtol=1e-5, atol=1e-30)


def test_tree_faults_and_empty_residual():
    rng = np.random.default_rng(6)
    B, N, V = 6, 4, 7
    zt = rng.normal(0, 1, (B, N, V)).astype(np.float32)
    parent = np.tile(np.array([-1, 0, 1, 1], np.int32), (B, 1))
    token = rng.integers(0, V, (B, N)).astype(np.int32)
    ua = np.zeros((B, N), np.float32)
    us = np.full((B, N), 0.5, np.float32)
    parent[1, 3] = 3
    token[2, 2] = V
    zt[3, 1, 2] = np.nan
    zt[4, 3, :] = np.nan
    # sequence 5: a root over 3 tokens whose 3 children carry every token and all fail (u = 1): empty residual
    zt[5] = np.log(np.array([0.5, 0.3, 0.2, 1e-30, 1e-30, 1e-30, 1e-30]))
    zt[5, :, 3:] = -np.inf
    parent[5] = [-1, 0, 0, 0]
    token[5] = [0, 0, 1, 2]
    ua[5] = 1.0
    case = dict(dtype="f32", temperature=1.0, target=zt, parent=parent, token=token, u_accept=ua, u_sample=us)
    g = run_tree(case)
    o = run_oracle(case)
    for k in ("accept", "n_accepted", "path", "out_token", "flags"):
        assert np.array_equal(g[k], o[k]), (k, g[k], o[k])
    assert g["flags"][1] == oracle.FLAG_ID_RANGE and g["flags"][3] == oracle.FLAG_NONFINITE
    assert g["flags"][5] == oracle.FLAG_EMPTY_RESIDUAL and g["n_accepted"][5] == 0


def test_tree_workload_full_size_and_workspace_shared_with_dense():
    """The tree workload at full size (64 trees of 17 nodes over V = 151936, bf16), in the benchmark's launch
    configuration, against the oracle on every sequence; the same workspace then serves a dense call and the tree
    call again (the control words of each layout are cleared inside the launch when the layout changes)."""
    from lossless_draft_verification_spec_amd import sv
    case = W.make("tree_B64_N17_V151936_bf16")
    o = run_oracle(case)
    dense = W.dense_case(5, 4, 30_000, dtype="bf16", seed=214)
    n = max(sv.sv_workspace_bytes(sv.SV_KIND_TREE, 64, 17, 151936), sv.sv_workspace_bytes(sv.SV_KIND_DENSE, 5, 4, 30_000))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    g1 = run_tree(case, ws=ws)
    print(f"tree full: {compare_tree(g1, o, 'bf16', 'tree full')}", flush=True)
    sv.sv_verify_dense(t_logits(dense["target"], "bf16"), t_logits(dense["draft"], "bf16"),
                       t_(dense["draft_ids"], torch.int32), t_(dense["u_accept"], torch.float32),
                       t_(dense["u_sample"], torch.float32), dense["temperature"], ws=ws)
    g2 = run_tree(case, ws=ws)
    for k in g1:
        assert np.array_equal(g1[k], g2[k], equal_nan=True), k
