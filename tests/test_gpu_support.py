"""GPU parity of the top-k / top-p support builder (through the C ABI) against the float64 CPU oracle.

Integer outputs are exact: the k ids (top-k is integer work on the logits' order) and the kept count, except that a
count may differ where the oracle's cumulative top-k mass lies within 1e-12 of top_p (both sides decide in float64,
with their sums in different orders). Probabilities agree to 1e-6 relative when renormalised over the kept slots
(float64 arithmetic on at most k values, rounded to float32) and to 1e-5 relative for the full-softmax
probabilities (the full-row sum is accumulated in float32 partials). Faulted rows must match exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from lossless_draft_verification_spec_amd import workloads as W

from gpu_helpers import dev, t_logits

pytestmark = pytest.mark.gpu

COUNT_MARGIN = 1e-12


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_draft_verification_spec_amd import sv  # noqa: F401  (raises if the library is missing)


def run_support(z, dtype, k, top_p, T, renorm, *, ld_pad=0, ws=None):
    """z: [rows, V] float32 values or bf16 bits (numpy). ld_pad > 0 places the rows ld_pad elements apart beyond V."""
    from lossless_draft_verification_spec_amd import sv
    rows, V = z.shape
    if ld_pad:
        big = np.zeros((rows, V + ld_pad), dtype=z.dtype)
        big[:, :V] = z
        x = t_logits(big, dtype)[:, :V]
    else:
        x = t_logits(z, dtype)
    out = sv.sv_build_support(x, k, top_p, T, renorm, ws=ws)
    torch.cuda.synchronize()
    return {n: v.cpu().numpy() for n, v in out.items()}


def check(g, o, renorm, rows=None):
    rows = np.arange(o["ids"].shape[0]) if rows is None else rows
    gf = g["flags"][rows].astype(np.uint32)
    np.testing.assert_array_equal(gf, o["flags"])
    ok = o["flags"] == 0
    np.testing.assert_array_equal(g["ids"][rows][~ok], -1)
    assert np.isnan(g["probs"][rows][~ok]).all()
    np.testing.assert_array_equal(g["count"][rows][~ok], 0)
    np.testing.assert_array_equal(g["ids"][rows][ok], o["ids"][ok])
    gc, oc = g["count"][rows][ok], o["count"][ok]
    diff = gc != oc
    assert (o["margin"][ok][diff] < COUNT_MARGIN).all(), "a kept count differs away from a near-tie"
    same = ok.copy()
    same[ok] = ~diff
    rtol = 1e-6 if renorm else 1e-5
    np.testing.assert_allclose(g["probs"][rows][same], o["probs"][same], rtol=rtol, atol=1e-30)


def zipf_rows(seed, rows, V, sigma=3.0, zipf=1.1, dtype="f32"):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, sigma, (rows, V)).astype(np.float32)
    if zipf:
        z += (-zipf * np.log1p(np.arange(V))).astype(np.float32)
    if dtype == "bf16":
        return W.f32_to_bf16_bits(z)
    return z


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("k,top_p,T", [(50, 0.95, 1.0), (1, 0.9, 1.0), (64, 0.5, 0.7), (256, 1.0, 1.3), (7, 0.999, 2.0)])
def test_small_rows(dtype, renorm, k, top_p, T):
    z = zipf_rows(1, 9, 3001, dtype=dtype)
    g = run_support(z, dtype, k, top_p, T, renorm)
    o = oracle.build_support(z, dtype, k, top_p, T, renorm=renorm)
    check(g, o, renorm)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("pad", [1, 3, 8])
def test_strided_rows_with_ragged_heads(dtype, pad):
    z = zipf_rows(2, 6, 20011, dtype=dtype)
    g = run_support(z, dtype, 50, 0.95, 1.0, True, ld_pad=pad)
    o = oracle.build_support(z, dtype, 50, 0.95, 1.0)
    check(g, o, True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("renorm", [True, False])
def test_segmented_rows_merge(dtype, renorm):
    # few long rows: the launch cuts each row into segments whose candidates are merged by the last to finish
    z = zipf_rows(3, 5, 151936, dtype=dtype)
    g = run_support(z, dtype, 50, 0.95, 1.0, renorm)
    o = oracle.build_support(z, dtype, 50, 0.95, 1.0, renorm=renorm)
    check(g, o, renorm)


@pytest.mark.parametrize("k", [1, 50, 256])
def test_ties_and_degenerate_rows(k):
    V = 70001
    rng = np.random.default_rng(4)
    z = np.empty((8, V), np.float32)
    z[0] = np.round(rng.normal(0, 1.5, V))                 # heavy ties: few distinct values
    z[1] = 0.0                                              # every logit equal
    z[2] = -np.inf
    z[2, [5, 70000, 333]] = [1.0, 1.0, -2.0]               # fewer finite logits than k (k > 3)
    z[3] = np.linspace(-5, 5, V)                            # ascending: every element beats the threshold
    z[4] = np.linspace(5, -5, V)                            # descending
    z[5] = rng.normal(0, 3, V)
    z[5, 123] = np.nan                                      # data faults
    z[6] = rng.normal(0, 3, V)
    z[6, 4000] = np.inf
    z[7] = -np.inf
    for dtype in ("f32", "bf16"):
        zz = W.f32_to_bf16_bits(z) if dtype == "bf16" else z
        for renorm in (True, False):
            g = run_support(zz, dtype, k, 0.9, 1.0, renorm)
            o = oracle.build_support(zz, dtype, k, 0.9, 1.0, renorm=renorm)
            check(g, o, renorm)


def test_tiny_vocabularies():
    for V in (1, 2, 5, 37, 64, 65, 257):
        z = zipf_rows(5, 3, V, zipf=0.0)
        for k in sorted({1, min(V, 3), min(V, 256)}):
            g = run_support(z, "f32", k, 0.8, 1.0, True)
            o = oracle.build_support(z, "f32", k, 0.8, 1.0)
            check(g, o, True)


def test_headline_shaped_rows_sampled():
    """The target and draft logits of the dense block workload (B=64, gamma=16, V=151936, bf16) in the launch
    configuration the benchmark times; the oracle checks 48 sampled rows of each, every row is checked for
    properties that hold at any size."""
    case = W.make("dense_block_B64_g16_V151936_bf16")
    rng = np.random.default_rng(6)
    for name in ("target", "draft"):
        z = case[name].reshape(-1, case["V"])
        g = run_support(z, "bf16", 50, 0.95, 1.0, True)
        rows = np.sort(rng.choice(z.shape[0], 48, replace=False))
        o = oracle.build_support(z[rows], "bf16", 50, 0.95, 1.0)
        check(g, o, True, rows)
        assert (g["flags"] == 0).all()
        assert ((g["count"] >= 1) & (g["count"] <= 50)).all()
        kept = np.arange(50)[None, :] < g["count"][:, None]
        np.testing.assert_allclose(np.where(kept, g["probs"], 0).sum(1), 1.0, rtol=1e-5)
        vals = W.bf16_bits_to_f32(z)
        top = np.take_along_axis(vals, g["ids"].astype(np.int64), 1)
        assert (np.diff(top, axis=1) <= 0).all()             # descending
        V = vals.shape[1]
        ref = -np.sort(-np.partition(vals, V - 50, axis=1)[:, V - 50:], axis=1)
        np.testing.assert_array_equal(top, ref)             # the k largest values


def test_workspace_shared_with_the_verifier():
    from lossless_draft_verification_spec_amd import sv
    case = W.make("dense_tiny_B1_g4_V1024")
    z = zipf_rows(7, 40, 151936, dtype="bf16")
    n = max(sv.sv_support_workspace_bytes(40, 151936, 64), sv.sv_workspace_bytes(sv.SV_KIND_DENSE, 1, 4, 1024))
    ws = sv._zeroed_workspace(n, dev())
    o = oracle.build_support(z, "bf16", 64, 0.95, 1.0)
    from gpu_helpers import oracle_dense, run_dense, compare_decisions
    for _ in range(2):
        g = run_support(z, "bf16", 64, 0.95, 1.0, True, ws=ws)
        check(g, o, True)
        gd = run_dense(case, ws=ws)
        od = oracle_dense(case)
        compare_decisions(gd, od, "dense tiny")
    g = run_support(z[:7], "bf16", 64, 0.95, 1.0, True, ws=ws)     # another shape through the same workspace
    check(g, oracle.build_support(z[:7], "bf16", 64, 0.95, 1.0), True)
