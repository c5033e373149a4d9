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


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [50, 256])
def test_long_rows_many_segments(dtype, k):
    """Three rows of V = 1,000,003: each row is cut into the most segments the merge area allows (16 at k = 50, 12
    at k = 256), the vocabulary's odd length leaves a ragged tail on the last segment, and the merge ranks up to
    12 x 256 keys."""
    z = zipf_rows(7 + k, 3, 1_000_003, dtype=dtype)
    for renorm in (True, False):
        g = run_support(z, dtype, k, 0.95, 1.0, renorm)
        o = oracle.build_support(z, dtype, k, 0.95, 1.0, renorm=renorm)
        check(g, o, renorm)


def test_faults_inside_later_segments():
    """Rows of 600,001 logits cut into segments: a NaN in the last segment and a +inf in a middle one are reported
    for their rows once the segments are merged; a row -inf past its first 1000 elements keeps its head's support."""
    z = zipf_rows(11, 4, 600_001)
    z[0, 600_001 - 3] = np.nan
    z[1, 300_000] = np.inf
    z[2, 1000:] = -np.inf
    for dtype in ("f32", "bf16"):
        zz = W.f32_to_bf16_bits(z) if dtype == "bf16" else z
        for renorm in (True, False):
            g = run_support(zz, dtype, 50, 0.95, 1.0, renorm)
            o = oracle.build_support(zz, dtype, 50, 0.95, 1.0, renorm=renorm)
            check(g, o, renorm)
            assert (g["flags"][:2] == o["flags"][:2]).all() and (o["flags"][:2] != 0).all()
            assert g["flags"][2] == 0 and g["flags"][3] == 0


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


# ----------------------------------------------------------------------------------------------------------------
# two row sets in one launch
# ----------------------------------------------------------------------------------------------------------------

def dev_rows(z, dtype, ld_pad=0):
    if not ld_pad:
        return t_logits(z, dtype)
    big = np.zeros((z.shape[0], z.shape[1] + ld_pad), dtype=z.dtype)
    big[:, :z.shape[1]] = z
    return t_logits(big, dtype)[:, :z.shape[1]]


def run_pair(za, zb, dtype, k, top_p, T, renorm, *, ld_pad_b=0, ws=None):
    from lossless_draft_verification_spec_amd import sv
    xa, xb = dev_rows(za, dtype), dev_rows(zb, dtype, ld_pad_b)
    oa, ob = sv.sv_build_support_pair(xa, xb, k, top_p, T, renorm, ws=ws)
    torch.cuda.synchronize()
    return ({n: v.cpu().numpy() for n, v in oa.items()}, {n: v.cpu().numpy() for n, v in ob.items()})


def assert_same(g, h):
    """Bit-for-bit equality of two support outputs (NaN payloads included)."""
    for n in ("ids", "count", "flags"):
        np.testing.assert_array_equal(g[n], h[n])
    np.testing.assert_array_equal(g["probs"].view(np.uint32), h["probs"].view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("renorm", [True, False])
def test_pair_small_against_oracle_and_single_calls(dtype, renorm):
    za = zipf_rows(11, 9, 3001, dtype=dtype)
    zb = zipf_rows(12, 5, 3001, sigma=1.0, dtype=dtype)
    ga, gb = run_pair(za, zb, dtype, 50, 0.95, 1.0, renorm, ld_pad_b=37)
    check(ga, oracle.build_support(za, dtype, 50, 0.95, 1.0, renorm=renorm), renorm)
    check(gb, oracle.build_support(zb, dtype, 50, 0.95, 1.0, renorm=renorm), renorm)
    assert_same(ga, run_support(za, dtype, 50, 0.95, 1.0, renorm))
    assert_same(gb, run_support(zb, dtype, 50, 0.95, 1.0, renorm, ld_pad=37))


@pytest.mark.parametrize("rows_a,rows_b", [(1026, 4), (700, 330), (1, 1029), (1029, 1), (2000, 113)])
def test_pair_rows_past_a_resident_round(rows_a, rows_b):
    """Sizes whose rows past the last full resident round (1024 workgroups on MI355X) are cut into segments, with
    that tail inside the first set, inside the second, or across the two; faulted rows in both sets. Every row
    matches the single-set calls bit for bit, and sampled rows of each set (the tail's among them) the oracle."""
    V = 20000
    za = zipf_rows(21, rows_a, V, dtype="bf16")
    zb = zipf_rows(22, rows_b, V, sigma=2.0, dtype="bf16")
    za[0, 5] = 0x7FC0                                        # NaN
    zb[-1, :] = 0xFF80                                       # a row all -inf
    ga, gb = run_pair(za, zb, "bf16", 50, 0.95, 1.0, True)
    assert_same(ga, run_support(za, "bf16", 50, 0.95, 1.0, True))
    assert_same(gb, run_support(zb, "bf16", 50, 0.95, 1.0, True))
    rng = np.random.default_rng(rows_a * 7 + rows_b)
    total = rows_a + rows_b
    tail = np.arange(total - total % 1024, total)
    for g, z, lo, n in ((ga, za, 0, rows_a), (gb, zb, rows_a, rows_b)):
        mine = tail[(tail >= lo) & (tail < lo + n)] - lo
        pick = np.unique(np.concatenate([rng.choice(n, min(n, 12), replace=False), mine[:6], mine[-6:], [0, n - 1]]))
        check(g, oracle.build_support(z[pick], "bf16", 50, 0.95, 1.0), True, pick)
    assert ga["flags"][0] != 0 and gb["flags"][-1] != 0


def test_pair_of_one_set_twice():
    """Both sets on the same logits: the two outputs are the one set's support."""
    from lossless_draft_verification_spec_amd import sv
    z = zipf_rows(31, 70, 151936, dtype="bf16")
    x = t_logits(z, "bf16")
    oa, ob = sv.sv_build_support_pair(x, x, 64, 0.9, 0.8, False)
    torch.cuda.synchronize()
    ga = {n: v.cpu().numpy() for n, v in oa.items()}
    gb = {n: v.cpu().numpy() for n, v in ob.items()}
    assert_same(ga, gb)
    check(ga, oracle.build_support(z, "bf16", 64, 0.9, 0.8, renorm=False), False)


def test_pair_headline_shaped_rows_sampled():
    """The target rows (B x (gamma + 1) = 1088) and the draft rows (B x gamma = 1024) of the dense block workload
    (V = 151936, bf16) in one launch, as the benchmark's chain runs them: every row bit for bit against the single-set
    calls, 48 sampled rows of each set (the 64 rows past the second resident round among them) against the oracle."""
    case = W.make("dense_block_B64_g16_V151936_bf16")
    V = case["V"]
    zt, zd = case["target"].reshape(-1, V), case["draft"].reshape(-1, V)
    gt, gd = run_pair(zt, zd, "bf16", 50, 0.95, 1.0, True)
    assert_same(gt, run_support(zt, "bf16", 50, 0.95, 1.0, True))
    assert_same(gd, run_support(zd, "bf16", 50, 0.95, 1.0, True))
    rng = np.random.default_rng(9)
    rows_d = zd.shape[0]
    tail_d = np.arange(rows_d - 64, rows_d)                  # global rows 2048 .. 2111: the draft set's last 64
    for g, z, extra in ((gt, zt, np.array([], dtype=np.int64)), (gd, zd, tail_d)):
        rows = np.unique(np.concatenate([rng.choice(z.shape[0], 40, replace=False), extra[::8]]))
        check(g, oracle.build_support(z[rows], "bf16", 50, 0.95, 1.0), True, rows)
        assert (g["flags"] == 0).all()


def test_pair_and_single_calls_share_a_workspace():
    from lossless_draft_verification_spec_amd import sv
    V = 151936
    za, zb = zipf_rows(41, 30, V, dtype="bf16"), zipf_rows(42, 12, V, dtype="bf16")
    ws = sv._zeroed_workspace(sv.sv_support_workspace_bytes(42, V, 64), dev())
    oa = oracle.build_support(za, "bf16", 64, 0.95, 1.0)
    ob = oracle.build_support(zb, "bf16", 64, 0.95, 1.0)
    for _ in range(2):
        ga, gb = run_pair(za, zb, "bf16", 64, 0.95, 1.0, True, ws=ws)
        check(ga, oa, True)
        check(gb, ob, True)
        check(run_support(za, "bf16", 64, 0.95, 1.0, True, ws=ws), oa, True)
        ga, gb = run_pair(zb, za[:5], "bf16", 64, 0.95, 1.0, True, ws=ws)   # fewer rows through the same workspace
        check(ga, ob, True)
        check(gb, oracle.build_support(za[:5], "bf16", 64, 0.95, 1.0), True)
