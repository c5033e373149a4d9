"""Calls captured in a HIP graph, the no-allocation dense variant among them: the library records kernel launches only
(no allocation, no memset, no host synchronisation), so a captured call replays correctly. Workspaces and outputs
are allocated before the capture; every replay is checked against the eager result, with the program's own eager
work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

from lossless_draft_verification_spec_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_draft_verification_spec_amd import sv  # noqa: F401  (raises if the library is missing)


def test_calls_replayed_from_a_captured_graph():
    from lossless_draft_verification_spec_amd import sv
    d = torch.device("cuda", 0)
    case = W.dense_case(8, 6, 30_011, dtype="bf16", sigma_t=3.0, sigma_d=1.0, zipf=1.1, seed=81)
    sc = W.sparse_case(8, 6, 64, 30_011, seed=82)
    tc = W.tree_case(4, 9, 30_011, dtype="bf16", seed=83)
    bf = lambda x: torch.from_numpy(x).view(torch.bfloat16).to(d)
    dev = lambda x: torch.from_numpy(x).to(d)
    B, G, V, T = case["B"], case["gamma"], case["V"], case["temperature"]
    tgt, dft, ids, ua, us = bf(case["target"]), bf(case["draft"]), dev(case["draft_ids"]), dev(case["u_accept"]), \
        dev(case["u_sample"])
    sp = [dev(sc[k]) for k in ("p_ids", "p_probs", "q_ids", "q_probs", "spec_ids", "u_accept", "u_sample")]
    tt, tp, tk, tua, tus = bf(tc["target"]), dev(tc["parent"]), dev(tc["token"]), dev(tc["u_accept"]), \
        dev(tc["u_sample"])
    ws_d = sv.workspace(sv.SV_KIND_DENSE, B, G, V, d)
    ws_s = sv.support_workspace(B * (G + 1) + B * G, V, 50, d)
    ws_t = sv.workspace(sv.SV_KIND_TREE, tc["B"], tc["N"], V, d)
    o_d, o_a, o_b, o_s, o_t, o_n = {}, {}, {}, {}, {}, {}

    def calls():
        sv.sv_verify_dense(tgt, dft, ids, ua, us, T, bonus=1, out=o_d, ws=ws_d)
        sv.sv_build_support_pair(tgt.view(-1, V), dft.view(-1, V), 50, 0.95, T, True, out_a=o_a, out_b=o_b, ws=ws_s)
        sv.sv_verify_sparse(*sp, bonus=1, vocab_size=sc["V"], out=o_s)
        sv.sv_verify_tree(tt, tp, tk, tua, tus, tc["temperature"], out=o_t, ws=ws_t)
        # the no-allocation variant on the library's static scratch (calls in one graph run in order: no overlap)
        sv.sv_verify_dense_noalloc(tgt, dft, ids, ua, us, T, bonus=1, out=o_n)

    outs = (o_d, o_a, o_b, o_s, o_t, o_n)
    calls()                                              # eager: allocates every output once
    torch.cuda.synchronize()
    want = [{k: v.cpu().numpy().copy() for k, v in o.items()} for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                                          # a warm-up on the capture's side of the allocator
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        for o in outs:                                   # eager work between the replays: scribble on the outputs
            for v in o.values():
                v.fill_(7) if v.dtype != torch.bool else v.fill_(True)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            for k, v in o.items():
                got = v.cpu().numpy()
                if np.issubdtype(got.dtype, np.floating):
                    np.testing.assert_allclose(got, w[k], rtol=1e-6, atol=1e-30, equal_nan=True,
                                               err_msg=f"replay {rep}: output set {i} {k}")
                else:
                    assert np.array_equal(got, w[k]), (rep, i, k)
    print("graph replays: 4 of 4 match the eager calls", flush=True)
