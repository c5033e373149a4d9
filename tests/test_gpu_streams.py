"""Stream ordering and independence of calls: every entry point enqueues its work on the stream it is given and keeps
no state outside its arguments and workspace, so the same calls on two side streams, launched one after the other
with nothing synchronised in between and a workspace each, give exactly the results of the default stream."""
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


def _inputs(d):
    case = W.dense_case(4, 5, 20_011, dtype="bf16", sigma_t=3.0, sigma_d=1.0, zipf=1.1, seed=61)
    sc = W.sparse_case(4, 5, 64, 20_011, seed=62)
    tc = W.tree_case(4, 9, 20_011, dtype="bf16", seed=63)
    bf = lambda x: torch.from_numpy(x).view(torch.bfloat16).to(d)
    dev = lambda x: torch.from_numpy(x).to(d)
    return dict(T=case["temperature"], V=case["V"], tgt=bf(case["target"]), dft=bf(case["draft"]),
                ids=dev(case["draft_ids"]), ua=dev(case["u_accept"]), us=dev(case["u_sample"]),
                sparse=[dev(sc[k]) for k in ("p_ids", "p_probs", "q_ids", "q_probs", "spec_ids", "u_accept",
                                             "u_sample")], sV=sc["V"],
                t_tgt=bf(tc["target"]), t_par=dev(tc["parent"]), t_tok=dev(tc["token"]), t_ua=dev(tc["u_accept"]),
                t_us=dev(tc["u_sample"]), t_T=tc["temperature"])


def _all_calls(x, stream):
    """Every entry point once on `stream` (None: the current stream); outputs and workspaces allocated for it."""
    from lossless_draft_verification_spec_amd import sv
    V, T = x["V"], x["T"]
    out = {}
    out["dense"] = sv.sv_verify_dense(x["tgt"], x["dft"], x["ids"], x["ua"], x["us"], T, bonus=1, stream=stream)
    out["onehot"] = sv.sv_verify_onehot_draft(x["tgt"], x["ids"], x["ua"], x["us"], T, bonus=1, stream=stream)
    out["sparse"] = sv.sv_verify_sparse(*x["sparse"], bonus=1, vocab_size=x["sV"], stream=stream)
    pa, pb = sv.sv_build_support_pair(x["tgt"].view(-1, V), x["dft"].view(-1, V), 50, 0.95, T, True, stream=stream)
    out["support_a"], out["support_b"] = pa, pb
    out["greedy"] = sv.sv_verify_greedy(x["tgt"], x["ids"], bonus=1, stream=stream)
    out["commit"] = sv.sv_confidence_commit(x["tgt"], 0.2, stream=stream)
    out["tree"] = sv.sv_verify_tree(x["t_tgt"], x["t_par"], x["t_tok"], x["t_ua"], x["t_us"], x["t_T"], stream=stream)
    return out


def _host(out):
    return {call: {k: v.cpu().numpy() for k, v in res.items()} for call, res in out.items()}


def test_side_streams_match_the_default_stream():
    d = torch.device("cuda", 0)
    x = _inputs(d)
    ref = _host(_all_calls(x, None))
    torch.cuda.synchronize()
    side = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for s in side:
        s.wait_stream(torch.cuda.current_stream())            # the inputs were written on the default stream
        with torch.cuda.stream(s):
            outs.append(_all_calls(x, s))
    torch.cuda.synchronize()
    for i, out in enumerate(outs):
        got = _host(out)
        for call, res in ref.items():
            for k, want in res.items():
                g = got[call][k]
                if np.issubdtype(want.dtype, np.floating):
                    np.testing.assert_allclose(g, want, rtol=1e-6, atol=1e-30, equal_nan=True,
                                               err_msg=f"stream {i}: {call}.{k}")
                else:
                    assert np.array_equal(g, want), (i, call, k, g, want)
    print("side streams: every entry point matches the default stream", flush=True)
