"""The C-ABI library loads, exports every declared symbol, sizes workspaces and rejects bad arguments on the host
before any HIP call (no GPU needed: no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sv.h")
LIB = os.path.join(ROOT, "lossless_draft_verification_spec_amd", "libsv.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsv.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


def test_exports_match_header():
    names = declared_functions()
    assert set(names) == {"sv_workspace_bytes", "sv_status_string", "sv_verify_dense", "sv_verify_dense_noalloc",
                          "sv_verify_onehot_draft", "sv_verify_sparse", "sv_support_workspace_bytes",
                          "sv_build_support", "sv_build_support_pair", "sv_verify_greedy", "sv_confidence_commit",
                          "sv_verify_tree"}
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sv_[a-z_]+)\b", out))
    assert set(names) <= exported
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n)


def test_header_constants_match_binding():
    from lossless_draft_verification_spec_amd import sv
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(SV_[A-Z_0-9]+)\s+\(?(-?\d+)u?\)?", text))
    assert int(consts["SV_OK"]) == sv.SV_OK
    assert int(consts["SV_F32"]) == sv.SV_F32 and int(consts["SV_BF16"]) == sv.SV_BF16
    assert int(consts["SV_KIND_DENSE"]) == sv.SV_KIND_DENSE and int(consts["SV_KIND_SPARSE"]) == sv.SV_KIND_SPARSE
    assert int(consts["SV_KIND_GREEDY"]) == sv.SV_KIND_GREEDY
    assert int(consts["SV_FLAG_NONFINITE"]) == sv.SV_FLAG_NONFINITE
    assert int(consts["SV_FLAG_Q_ZERO"]) == sv.SV_FLAG_Q_ZERO
    assert int(consts["SV_FLAG_INTERNAL"]) == sv.SV_FLAG_INTERNAL
    assert int(consts["SV_MAX_GAMMA"]) == sv.SV_MAX_GAMMA and int(consts["SV_MAX_K"]) == sv.SV_MAX_K


def test_workspace_sizes():
    from lossless_draft_verification_spec_amd import sv
    bad = (1 << 64) - 1
    for kind in (sv.SV_KIND_DENSE, sv.SV_KIND_ONEHOT):
        for (B, G, V) in [(1, 4, 1024), (64, 16, 151936), (256, 8, 128256), (32, 32, 262144), (3, 1, 7)]:
            n = sv.sv_workspace_bytes(kind, B, G, V)
            assert 0 < n < 64 << 20 and n % 256 == 0
        assert sv.sv_workspace_bytes(kind, 0, 4, 100) == bad
        assert sv.sv_workspace_bytes(kind, 1, 0, 100) == bad
        assert sv.sv_workspace_bytes(kind, 1, sv.SV_MAX_GAMMA + 1, 100) == bad
        assert sv.sv_workspace_bytes(kind, 1, 4, 0) == bad
    assert sv.sv_workspace_bytes(sv.SV_KIND_SPARSE, 1024, 16, 64) == 0
    assert sv.sv_workspace_bytes(sv.SV_KIND_SPARSE, 1024, 16, sv.SV_MAX_K + 1) == bad
    assert sv.sv_workspace_bytes(7, 1, 1, 1) == bad
    assert sv.sv_status_string(0) == "ok" and "NULL" in sv.sv_status_string(-1)


# Fake, suitably aligned addresses: every call below fails validation, so none of them is ever dereferenced.
A = 1 << 20


def dense_args(**kw):
    args = dict(tgt=A, t_seq=5 * 128, t_row=128, dft=A, d_seq=4 * 128, d_row=128, dtype=0, B=2, G=4, V=128, ids=A,
                ua=A, us=A, T=1.0, bonus=1, start=None, order=None, accept=A, n=A, tok=A, pd=A, qd=A, flags=A, ws=A,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return args


def call_dense(a):
    from lossless_draft_verification_spec_amd import sv
    return sv.LIB.sv_verify_dense(a["tgt"], a["t_seq"], a["t_row"], a["dft"], a["d_seq"], a["d_row"], a["dtype"],
                                  a["B"], a["G"], a["V"], a["ids"], a["ua"], a["us"], a["T"], a["bonus"], a["start"],
                                  a["order"], a["accept"], a["n"], a["tok"], a["pd"], a["qd"], a["flags"], a["ws"],
                                  a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(tgt=None), -1), (dict(dft=None), -1), (dict(ids=None), -1), (dict(ua=None), -1), (dict(us=None), -1),
    (dict(n=None), -1), (dict(tok=None), -1),
    (dict(dtype=5), -3),
    (dict(B=0), -2), (dict(G=0), -2), (dict(G=1025), -2), (dict(V=0), -2), (dict(V=1 << 31), -2),
    (dict(t_row=0), -2), (dict(d_seq=0), -2),
    (dict(T=0.0), -4), (dict(T=-1.0), -4), (dict(T=float("nan")), -4), (dict(T=float("inf")), -4),
    (dict(bonus=2), -8),
    (dict(tgt=A + 2), -5), (dict(dft=A + 1, dtype=1), -5), (dict(ids=A + 2), -5), (dict(ws=A + 16), -5),
    (dict(ws=None), -6), (dict(ws_bytes=16), -6),
])
def test_dense_rejects_bad_arguments(kw, code):
    assert call_dense(dense_args(**kw)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(tgt=None), -1), (dict(B=-1), -2), (dict(T=0.0), -4), (dict(dtype=2), -3), (dict(ws_bytes=1), -6),
    (dict(tgt=A + 1, dtype=1), -5),
])
def test_onehot_rejects_bad_arguments(kw, code):
    from lossless_draft_verification_spec_amd import sv
    a = dense_args(**kw)
    st = sv.LIB.sv_verify_onehot_draft(a["tgt"], a["t_seq"], a["t_row"], a["dtype"], a["B"], a["G"], a["V"], a["ids"],
                                       a["ua"], a["us"], a["T"], a["bonus"], a["start"], a["order"], a["accept"],
                                       a["n"], a["tok"], a["pd"], a["flags"], a["ws"], a["ws_bytes"], a["stream"])
    assert st == code


@pytest.mark.parametrize("kw,code", [
    (dict(pi=None), -1), (dict(qp=None), -1), (dict(spec=None), -1), (dict(n=None), -1),
    (dict(B=0), -2), (dict(G=0), -2), (dict(kp=0), -2), (dict(kp=257), -2), (dict(kq=300), -2), (dict(vocab=-1), -2),
    (dict(bonus=-1), -8), (dict(pp=A + 2), -5), (dict(corr=A + 1), -5),
])
def test_sparse_rejects_bad_arguments(kw, code):
    from lossless_draft_verification_spec_amd import sv
    a = dict(pi=A, pp=A, qi=A, qp=A, B=4, G=3, kp=8, kq=8, vocab=0, spec=A, ua=A, us=A, bonus=1, accept=A, n=A,
             tok=A, corr=A, ps=A, qs=A, flags=A)
    a.update(kw)
    st = sv.LIB.sv_verify_sparse(a["pi"], a["pp"], a["qi"], a["qp"], a["B"], a["G"], a["kp"], a["kq"], a["vocab"],
                                 a["spec"], a["ua"], a["us"], a["bonus"], a["accept"], a["n"], a["tok"], a["corr"],
                                 a["ps"], a["qs"], a["flags"], None, 0, None)
    assert st == code


def test_support_workspace_sizes():
    from lossless_draft_verification_spec_amd import sv
    bad = (1 << 64) - 1
    for (rows, V, k) in [(1, 1024, 50), (1088, 151936, 50), (17408, 151936, 64), (5, 37, 37), (2, 300000, 256)]:
        n = sv.sv_support_workspace_bytes(rows, V, k)
        assert 0 < n < 256 << 20 and n % 256 == 0
        assert n >= rows * 256                     # one counter line per row
    assert sv.sv_support_workspace_bytes(0, 100, 5) == bad
    assert sv.sv_support_workspace_bytes(4, 0, 1) == bad
    assert sv.sv_support_workspace_bytes(4, 100, 0) == bad
    assert sv.sv_support_workspace_bytes(4, 100, 101) == bad           # k > V
    assert sv.sv_support_workspace_bytes(4, 1000, sv.SV_MAX_K + 1) == bad


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), -1), (dict(ids=None), -1), (dict(probs=None), -1),
    (dict(dtype=3), -3),
    (dict(rows=0), -2), (dict(V=0), -2), (dict(k=0), -2), (dict(k=257, V=1000), -2), (dict(k=129), -2),
    (dict(ld=127), -2), (dict(V=1 << 31, ld=1 << 31), -2),
    (dict(T=0.0), -4), (dict(T=float("nan")), -4),
    (dict(top_p=0.0), -8), (dict(top_p=1.5), -8), (dict(top_p=float("nan")), -8), (dict(renorm=2), -8),
    (dict(logits=A + 2), -5), (dict(logits=A + 1, dtype=1), -5), (dict(ids=A + 2), -5), (dict(count=A + 1), -5),
    (dict(ws=A + 16), -5), (dict(ws=None), -6), (dict(ws_bytes=16), -6),
])
def test_support_rejects_bad_arguments(kw, code):
    from lossless_draft_verification_spec_amd import sv
    a = dict(logits=A, ld=128, dtype=0, rows=3, V=128, T=1.0, k=8, top_p=0.9, renorm=1, ids=A, probs=A, count=A,
             flags=A, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    st = sv.LIB.sv_build_support(a["logits"], a["ld"], a["dtype"], a["rows"], a["V"], a["T"], a["k"], a["top_p"],
                                 a["renorm"], a["ids"], a["probs"], a["count"], a["flags"], a["ws"], a["ws_bytes"],
                                 None)
    assert st == code


@pytest.mark.parametrize("kw,code", [
    (dict(la=None), -1), (dict(lb=None), -1), (dict(ids_a=None), -1), (dict(probs_b=None), -1),
    (dict(dtype=3), -3),
    (dict(rows_a=0), -2), (dict(rows_b=0), -2), (dict(rows_a=1 << 30, rows_b=1 << 30, V=1, ld_a=1, ld_b=1, k=1), -2),
    (dict(ld_b=127), -2), (dict(V=0), -2), (dict(k=129), -2),
    (dict(T=0.0), -4), (dict(top_p=0.0), -8), (dict(renorm=2), -8),
    (dict(lb=A + 2), -5), (dict(flags_b=A + 1), -5), (dict(count_a=A + 3), -5),
    (dict(ws=A + 16), -5), (dict(ws=None), -6), (dict(ws_bytes=16), -6),
])
def test_support_pair_rejects_bad_arguments(kw, code):
    from lossless_draft_verification_spec_amd import sv
    a = dict(la=A, ld_a=128, rows_a=3, lb=A, ld_b=128, rows_b=2, dtype=0, V=128, T=1.0, k=8, top_p=0.9, renorm=1,
             ids_a=A, probs_a=A, count_a=A, flags_a=A, ids_b=A, probs_b=A, count_b=A, flags_b=A, ws=A,
             ws_bytes=1 << 30)
    a.update(kw)
    st = sv.LIB.sv_build_support_pair(a["la"], a["ld_a"], a["rows_a"], a["lb"], a["ld_b"], a["rows_b"], a["dtype"],
                                      a["V"], a["T"], a["k"], a["top_p"], a["renorm"], a["ids_a"], a["probs_a"],
                                      a["count_a"], a["flags_a"], a["ids_b"], a["probs_b"], a["count_b"],
                                      a["flags_b"], a["ws"], a["ws_bytes"], None)
    assert st == code


def test_support_pair_workspace_is_that_of_the_rows_together():
    from lossless_draft_verification_spec_amd import sv
    need = sv.sv_support_workspace_bytes(5, 128, 8)
    # one byte short of the two sets' rows together is refused before any launch
    st = sv.LIB.sv_build_support_pair(A, 128, 3, A, 128, 2, 0, 128, 1.0, 8, 0.9, 1, A, A, A, A, A, A, A, A, A,
                                      need - 1, None)
    assert st == -6


def test_binding_marshalling_checks_without_gpu():
    import torch
    from lossless_draft_verification_spec_amd import sv
    t = torch.zeros(2, 5, 16)
    d = torch.zeros(2, 4, 16)
    ids = torch.zeros(2, 4, dtype=torch.int64)
    u = torch.zeros(2, 4)
    us = torch.zeros(2, 5)
    with pytest.raises(TypeError):
        sv.sv_verify_dense(t, d, ids, u, us, 1.0)          # int64 ids rejected before any call
    with pytest.raises(ValueError):
        sv.sv_verify_dense(t[:, :3], d, ids.int(), u, us, 1.0)   # too few target rows


def test_greedy_workspace_sizes():
    from lossless_draft_verification_spec_amd import sv
    bad = (1 << 64) - 1
    for (B, G, V) in [(1, 4, 1024), (64, 16, 151936), (256, 8, 128256), (3, 1, 7), (2, 1024, 1 << 30)]:
        n = sv.sv_workspace_bytes(sv.SV_KIND_GREEDY, B, G, V)
        assert 0 < n < 1 << 30 and n % 8 == 0
        assert n >= B * (G + 1) * 8 + B * 4             # a counter per sequence, a key per row and segment
        assert n <= 256 + B * (G + 1) * 64 * 8 + B * 4 + 4096 * 64 * 8
    assert sv.sv_workspace_bytes(sv.SV_KIND_GREEDY, 0, 4, 100) == bad
    assert sv.sv_workspace_bytes(sv.SV_KIND_GREEDY, 4, 1025, 100) == bad
    assert sv.sv_workspace_bytes(sv.SV_KIND_GREEDY, 4, 4, 1 << 31) == bad


@pytest.mark.parametrize("kw,code", [
    (dict(tgt=None), -1), (dict(ids=None), -1), (dict(n=None), -1), (dict(tok=None), -1),
    (dict(dtype=2), -3),
    (dict(B=0), -2), (dict(G=0), -2), (dict(G=1025), -2), (dict(V=0), -2), (dict(V=1 << 31), -2),
    (dict(t_seq=0), -2), (dict(t_row=0), -2),
    (dict(bonus=2), -8),
    (dict(tgt=A + 2), -5), (dict(tgt=A + 1, dtype=1), -5), (dict(ids=A + 2), -5), (dict(start=A + 1), -5),
    (dict(order=A + 3), -5), (dict(flags=A + 2), -5), (dict(ws=A + 16), -5),
    (dict(ws=None), -6), (dict(ws_bytes=16), -6),
])
def test_greedy_rejects_bad_arguments(kw, code):
    from lossless_draft_verification_spec_amd import sv
    a = dict(tgt=A, t_seq=5 * 64, t_row=64, dtype=0, B=4, G=4, V=64, ids=A, bonus=1, start=A, order=A, accept=A,
             n=A, tok=A, flags=A, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    st = sv.LIB.sv_verify_greedy(a["tgt"], a["t_seq"], a["t_row"], a["dtype"], a["B"], a["G"], a["V"], a["ids"],
                                 a["bonus"], a["start"], a["order"], a["accept"], a["n"], a["tok"], a["flags"],
                                 a["ws"], a["ws_bytes"], None)
    assert st == code


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), -1), (dict(tok=None), -1), (dict(n=None), -1), (dict(dtype=7), -3),
    (dict(B=0), -2), (dict(W=0), -2), (dict(W=1025), -2), (dict(V=0), -2), (dict(l_row=0), -2),
    (dict(tau=-0.1), -8), (dict(tau=1.5), -8), (dict(tau=float("nan")), -8),
    (dict(logits=A + 1, dtype=1), -5), (dict(tok=A + 2), -5), (dict(conf=A + 1), -5), (dict(ws=A + 8), -5),
    (dict(ws=None), -6), (dict(ws_bytes=8), -6),
])
def test_commit_rejects_bad_arguments(kw, code):
    from lossless_draft_verification_spec_amd import sv
    a = dict(logits=A, l_seq=4 * 64, l_row=64, dtype=0, B=3, W=4, V=64, masked=A, tau=0.9, commit=A, tok=A, conf=A,
             n=A, flags=A, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    st = sv.LIB.sv_confidence_commit(a["logits"], a["l_seq"], a["l_row"], a["dtype"], a["B"], a["W"], a["V"],
                                     a["masked"], a["tau"], a["commit"], a["tok"], a["conf"], a["n"], a["flags"],
                                     a["ws"], a["ws_bytes"], None)
    assert st == code
