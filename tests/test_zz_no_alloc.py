"""The no-allocation entry point (sv_verify_dense_noalloc, the library's static per-GPU scratch) against the
workspace entry point sv_verify_dense on the same inputs, two calls in a row, the second with a smaller input:
identical kernels on identical inputs, so every output must match bit for bit. Also: a shape whose plan exceeds the
scratch is refused on the host with SV_ERR_SCRATCH, before any HIP call."""
import ctypes

import numpy as np
import pytest
import torch

from lossless_draft_verification_spec_amd import workloads as W

from gpu_helpers import compare_decisions, oracle_dense, t_, t_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(case):
    from lossless_draft_verification_spec_amd import sv
    tgt = t_logits(case["target"], case["dtype"])
    dft = t_logits(case["draft"], case["dtype"])
    ids = t_(case["draft_ids"], torch.int32)
    ua = t_(case["u_accept"], torch.float32)
    us = t_(case["u_sample"], torch.float32)
    st_a = torch.ones(case["B"], dtype=torch.int32, device="cuda")
    st_b = st_a.clone()
    a = sv.sv_verify_dense(tgt, dft, ids, ua, us, case["temperature"], bonus=case["bonus"], start=st_a)
    b = sv.sv_verify_dense_noalloc(tgt, dft, ids, ua, us, case["temperature"], bonus=case["bonus"], start=st_b)
    torch.cuda.synchronize()
    ha = {k: v.cpu().numpy() for k, v in a.items()}
    hb = {k: v.cpu().numpy() for k, v in b.items()}
    ha["start_out"], hb["start_out"] = st_a.cpu().numpy(), st_b.cpu().numpy()
    return ha, hb


def test_noalloc_matches_workspace_entry_point_two_calls():
    cases = [W.dense_case(8, 6, 50_000, dtype="bf16", sigma_t=3.0, sigma_d=1.0, zipf=1.1, seed=61),
             W.dense_case(3, 4, 20_011, dtype="f32", sigma_t=2.0, sigma_d=0.5, seed=62)]       # smaller, second
    for i, case in enumerate(cases):
        print(f"no-alloc call {i}: B={case['B']} gamma={case['gamma']} V={case['V']} {case['dtype']}", flush=True)
        ha, hb = _both(case)
        for k in ha:
            assert np.array_equal(ha[k], hb[k], equal_nan=True), (i, k)
        # and both meet the oracle (start = 1 for every sequence)
        o = oracle_dense(case, start=np.ones(case["B"], np.int32))
        print(f"  {compare_decisions(hb, o, f'no-alloc call {i}')}", flush=True)


def test_noalloc_refuses_shapes_beyond_the_scratch():
    from lossless_draft_verification_spec_amd import sv
    B, G, V = 1024, 16, 151936
    assert sv.sv_workspace_bytes(sv.SV_KIND_DENSE, B, G, V) > sv.SV_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)      # never dereferenced: the size check returns before any HIP call
    st = sv.LIB.sv_verify_dense_noalloc(fake, G * V + V, V, fake, G * V, V, sv.SV_BF16, B, G, V, fake, fake, fake,
                                        1.0, 1, None, None, None, fake, fake, None, None, None, None)
    assert st == sv.SV_ERR_SCRATCH
