"""Benchmark of the speculative-sampling verifier on one MI355X.

One step = one full verification call (statistics, accept/first-reject scan, float64 draw: one kernel launch) over the
dense block workload: B=64 sequences, gamma=16 drafts, V=151936, bf16 target and draft logits (synthetic, seeded). The
headline value is verified draft positions per second. The roofline object reports the verifier kernel's achieved HBM
bandwidth: algorithmic bytes per launch (every verified logit of both tensors, 2*B*gamma*V*2, plus the row pair each
rejected sequence's draw reads again, or the target row of a bonus draw) over the average launch duration, taken
from HIP events on the launch stream around the K timed steps (each step is exactly one launch, so this average
includes the gap between back-to-back launches: it bounds the kernel's own duration from above).

The other workloads are timed after it, each in its own region of back-to-back launches of one kernel, and reported
under "workloads": the dense -> top-k/top-p support -> sparse verify chain on the headline's logits (each of its three
kernels alone, then the whole chain), tiny dense, greedy one-hot, sparse top-64, the masked-diffusion window (per
round, from events between the rounds of each chained step, and the whole 4-round chain), greedy verification at
T = 0, the confidence-threshold commit, and tree verification.

The CPU baseline is the float64 oracle as it stands, timed before the GPU is touched on bounded samples of the
headline workload: once in this process (one thread) and once over a pool of worker processes on the host cores this
process may run on (at most 16).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--cpu-seconds S] [--only NAME]
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
HEADLINE = "dense_block_B64_g16_V151936_bf16"
METRIC = "verified draft positions/sec + achieved HBM GB/s (% of peak), dense B x gamma x V"
CPU_POOL_MAX = 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev_logits(x, dtype, torch, d):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.view(torch.bfloat16) if dtype == "bf16" else t).to(d)


def time_region(fn, steps, warmup, torch):
    """Average ms per step over `steps` back-to-back calls of fn(i), from events on the current stream (the stream
    every call launches on), after `warmup` untimed calls. Also returns the host wall time per step."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, (time.perf_counter() - t0) * 1e3 / steps


def hbm(nbytes, ms):
    gbps = nbytes / (ms * 1e-3) / 1e9
    return gbps, gbps / HBM_PEAK_GBPS


def roofline(nbytes, ms, kernel, traffic=None):
    gbps, frac = hbm(nbytes, ms)
    return {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": frac,
            "traffic": traffic, "kernel": kernel, "kernel_ms": ms, "bytes_per_launch": nbytes}


# ----------------------------------------------------------------------------------------------------------------------
# dense / one-hot
# ----------------------------------------------------------------------------------------------------------------------

def bench_dense(case, steps, warmup, torch, sv, d, traffic=None):
    """Dense or one-hot workload: one launch of k_verify per step."""
    onehot = case["kind"] == "onehot"
    B, G, V = case["B"], case["gamma"], case["V"]
    s = 2 if case["dtype"] == "bf16" else 4
    verified_bytes = (1 if onehot else 2) * B * G * V * s
    ncopies = max(1, min(4, int(np.ceil(768e6 / verified_bytes))))       # defeat the 256 MB last-level cache
    tgts = [to_dev_logits(case["target"], case["dtype"], torch, d) for _ in range(ncopies)]
    dfts = [None if onehot else to_dev_logits(case["draft"], case["dtype"], torch, d) for _ in range(ncopies)]
    ids = torch.from_numpy(case["draft_ids"]).to(d)
    ua = torch.from_numpy(case["u_accept"]).to(d)
    us = torch.from_numpy(case["u_sample"]).to(d)
    kind = sv.SV_KIND_ONEHOT if onehot else sv.SV_KIND_DENSE
    ws = sv.workspace(kind, B, G, V, d)
    out = {}

    def step(i):
        c = i % ncopies
        if onehot:
            sv.sv_verify_onehot_draft(tgts[c], ids, ua, us, case["temperature"], bonus=case["bonus"], out=out, ws=ws)
        else:
            sv.sv_verify_dense(tgts[c], dfts[c], ids, ua, us, case["temperature"], bonus=case["bonus"], out=out,
                               ws=ws)

    ms, wall_ms = time_region(step, steps, warmup, torch)
    n = out["n_accepted"].cpu().numpy()
    tok = out["out_token"].cpu().numpy()
    draws = int((tok >= 0).sum())
    # a residual draw re-reads the rejected row (both tensors for dense); a bonus draw reads target row gamma
    resid = int(((n >= 0) & (n < G)).sum())
    bonus_draws = draws - resid
    draw_bytes = resid * (1 if onehot else 2) * V * s + bonus_draws * V * s
    total_bytes = verified_bytes + draw_bytes
    gbps, frac = hbm(total_bytes, ms)
    return dict(ms_per_step=ms, wall_ms_per_step=wall_ms, positions=B * G, positions_per_s=B * G / (ms * 1e-3),
                algorithmic_bytes=total_bytes, hbm_GBps=gbps, hbm_frac=frac, mean_n_accepted=float(n.mean()),
                residual_draws=resid, bonus_draws=bonus_draws, input_copies=ncopies,
                roofline=roofline(total_bytes, ms, "k_verify<bf16>" if s == 2 else "k_verify<f32>", traffic))


# ----------------------------------------------------------------------------------------------------------------------
# dense -> support -> sparse chain
# ----------------------------------------------------------------------------------------------------------------------

SUPPORT = "support_chain_B64_g16_V151936_k50_p095_bf16"


def bench_support(case, steps, warmup, torch, sv, d, k=50, top_p=0.95):
    """Dense -> sparse -> verify on the headline workload's logits: top-k / top-p supports of the target rows
    (B x (gamma+1)) and of the draft rows (B x gamma) in one launch, then the sparse verify of the drafted ids on
    them. Each kernel is timed alone in its own region (the two row sets also each in a launch of its own), then the
    whole chain."""
    B, G, V = case["B"], case["gamma"], case["V"]
    rows_t, rows_d = B * (G + 1), B * G
    ncopies = 2                                                         # 1.28 GB per step pair: no cache reuse
    tgts = [to_dev_logits(case["target"], "bf16", torch, d).view(rows_t, V) for _ in range(ncopies)]
    dfts = [to_dev_logits(case["draft"], "bf16", torch, d).view(rows_d, V) for _ in range(ncopies)]
    ids = torch.from_numpy(case["draft_ids"]).to(d)
    ua = torch.from_numpy(case["u_accept"]).to(d)
    us = torch.from_numpy(case["u_sample"]).to(d)
    ws = sv.support_workspace(rows_t + rows_d, V, k, d)
    po, qo, vo = {}, {}, {}

    def sup_t(i):
        sv.sv_build_support(tgts[i % ncopies], k, top_p, case["temperature"], True, out=po, ws=ws)

    def sup_d(i):
        sv.sv_build_support(dfts[i % ncopies], k, top_p, case["temperature"], True, out=qo, ws=ws)

    def sup_pair(i):
        sv.sv_build_support_pair(tgts[i % ncopies], dfts[i % ncopies], k, top_p, case["temperature"], True,
                                 out_a=po, out_b=qo, ws=ws)

    def verify(i):
        sv.sv_verify_sparse(po["ids"].view(B, G + 1, k), po["probs"].view(B, G + 1, k), qo["ids"].view(B, G, k),
                            qo["probs"].view(B, G, k), ids, ua, us, bonus=1, vocab_size=V, out=vo)

    def chain(i):
        sup_pair(i)
        verify(i)

    kt, _ = time_region(sup_t, steps, warmup, torch)
    kd, _ = time_region(sup_d, steps, warmup, torch)
    kp, _ = time_region(sup_pair, steps, warmup, torch)
    kv, _ = time_region(verify, steps, warmup, torch)
    ms, wall = time_region(chain, steps, warmup, torch)
    out_row = k * 8 + 8                                                 # ids, probs, count, flags per row
    bytes_t, bytes_d = rows_t * (V * 2 + out_row), rows_d * (V * 2 + out_row)
    n = vo["n_accepted"].cpu().numpy()
    gt, ft = hbm(bytes_t, kt)
    gd, fd = hbm(bytes_d, kd)
    gp, fp = hbm(bytes_t + bytes_d, kp)
    return dict(ms_per_step=ms, wall_ms_per_step=wall, positions=B * G, positions_per_s=B * G / (ms * 1e-3),
                k=k, top_p=top_p, mean_n_accepted=float(n.mean()),
                mean_kept_target=float(po["count"].float().mean().item()),
                mean_kept_draft=float(qo["count"].float().mean().item()),
                support_ms_pair=kp, support_ms_target=kt, support_ms_draft=kd, sparse_ms=kv,
                support_bytes_target=bytes_t, support_bytes_draft=bytes_d,
                support_GBps_pair=gp, support_frac_pair=fp,
                support_GBps_target=gt, support_GBps_draft=gd, support_frac_target=ft, support_frac_draft=fd,
                roofline=roofline(bytes_t + bytes_d, kp, "k_support<bf16> (target and draft rows, one launch)",
                                  profile_traffic("k_support.txt",
                                                  "support_chain target and draft rows (2112 x 151936 bf16)")))


# ----------------------------------------------------------------------------------------------------------------------
# greedy, commit
# ----------------------------------------------------------------------------------------------------------------------

GREEDY = "greedy_block_B64_g16_V151936_bf16"


def bench_greedy(steps, warmup, torch, sv, d):
    """Greedy (T = 0) verification of the block workload's shape: B = 64, gamma = 16, V = 151936, bf16 target with
    the Zipf bias; drafts equal the target argmax with probability 0.85. Every target row (gamma + 1 per sequence)
    is read once; one launch of k_greedy per step."""
    from lossless_draft_verification_spec_amd import workloads
    case = workloads.greedy_case(64, 16, 151936, seed=0)
    B, G, V = case["B"], case["gamma"], case["V"]
    ncopies = 3                                                         # 0.99 GB: no reuse in the 256 MB cache
    tgts = [to_dev_logits(case["target"], "bf16", torch, d) for _ in range(ncopies)]
    ids = torch.from_numpy(case["draft_ids"]).to(d)
    ws = sv.workspace(sv.SV_KIND_GREEDY, B, G, V, d)
    out = {}

    def step(i):
        sv.sv_verify_greedy(tgts[i % ncopies], ids, bonus=1, out=out, ws=ws)

    ms, wall = time_region(step, steps, warmup, torch)
    # every target row once, the draft ids, and accept / n / token / flags written
    nbytes = B * (G + 1) * V * 2 + B * G * 4 + B * G + B * 12
    n = out["n_accepted"].cpu().numpy()
    del tgts
    gbps, frac = hbm(nbytes, ms)
    return dict(ms_per_step=ms, wall_ms_per_step=wall, positions=B * G, positions_per_s=B * G / (ms * 1e-3),
                mean_n_accepted=float(n.mean()), algorithmic_bytes=nbytes, hbm_GBps=gbps, hbm_frac=frac,
                input_copies=ncopies, roofline=roofline(nbytes, ms, "k_greedy<bf16>",
                                                        profile_traffic("k_greedy.txt", GREEDY)))


COMMIT = "commit_block_B256_W4_V151936_bf16"


def bench_commit(steps, warmup, torch, sv, d):
    """Confidence-threshold commit of masked-diffusion blocks: B = 256 blocks of W = 4 slots over V = 151936, bf16,
    three quarters of the slots still masked, tau = 0.9. Only masked slots are read; one launch per step."""
    from lossless_draft_verification_spec_amd import workloads
    case = workloads.commit_case(256, 4, 151936, seed=0)
    B, Wn, V = case["B"], case["W"], case["V"]
    ncopies = 4                                                         # 1.24 GB: no reuse in the 256 MB cache
    zs = [to_dev_logits(case["logits"], "bf16", torch, d) for _ in range(ncopies)]
    masked = torch.from_numpy(case["masked"]).to(d)
    ws = sv.workspace(sv.SV_KIND_GREEDY, B, Wn, V, d)
    out = {}

    def step(i):
        sv.sv_confidence_commit(zs[i % ncopies], case["tau"], masked, out=out, ws=ws)

    ms, wall = time_region(step, steps, warmup, torch)
    nm = int(case["masked"].sum())
    # every masked row once, the mask, and commit / token / confidence per slot and the count and flags per block
    nbytes = nm * V * 2 + B * Wn + B * Wn * 9 + B * 8
    del zs
    gbps, frac = hbm(nbytes, ms)
    return dict(ms_per_step=ms, wall_ms_per_step=wall, slots=B * Wn, masked_slots=nm,
                committed=int(out["n_commit"].sum().item()), algorithmic_bytes=nbytes, hbm_GBps=gbps,
                hbm_frac=frac, roofline=roofline(nbytes, ms, "k_greedy<bf16> (commit mode)",
                                                 profile_traffic("k_greedy.txt", COMMIT)))


# ----------------------------------------------------------------------------------------------------------------------
# sparse, windows
# ----------------------------------------------------------------------------------------------------------------------

def bench_sparse(case, steps, warmup, torch, sv, d):
    B, G = case["B"], case["gamma"]
    t = {key: torch.from_numpy(np.ascontiguousarray(case[key])).to(d)
         for key in ("p_ids", "p_probs", "q_ids", "q_probs", "spec_ids", "u_accept", "u_sample")}
    out = {}

    def step(i):
        sv.sv_verify_sparse(t["p_ids"], t["p_probs"], t["q_ids"], t["q_probs"], t["spec_ids"], t["u_accept"],
                            t["u_sample"], bonus=1, vocab_size=case["V"], out=out)

    ms, wall = time_region(step, steps, warmup, torch)
    in_bytes = sum(int(v.numel() * v.element_size()) for v in t.values())
    out_bytes = sum(int(v.numel() * v.element_size()) for v in out.values())
    gbps, frac = hbm(in_bytes + out_bytes, ms)
    return dict(ms_per_step=ms, wall_ms_per_step=wall, positions=B * G, positions_per_s=B * G / (ms * 1e-3),
                algorithmic_bytes=in_bytes + out_bytes, hbm_GBps=gbps, hbm_frac=frac,
                roofline=roofline(in_bytes + out_bytes, ms, "k_sparse",
                                  profile_traffic("k_sparse.txt", "sparse_B1024_g16_k64_V151936")))


def bench_window(case, steps, warmup, torch, sv, d):
    """The masked-diffusion window: every step runs the 4 chained rounds from start = 0. Events recorded between the
    rounds of each step give each round's time; the chain's time is the whole step."""
    B, W, V, R = case["B"], case["gamma"], case["V"], case["rounds"]
    tgt = to_dev_logits(case["target"], "f32", torch, d)
    dft = to_dev_logits(case["draft"], "f32", torch, d)
    ids = torch.from_numpy(case["draft_ids"]).to(d)
    order = torch.from_numpy(case["order"]).to(d)
    ua = [torch.from_numpy(case["u_accept"][r]).to(d) for r in range(R)]
    us = [torch.from_numpy(case["u_sample"][r]).to(d) for r in range(R)]
    ws = sv.workspace(sv.SV_KIND_DENSE, B, W, V, d)
    start = torch.zeros(B, dtype=torch.int32, device=d)
    zero = torch.zeros(B, dtype=torch.int32, device=d)
    outs = [dict() for _ in range(R)]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(R + 1)] for _ in range(steps)]
    state = {"timed": False}

    def step(i):
        start.copy_(zero)
        for r in range(R):
            if state["timed"]:
                evs[i][r].record()
            sv.sv_verify_dense(tgt, dft, ids, ua[r], us[r], case["temperature"], bonus=0, start=start, order=order,
                               out=outs[r], ws=ws)
        if state["timed"]:
            evs[i][R].record()

    ms, wall = time_region(step, steps, warmup, torch)
    state["timed"] = True
    time_region(step, steps, 0, torch)
    round_ms = [float(np.mean([evs[i][r].elapsed_time(evs[i][r + 1]) for i in range(steps)])) for r in range(R)]
    # verified positions and bytes of each round, replayed once with the starts observed per round
    start.zero_()
    rounds = []
    for r in range(R):
        st = start.cpu().numpy()
        verified = int(np.sum(W - st))
        sv.sv_verify_dense(tgt, dft, ids, ua[r], us[r], case["temperature"], bonus=0, start=start, order=order,
                           out=outs[r], ws=ws)
        tok = outs[r]["out_token"].cpu().numpy()
        nbytes = 2 * verified * V * 4 + int((tok >= 0).sum()) * 2 * V * 4
        gbps, frac = hbm(nbytes, round_ms[r])
        rounds.append(dict(round=r, ms=round_ms[r], positions=verified, positions_per_s=verified / (round_ms[r] * 1e-3),
                           algorithmic_bytes=nbytes, logits=2 * verified * V, hbm_GBps=gbps, hbm_frac=frac))
    torch.cuda.synchronize()
    positions = sum(x["positions"] for x in rounds)
    total_bytes = sum(x["algorithmic_bytes"] for x in rounds)
    gbps, frac = hbm(total_bytes, ms)
    return dict(ms_per_step=ms, wall_ms_per_step=wall, rounds=rounds, positions=positions,
                positions_per_s=positions / (ms * 1e-3), algorithmic_bytes=total_bytes, hbm_GBps=gbps, hbm_frac=frac,
                roofline=roofline(rounds[0]["algorithmic_bytes"], rounds[0]["ms"], "k_verify<f32> (round 0)",
                                  profile_traffic("k_verify.txt", "window_B32_W32_V262144_r4 round 0")))


# ----------------------------------------------------------------------------------------------------------------------
# tree verification
# ----------------------------------------------------------------------------------------------------------------------

TREE = "tree_B64_N17_V151936_bf16"


def bench_tree(steps, warmup, torch, sv, d):
    from lossless_draft_verification_spec_amd import workloads
    case = workloads.make(TREE)
    B, N, V = case["B"], case["N"], case["V"]
    ncopies = 3
    tgts = [to_dev_logits(case["target"], "bf16", torch, d) for _ in range(ncopies)]
    par = torch.from_numpy(case["parent"]).to(d)
    tok = torch.from_numpy(case["token"]).to(d)
    ua = torch.from_numpy(case["u_accept"]).to(d)
    us = torch.from_numpy(case["u_sample"]).to(d)
    ws = sv.workspace(sv.SV_KIND_TREE, B, N, V, d)
    out = {}

    def step(i):
        sv.sv_verify_tree(tgts[i % ncopies], par, tok, ua, us, case["temperature"], out=out, ws=ws)

    ms, wall = time_region(step, steps, warmup, torch)
    n = out["n_accepted"].cpu().numpy()
    # every node row once; the stop node's row once more for the draw
    nbytes = B * N * V * 2 + int((out["out_token"].cpu().numpy() >= 0).sum()) * V * 2
    gbps, frac = hbm(nbytes, ms)
    del tgts
    return dict(ms_per_step=ms, wall_ms_per_step=wall, sequences=B, nodes=N, mean_accepted_path=float(n.mean()),
                algorithmic_bytes=nbytes, hbm_GBps=gbps, hbm_frac=frac,
                roofline=roofline(nbytes, ms, "k_tree<bf16>", profile_traffic("k_tree.txt", TREE)))


# ----------------------------------------------------------------------------------------------------------------------
# CPU baseline (the oracle as it stands)
# ----------------------------------------------------------------------------------------------------------------------

_POOL_CASE = None


def _oracle_slice(b0):
    import oracle
    c = _POOL_CASE
    sl = slice(b0, b0 + 4)
    oracle.verify_dense(c["target"][sl], c["draft"][sl], c["draft_ids"][sl], c["u_accept"][sl], c["u_sample"][sl],
                        c["temperature"], dtype=c["dtype"])
    return c["draft_ids"][sl].shape[0]


def cpu_baseline(case, seconds):
    """The float64 oracle on bounded samples of the headline workload (4 whole sequences per task): one thread in
    this process for about `seconds`, then a pool of worker processes, one per usable core (at most 16), for about as
    long. Runs before the GPU is touched, so the workers are plain CPU processes."""
    global _POOL_CASE
    import oracle
    B, G = case["B"], case["gamma"]
    t0 = time.perf_counter()
    done, b = 0, 0
    while time.perf_counter() - t0 < seconds:
        sl = slice(b % B, b % B + 4)
        oracle.verify_dense(case["target"][sl], case["draft"][sl], case["draft_ids"][sl], case["u_accept"][sl],
                            case["u_sample"][sl], case["temperature"], dtype=case["dtype"])
        done += case["draft_ids"][sl].shape[0]
        b += 4
    dt1 = time.perf_counter() - t0
    rate1 = done * G / dt1
    cores = min(CPU_POOL_MAX, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count())
    _POOL_CASE = case
    per_task = dt1 / max(1, done // 4)
    ntask = max(cores, int(round(seconds / per_task)) * cores)
    starts = [(4 * i) % B for i in range(ntask)]
    with mp.get_context("fork").Pool(cores) as pool:
        pool.map(_oracle_slice, [0] * cores)                   # workers started and warm
        t0 = time.perf_counter()
        seqs = sum(pool.map(_oracle_slice, starts, chunksize=1))
        dtp = time.perf_counter() - t0
    _POOL_CASE = None
    ratep = seqs * G / dtp
    log(f"cpu oracle: {rate1:.0f} positions/s on 1 thread, {ratep:.0f} on {cores} processes")
    return dict(value=ratep, unit="positions/s", cores=cores, kind="oracle",
                sample=f"{seqs} sequences x {G} drafts of the headline workload (4 per task, wrapping over its {B}) "
                       f"on a pool of {cores} worker processes in {dtp:.1f} s; numpy float64",
                single_thread=dict(value=rate1, cores=1, sample=f"{done} sequences in {dt1:.1f} s, one thread"))


# ----------------------------------------------------------------------------------------------------------------------
# measured HBM traffic from committed counter summaries
# ----------------------------------------------------------------------------------------------------------------------

def _sources_sha(names):
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "lossless_draft_verification_spec_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_traffic(profile, key):
    """HBM bytes per launch from a committed FETCH_SIZE / WRITE_SIZE summary (line 'TRAFFIC_JSON {...}' holding
    source_files, source_sha256 and per-workload traffic_bytes), or None when the kernel's sources have changed since
    the counters were taken."""
    try:
        rec = None
        with open(os.path.join(ROOT, "profiles", profile)) as f:
            for ln in f:
                if ln.startswith("TRAFFIC_JSON "):
                    rec = json.loads(ln[len("TRAFFIC_JSON "):])
        if rec is None or rec.get("source_sha256") != _sources_sha(rec["source_files"]):
            return None
        return int(rec["workloads"][key]["traffic_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", default=None,
                    help="time only this workload besides the headline ('headline': the headline alone)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy, the reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); sequences shard across GPUs with no "
              f"exchange, so the per-GPU figure is the one this run measures.", file=sys.stderr)
        sys.exit(2)

    from lossless_draft_verification_spec_amd import workloads
    log("generating", HEADLINE)
    head = workloads.make(HEADLINE)
    cpu = None if args.no_cpu else cpu_baseline(head, args.cpu_seconds)

    import torch
    from lossless_draft_verification_spec_amd import sv

    d = torch.device("cuda", 0)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=d)        # 1 GiB read + 1 GiB written per copy
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 3 x 1 GiB")
        del src, dst
        torch.cuda.empty_cache()
    r = bench_dense(head, args.steps, args.warmup, torch, sv, d,
                    traffic=profile_traffic("k_verify.txt", HEADLINE))
    log("headline", json.dumps(r))

    others = {}
    legs = [(SUPPORT, lambda: bench_support(head, args.steps, args.warmup, torch, sv, d)),
            (GREEDY, lambda: bench_greedy(args.steps, args.warmup, torch, sv, d)),
            (COMMIT, lambda: bench_commit(args.steps, args.warmup, torch, sv, d))]
    if hasattr(sv, "sv_verify_tree"):
        legs.append((TREE, lambda: bench_tree(args.steps, args.warmup, torch, sv, d)))
    for name, fn in legs:
        if args.only in (None, name):
            others[name] = fn()
            log(name, json.dumps(others[name]))
            torch.cuda.empty_cache()
    del head
    names = [n for n in workloads.WORKLOADS if n != HEADLINE and n != TREE]
    if args.only:
        names = [n for n in names if n == args.only]
    for name in names:
        log("generating", name)
        c = workloads.make(name)
        if c["kind"] in ("dense", "onehot"):
            others[name] = bench_dense(c, args.steps, args.warmup, torch, sv, d,
                                       traffic=profile_traffic("k_verify.txt", name))
        elif c["kind"] == "sparse":
            others[name] = bench_sparse(c, args.steps, args.warmup, torch, sv, d)
        else:
            others[name] = bench_window(c, max(5, args.steps // 4), min(args.warmup, 3), torch, sv, d)
        log(name, json.dumps(others[name]))
        del c
        torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": r["positions_per_s"], "unit": "positions/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": HEADLINE, "B": 64, "gamma": 16, "V": 151936, "logits": "bf16", "temperature": 1.0,
                   "bonus": 1},
        "hbm_GBps": r["hbm_GBps"], "hbm_frac_of_peak": r["hbm_frac"],
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
        "workloads": {HEADLINE: r, **others},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
