"""Benchmark of the speculative-sampling verifier on one MI355X.

One step = one full verification call (statistics, accept/first-reject scan, float64 draw: one kernel launch) over the
dense block workload: B=64 sequences, gamma=16 drafts, V=151936, bf16 target and draft logits (synthetic, seeded). The
headline value is verified draft positions per second; the roofline object reports the verifier kernel's achieved HBM
bandwidth: algorithmic bytes per launch (every verified logit of both tensors, 2*B*gamma*V*2, plus the row pair each
rejected sequence's draw reads again, or the target row of a bonus draw) over its average duration, timed with HIP
events taken from the kernel's own dispatch on its stream, in a second timed region of the same steps (the whole-call
figure comes from steps without the events). The other workloads (the dense -> top-k/top-p support -> sparse verify
chain on the headline's logits, tiny dense, greedy one-hot, sparse top-64, masked-diffusion window with 4 chained
rounds) are timed after it and reported under "workloads".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--cpu-seconds S] [--only NAME]
Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import ctypes
import json
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t pairs from the process's HIP runtime (the one torch loaded)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0 and self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a, b))

    def elapsed_ms(self, i):
        ms = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.pairs[i][0], self.pairs[i][1])
        assert st == 0, f"hipEventElapsedTime failed: {st}"
        return ms.value

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


def to_dev_logits(x, dtype, torch, d):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.view(torch.bfloat16) if dtype == "bf16" else t).to(d)


def time_steps(fn, steps, warmup, torch):
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
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall / steps * 1e3


def bench_dense(case, steps, warmup, torch, sv, d, profile_events=True):
    """Dense or one-hot workload: returns timing and byte accounting."""
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
    ev = HipEvents(steps) if profile_events else None
    state = {"timed": False}

    def step(i):
        c = i % ncopies
        if state["timed"] and ev is not None:
            sv.sv_profile_next_stats(ev.pairs[i][0], ev.pairs[i][1])
        if onehot:
            sv.sv_verify_onehot_draft(tgts[c], ids, ua, us, case["temperature"], bonus=case["bonus"], out=out, ws=ws)
        else:
            sv.sv_verify_dense(tgts[c], dfts[c], ids, ua, us, case["temperature"], bonus=case["bonus"], out=out,
                               ws=ws)

    def region(profiled):
        state["timed"] = profiled
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        state["timed"] = False
        return e0.elapsed_time(e1) / steps, (time.perf_counter() - t0) * 1e3 / steps

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # The whole-call figure comes from steps with no event hook; a second region of the same steps records the
    # kernel's own start/stop events on every launch.
    ms, wall_ms = region(False)
    stats_ms = None
    if ev is not None:
        ms_profiled, _ = region(True)
        stats_ms = float(np.mean([ev.elapsed_ms(i) for i in range(steps)]))
        ev.close()
    n = out["n_accepted"].cpu().numpy()
    tok = out["out_token"].cpu().numpy()
    draws = int((tok >= 0).sum())
    # a residual draw re-reads the rejected row (both tensors for dense); a bonus draw reads target row gamma
    resid = int(((n >= 0) & (n < G)).sum())
    bonus_draws = draws - resid
    draw_bytes = resid * (1 if onehot else 2) * V * s + bonus_draws * V * s
    total_bytes = verified_bytes + draw_bytes
    res = dict(ms_per_step=ms, wall_ms_per_step=wall_ms, positions=B * G, positions_per_s=B * G / (ms * 1e-3),
               algorithmic_bytes=total_bytes, hbm_GBps=total_bytes / (ms * 1e-3) / 1e9,
               hbm_frac=total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, mean_n_accepted=float(n.mean()),
               input_copies=ncopies)
    if stats_ms is not None:
        res.update(ms_per_step_with_kernel_events=ms_profiled, kernel_ms=stats_ms, kernel_bytes=total_bytes,
                   kernel_GBps=total_bytes / (stats_ms * 1e-3) / 1e9)
    return res


SUPPORT = "support_chain_B64_g16_V151936_k50_p095_bf16"


def bench_support(case, steps, warmup, torch, sv, d, k=50, top_p=0.95):
    """Dense -> sparse -> verify on the headline workload's logits: top-k / top-p supports of the target rows
    (B x (gamma+1)) and of the draft rows (B x gamma), then the sparse verify of the drafted ids on them. The two
    support builds are timed from their own dispatches (HIP events) in a second region of the same steps."""
    B, G, V = case["B"], case["gamma"], case["V"]
    rows_t, rows_d = B * (G + 1), B * G
    ncopies = 2                                                         # 1.28 GB per step pair: no cache reuse
    tgts = [to_dev_logits(case["target"], "bf16", torch, d).view(rows_t, V) for _ in range(ncopies)]
    dfts = [to_dev_logits(case["draft"], "bf16", torch, d).view(rows_d, V) for _ in range(ncopies)]
    ids = torch.from_numpy(case["draft_ids"]).to(d)
    ua = torch.from_numpy(case["u_accept"]).to(d)
    us = torch.from_numpy(case["u_sample"]).to(d)
    ws_t = sv.support_workspace(rows_t, V, k, d)
    ws_d = sv.support_workspace(rows_d, V, k, d)
    po, qo, vo = {}, {}, {}
    ev_t, ev_d = HipEvents(steps), HipEvents(steps)
    state = {"timed": False}

    def step(i):
        c = i % ncopies
        if state["timed"]:
            sv.sv_profile_next_stats(ev_t.pairs[i][0], ev_t.pairs[i][1])
        sv.sv_build_support(tgts[c], k, top_p, case["temperature"], True, out=po, ws=ws_t)
        if state["timed"]:
            sv.sv_profile_next_stats(ev_d.pairs[i][0], ev_d.pairs[i][1])
        sv.sv_build_support(dfts[c], k, top_p, case["temperature"], True, out=qo, ws=ws_d)
        sv.sv_verify_sparse(po["ids"].view(B, G + 1, k), po["probs"].view(B, G + 1, k), qo["ids"].view(B, G, k),
                            qo["probs"].view(B, G, k), ids, ua, us, bonus=1, vocab_size=V, out=vo)

    ms, wall = time_steps(step, steps, warmup, torch)
    state["timed"] = True
    time_steps(step, steps, 0, torch)
    state["timed"] = False
    kt = float(np.mean([ev_t.elapsed_ms(i) for i in range(steps)]))
    kd = float(np.mean([ev_d.elapsed_ms(i) for i in range(steps)]))
    ev_t.close()
    ev_d.close()
    out_row = k * 8 + 8                                                 # ids, probs, count, flags per row
    bytes_t, bytes_d = rows_t * (V * 2 + out_row), rows_d * (V * 2 + out_row)
    n = vo["n_accepted"].cpu().numpy()
    return dict(ms_per_step=ms, wall_ms_per_step=wall, positions=B * G, positions_per_s=B * G / (ms * 1e-3),
                k=k, top_p=top_p, mean_n_accepted=float(n.mean()),
                mean_kept_target=float(po["count"].float().mean().item()),
                mean_kept_draft=float(qo["count"].float().mean().item()),
                support_kernel_ms_target=kt, support_kernel_ms_draft=kd,
                support_bytes_target=bytes_t, support_bytes_draft=bytes_d,
                support_GBps_target=bytes_t / (kt * 1e-3) / 1e9, support_GBps_draft=bytes_d / (kd * 1e-3) / 1e9,
                support_hbm_frac=(bytes_t + bytes_d) / ((kt + kd) * 1e-3) / 1e9 / HBM_PEAK_GBPS)


GREEDY = "greedy_block_B64_g16_V151936_bf16"


def bench_greedy(steps, warmup, torch, sv, d):
    """Greedy (T = 0) verification of the block workload's shape: B = 64, gamma = 16, V = 151936, bf16 target with
    the Zipf bias; drafts equal the target argmax with probability 0.85. Every target row (gamma + 1 per sequence)
    is read once; the kernel is timed from its own dispatches in a second region of the same steps."""
    from lossless_draft_verification_spec_amd import workloads
    case = workloads.greedy_case(64, 16, 151936, seed=0)
    B, G, V = case["B"], case["gamma"], case["V"]
    ncopies = 3                                                         # 0.99 GB: no reuse in the 256 MB cache
    tgts = [to_dev_logits(case["target"], "bf16", torch, d) for _ in range(ncopies)]
    ids = torch.from_numpy(case["draft_ids"]).to(d)
    ws = sv.workspace(sv.SV_KIND_GREEDY, B, G, V, d)
    out = {}
    ev = HipEvents(steps)
    state = {"timed": False}

    def step(i):
        if state["timed"]:
            sv.sv_profile_next_stats(ev.pairs[i][0], ev.pairs[i][1])
        sv.sv_verify_greedy(tgts[i % ncopies], ids, bonus=1, out=out, ws=ws)

    ms, wall = time_steps(step, steps, warmup, torch)
    state["timed"] = True
    time_steps(step, steps, 0, torch)
    state["timed"] = False
    km = float(np.mean([ev.elapsed_ms(i) for i in range(steps)]))
    ev.close()
    # every target row once, the draft ids, and accept / n / token / flags written
    nbytes = B * (G + 1) * V * 2 + B * G * 4 + B * G + B * 12
    n = out["n_accepted"].cpu().numpy()
    del tgts
    gbps = nbytes / (km * 1e-3) / 1e9
    return dict(ms_per_step=ms, wall_ms_per_step=wall, positions=B * G, positions_per_s=B * G / (ms * 1e-3),
                mean_n_accepted=float(n.mean()), kernel_ms=km, kernel_bytes=nbytes, kernel_GBps=gbps,
                kernel_hbm_frac=gbps / HBM_PEAK_GBPS, input_copies=ncopies,
                roofline={"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": gbps / HBM_PEAK_GBPS, "traffic": greedy_traffic(), "kernel": "k_greedy"})


COMMIT = "commit_block_B256_W4_V151936_bf16"


def bench_commit(steps, warmup, torch, sv, d):
    """Confidence-threshold commit of masked-diffusion blocks: B = 256 blocks of W = 4 slots over V = 151936, bf16,
    three quarters of the slots still masked, tau = 0.9. Only masked slots are read; the kernel is timed from its own
    dispatches in a second region of the same steps."""
    from lossless_draft_verification_spec_amd import workloads
    case = workloads.commit_case(256, 4, 151936, seed=0)
    B, Wn, V = case["B"], case["W"], case["V"]
    ncopies = 4                                                         # 1.24 GB: no reuse in the 256 MB cache
    zs = [to_dev_logits(case["logits"], "bf16", torch, d) for _ in range(ncopies)]
    masked = torch.from_numpy(case["masked"]).to(d)
    ws = sv.workspace(sv.SV_KIND_GREEDY, B, Wn, V, d)
    out = {}
    ev = HipEvents(steps)
    state = {"timed": False}

    def step(i):
        if state["timed"]:
            sv.sv_profile_next_stats(ev.pairs[i][0], ev.pairs[i][1])
        sv.sv_confidence_commit(zs[i % ncopies], case["tau"], masked, out=out, ws=ws)

    ms, wall = time_steps(step, steps, warmup, torch)
    state["timed"] = True
    time_steps(step, steps, 0, torch)
    state["timed"] = False
    km = float(np.mean([ev.elapsed_ms(i) for i in range(steps)]))
    ev.close()
    nm = int(case["masked"].sum())
    # every masked row once, the mask, and commit / token / confidence per slot and the count and flags per block
    nbytes = nm * V * 2 + B * Wn + B * Wn * 9 + B * 8
    gbps = nbytes / (km * 1e-3) / 1e9
    del zs
    return dict(ms_per_step=ms, wall_ms_per_step=wall, slots=B * Wn, masked_slots=nm,
                committed=int(out["n_commit"].sum().item()), kernel_ms=km, kernel_bytes=nbytes, kernel_GBps=gbps,
                kernel_hbm_frac=gbps / HBM_PEAK_GBPS,
                roofline={"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": gbps / HBM_PEAK_GBPS,
                          "traffic": greedy_traffic("k_greedy_commit_block_traffic.txt", "masked"),
                          "kernel": "k_greedy (commit mode)"})


def bench_sparse(case, steps, warmup, torch, sv, d):
    B, G, k = case["B"], case["gamma"], case["k"]
    t = {key: torch.from_numpy(np.ascontiguousarray(case[key])).to(d)
         for key in ("p_ids", "p_probs", "q_ids", "q_probs", "spec_ids", "u_accept", "u_sample")}
    out = {}

    def step(i):
        sv.sv_verify_sparse(t["p_ids"], t["p_probs"], t["q_ids"], t["q_probs"], t["spec_ids"], t["u_accept"],
                            t["u_sample"], bonus=1, vocab_size=case["V"], out=out)

    ms, wall = time_steps(step, steps, warmup, torch)
    in_bytes = sum(int(v.numel() * v.element_size()) for v in t.values())
    out_bytes = sum(int(v.numel() * v.element_size()) for v in out.values())
    return dict(ms_per_step=ms, wall_ms_per_step=wall, positions=B * G, positions_per_s=B * G / (ms * 1e-3),
                algorithmic_bytes=in_bytes + out_bytes, hbm_GBps=(in_bytes + out_bytes) / (ms * 1e-3) / 1e9)


def bench_window(case, steps, warmup, torch, sv, d):
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

    def step(i):
        start.copy_(zero)
        for r in range(R):
            sv.sv_verify_dense(tgt, dft, ids, ua[r], us[r], case["temperature"], bonus=0, start=start, order=order,
                               out=outs[r], ws=ws)

    ms, wall = time_steps(step, steps, warmup, torch)
    # verified positions and bytes of the chain, replayed once with the starts observed per round
    start.zero_()
    positions, total_bytes = 0, 0
    for r in range(R):
        st = start.cpu().numpy()
        verified = int(np.sum(W - st))
        sv.sv_verify_dense(tgt, dft, ids, ua[r], us[r], case["temperature"], bonus=0, start=start, order=order,
                           out=outs[r], ws=ws)
        tok = outs[r]["out_token"].cpu().numpy()
        positions += verified
        total_bytes += 2 * verified * V * 4 + int((tok >= 0).sum()) * 2 * V * 4
    torch.cuda.synchronize()
    return dict(ms_per_step=ms, wall_ms_per_step=wall, rounds=R, positions=positions,
                positions_per_s=positions / (ms * 1e-3), algorithmic_bytes=total_bytes,
                hbm_GBps=total_bytes / (ms * 1e-3) / 1e9, hbm_frac=total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)


def cpu_baseline(case, seconds):
    """The float64 oracle, as it stands, on a bounded sample of the headline workload (whole sequences)."""
    import oracle
    B, G = case["B"], case["gamma"]
    t0 = time.perf_counter()
    done = 0
    b = 0
    while time.perf_counter() - t0 < seconds:
        sl = slice(b % B, b % B + 4)
        oracle.verify_dense(case["target"][sl], case["draft"][sl], case["draft_ids"][sl], case["u_accept"][sl],
                            case["u_sample"][sl], case["temperature"], dtype=case["dtype"])
        done += case["draft_ids"][sl].shape[0]
        b += 4
    dt = time.perf_counter() - t0
    return dict(value=done * G / dt, unit="positions/s", cores=1, kind="oracle",
                sample=f"{done} of the {B} sequences x {G} drafts (4 at a time, wrapping) in {dt:.1f} s, "
                       f"numpy float64, one thread")


KERNEL_SOURCES = ("sv_dense.hip", "sv_device.h", "sv_internal.h")    # what k_verify is compiled from


def kernel_source_sha():
    """sha256 over the verifier kernel's source files, in KERNEL_SOURCES order."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "lossless_draft_verification_spec_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


GREEDY_SOURCES = ("sv_greedy.hip", "sv_greedy.h", "sv_device.h", "sv_internal.h")   # what k_greedy is built from


def greedy_traffic(profile="k_greedy_block_traffic.txt", key="target"):
    """HBM bytes per launch of k_greedy (greedy verification, or commit mode with the commit profile) from the
    committed counter summary, or None when its sources have changed since the counters were taken."""
    import hashlib
    h = hashlib.sha256()
    try:
        for name in GREEDY_SOURCES:
            with open(os.path.join(ROOT, "lossless_draft_verification_spec_amd", "csrc", name), "rb") as f:
                h.update(f.read())
        rec = None
        with open(os.path.join(ROOT, "profiles", profile)) as f:
            for ln in f:
                if ln.startswith("TRAFFIC_JSON "):
                    rec = json.loads(ln[len("TRAFFIC_JSON "):])
    except OSError:
        return None
    if rec is None or rec.get("source_sha256") != h.hexdigest():
        return None
    return int(rec[key]["traffic_bytes"])


def measured_traffic():
    """HBM bytes per launch of the verifier kernel from the committed FETCH_SIZE / WRITE_SIZE counter summary, or
    None when the kernel source has changed since the counters were taken."""
    prof = os.path.join(ROOT, "profiles", "k_verify_dense_block_traffic.txt")
    try:
        rec = None
        with open(prof) as f:
            for ln in f:
                if ln.startswith("TRAFFIC_JSON "):
                    rec = json.loads(ln[len("TRAFFIC_JSON "):])
        sha = kernel_source_sha()
    except OSError:
        return None
    if rec is None or rec.get("source_sha256") != sha:
        return None
    return int(rec["traffic_bytes"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", default=None,
                    help="time only this workload besides the headline ('headline': the headline alone)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy, the reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); sequences shard across GPUs with no "
              f"exchange, so the per-GPU figure is the one this run measures.", file=sys.stderr)
        sys.exit(2)

    import torch
    from lossless_draft_verification_spec_amd import sv, workloads

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
    log("generating", HEADLINE)
    head = workloads.make(HEADLINE)
    r = bench_dense(head, args.steps, args.warmup, torch, sv, d)
    log("headline", json.dumps(r))

    others = {}
    if args.only in (None, SUPPORT):
        others[SUPPORT] = bench_support(head, args.steps, args.warmup, torch, sv, d)
        log(SUPPORT, json.dumps(others[SUPPORT]))
        torch.cuda.empty_cache()
    if args.only in (None, GREEDY):
        others[GREEDY] = bench_greedy(args.steps, args.warmup, torch, sv, d)
        log(GREEDY, json.dumps(others[GREEDY]))
        torch.cuda.empty_cache()
    if args.only in (None, COMMIT):
        others[COMMIT] = bench_commit(args.steps, args.warmup, torch, sv, d)
        log(COMMIT, json.dumps(others[COMMIT]))
        torch.cuda.empty_cache()
    names = [n for n in workloads.WORKLOADS if n != HEADLINE]
    if args.only:
        names = [n for n in names if n == args.only]
    for name in names:
        log("generating", name)
        c = workloads.make(name)
        if c["kind"] in ("dense", "onehot"):
            others[name] = bench_dense(c, args.steps, args.warmup, torch, sv, d)
        elif c["kind"] == "sparse":
            others[name] = bench_sparse(c, args.steps, args.warmup, torch, sv, d)
        else:
            others[name] = bench_window(c, max(5, args.steps // 4), min(args.warmup, 3), torch, sv, d)
        log(name, json.dumps(others[name]))
        del c
        torch.cuda.empty_cache()

    cpu = None if args.no_cpu else cpu_baseline(head, args.cpu_seconds)
    line = {
        "metric": METRIC, "value": r["positions_per_s"], "unit": "positions/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": HEADLINE, "B": 64, "gamma": 16, "V": 151936, "logits": "bf16", "temperature": 1.0,
                   "bonus": 1},
        "hbm_GBps": r["hbm_GBps"], "hbm_frac_of_peak": r["hbm_frac"],
        "roofline": {"bound": "hbm", "achieved": r.get("kernel_GBps"), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": (r["kernel_GBps"] / HBM_PEAK_GBPS) if r.get("kernel_GBps") else None,
                     "traffic": measured_traffic(), "kernel": "k_verify (statistics, scan and draw)",
                     "traffic_unit": "B/launch", "kernel_ms": r.get("kernel_ms"), "kernel_bytes": r.get("kernel_bytes")},
        "cpu_baseline": cpu,
        "workloads": {HEADLINE: r, **others},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
