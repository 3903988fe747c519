#!/usr/bin/env python3
"""Benchmark of the tree-packed chunkwise gated-delta path on one MI355X.

One step = the whole hot path for one batch: the packed forward over every
round of the minimum-call plan (with state handoffs) followed by the backward
over every round in reverse (recompute, state-gradient pass with handoff
gradients, per-chunk gradients, replay-gradient fixup), on the 64-leaf
synthetic rollout tree (16384-token root, fan-out 2-4, fork offsets never
chunk-aligned, leaf lengths log-uniform in [64, 4096]), H=16, d_k=d_v=128,
B=64, bf16 inputs, fp32 state.  Planning (host, once per batch and reused by
every layer) and the input upload are outside the timed region and reported
separately.

Prints ONE JSON line:  metric / value (compact tokens/s) / roofline of the
dominant kernel / cpu_baseline (the float64 oracle on a bounded sample) /
the log-prob gather (32768 x 131072 bf16) as an extra HBM measurement.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s
RIDGE = PEAK_BF16 / PEAK_HBM
H, D, B = 16, 128, 64
ES = 2                  # bf16 bytes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-logprob", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--only-conv", action="store_true",
                    help="only the tree causal convolution (for profiling it alone)")
    ap.add_argument("--no-attn", action="store_true")
    ap.add_argument("--only-attn", action="store_true",
                    help="only the tree softmax attention (for profiling it alone)")
    ap.add_argument("--no-moe", action="store_true")
    ap.add_argument("--only-moe", action="store_true",
                    help="only the router statistics (for profiling them alone)")
    ap.add_argument("--only-logprob", action="store_true",
                    help="only the log-prob gather and its backward (for profiling them alone)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain device copy of known size (for HBM counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------------ algorithmic work per kernel
# Multiply-accumulates per chunk of l tokens (replay included) and head, d = d_k = d_v, for the
# products each kernel performs ("Kernels and their rooflines").  The benchmark
# runs the forward that keeps the backward's operands: kda_prep_fwd is then the preparation of
# both directions (A and M, W, U', Qeff, O', the diagonal-block inverse), kda_state_fwd also
# writes the chunk-start states, and the backward runs no kda_prep_bwd or kda_state_bwd.
def macs(kernel, l, d=D):
    l2d, ld2, l3 = l * l * d, l * d * d, l ** 3
    return {
        "kda_prep_fwd": 5 * l2d + l3 / 6,
        "kda_state_fwd": 3 * ld2,
        "kda_prep_bwd": 4 * l2d + l3 / 6,
        "kda_state_bwd": 2 * ld2,
        "kda_dstate": 3 * ld2,
        "kda_grad": 9 * l2d + 5 * ld2 + 2 * l3,
    }[kernel]


def hbm_bytes(kernel, l, d=D, bt=B):
    """Bytes each kernel must move once per chunk-head: its inputs read once and its
    outputs written once (workspace arrays are chunk-sized)."""
    tok = l * d * ES        # one [l, d] bf16 tensor of the chunk's rows
    blk = bt * d * ES       # one [B, d] workspace array
    sq = bt * bt * ES       # one [B, B] workspace array
    st = d * d * ES         # one bf16 state [d, d]
    return {
        "kda_prep_fwd": 4 * tok + l * ES + 5 * blk + 4 * sq + d * 4,
        "kda_state_fwd": 5 * blk + d * 4 + tok + st,
        "kda_prep_bwd": 4 * tok + l * ES + 4 * blk + 4 * sq + d * 4,
        "kda_state_bwd": 3 * blk + d * 4 + st,
        "kda_dstate": 3 * blk + d * 4 + tok + st,
        # q, k, v, g, dO, beta, S, dS, T, M, X, A in; dq, dk, dv, dg, dbeta out
        "kda_grad": 5 * tok + l * ES + 2 * st + 4 * sq + 4 * tok + l * ES,
    }[kernel]


def round_chunks(plan):
    """Chunk lengths (replay included) per round."""
    seqs = plan.sequences()
    out = {}
    for s in seqs:
        vlen = s["n_replay"] + s["row_end"] - s["row_begin"]
        lens = [min(B, vlen - c) for c in range(0, vlen, B)]
        out.setdefault(s["round"], []).extend(lens)
    return out


def path_flops(chunk_lens):
    """Dense-block algorithmic flops of forward + backward (with recompute) per head
    for all chunks: forward 4 l^2 d + 3 l d^2 + l^3/6 MAC, backward 11 l^2 d + 8 l d^2
    + 7/3 l^3 MAC."""
    tot = 0.0
    for l in chunk_lens:
        tot += (4 + 11) * l * l * D + (3 + 8) * l * D * D + (1 / 6 + 7 / 3) * l ** 3
    return 2 * tot * H


def kernel_src_hash():
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "chunkwise_linear_attention_gated_amd", "csrc", "kernels", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken
    on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except ValueError:
        return None
    if t.get("kernel_src_hash") != kernel_src_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def cpu_baseline(t, feats, C, S, target_positions=250000, seed=0):
    """The float64 oracle (trajectory-expanded, token by token, forward + reverse pass)
    on a bounded sample: whole trajectories in a seeded random order until about
    ``target_positions`` semantic positions (about 12 s on 16 cores), extrapolated per
    semantic position to the whole batch."""
    from oracle.recurrent import Trajectories, default_threads
    lens = np.diff(t.offsets)
    order = np.random.default_rng(seed).permutation(t.n_traj)
    which, P = [], 0
    for x in order:
        which.append(int(x))
        P += int(lens[x])
        if P >= target_positions:
            break
    rows = [t.node_of_pos[t.offsets[x]:t.offsets[x + 1]] for x in which]
    F = {n: getattr(feats, n) for n in ("q", "k", "v", "g", "beta", "do")}
    threads = min(default_threads(), int(os.environ.get("OMP_NUM_THREADS", "16") or 16), H * len(which))
    tr = Trajectories(rows, F["q"], F["k"], F["v"], F["g"], F["beta"])
    dO = np.concatenate([F["do"][r] for r in rows]).astype(np.float64)
    t0 = time.perf_counter()
    tr.forward(nthreads=threads)
    tr.backward(dO, nthreads=threads)
    dt = time.perf_counter() - t0
    full = dt * S / P
    return {"value": C / full, "unit": "compact tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d trajectories (%d of %d semantic positions, %d heads), forward + reverse pass in "
                      "%.1f s; extrapolated per semantic position" % (len(which), t.n_traj, P, S, H, dt)}


def conv_bench(args, out, t, plan, C):
    """The tree causal convolution of the KDA layer's q, k, v projections (3 H d = 6144 channels,
    window 4, bf16) over the benchmark tree's compact rows: forward and both gradients, timed with
    HIP events, into ``out``."""
    import torch
    import chunkwise_linear_attention_gated_amd as harts
    dev = "cuda"
    ch, w = 3 * H * D, 4
    m = np.asarray(plan.maps()[0], np.int64)
    anc, goff, gl = harts.conv_tables(m, np.asarray(t.offsets, np.int64), C, w)
    ancd, goffd, gld = (torch.from_numpy(a).to(dev) for a in (anc, goff, gl))
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    x = torch.randn((C, ch), generator=gen, device=dev).to(torch.bfloat16)
    dout = torch.randn((C, ch), generator=gen, device=dev).to(torch.bfloat16)
    wt = torch.randn((ch, w), generator=gen, device=dev) / w
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dw = torch.empty((ch, w), device=dev)
    ws = torch.empty(harts.conv_workspace_size(C, ch, w), dtype=torch.uint8, device=dev)
    reps = max(3, min(args.steps, 10))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"C": C, "channels": ch, "w": w}
    for name, fn, by in (("fwd", lambda: harts.conv_fwd(x, wt, ancd, y), 2 * C * ch * 2),
                         ("bwd", lambda: harts.conv_bwd(x, wt, ancd, goffd, gld, dout, dx=dx, dweight=dw, workspace=ws),
                          4 * C * ch * 2)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"ms": ms, "bytes": by, "achieved_gbps": by / (ms / 1e3) / 1e9, "frac_hbm": by / (ms / 1e3) / PEAK_HBM}
    out["tree_conv"] = res
    del x, dout, y, dx


def attn_bench(args, out, t, plan, C):
    """Tree softmax attention of the full-attention (MLA) layer over the benchmark tree's compact
    rows: 16 heads, q/k head dim 192 (128 + 64 rotary), v head dim 128, bf16.  Forward and
    backward timed with HIP events; algorithmic flops count only the visible (query, key) pairs:
    forward 2 (dqk + dv), backward 2 (3 dqk + 2 dv) per pair and head."""
    import torch
    import chunkwise_linear_attention_gated_amd as harts
    dev = "cuda"
    Ha, dqk, dv = 16, 192, 128
    m = np.asarray(plan.maps()[0], np.int64)
    tb = harts.attn_tables(m, np.asarray(t.offsets, np.int64), C)
    qt, kv, kt, ql = (torch.from_numpy(tb[k]).to(dev) for k in ("qtiles", "kv_list", "ktiles", "q_list"))
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    mk = lambda d: torch.randn((C, Ha, d), generator=gen, device=dev).to(torch.bfloat16)
    q, k, v, do = mk(dqk), mk(dqk), mk(dv), mk(dv)
    o = torch.empty_like(v)
    lse = torch.empty((C, Ha), device=dev)
    dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(harts.attn_workspace_size(C, Ha), dtype=torch.uint8, device=dev)
    scale = dqk ** -0.5
    pairs = tb["info"]["pairs"]
    reps = max(3, min(args.steps, 10))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"C": C, "H": Ha, "dqk": dqk, "dv": dv, "pairs_per_head": pairs, "max_depth": tb["info"]["max_depth"],
           "n_segments": tb["info"]["n_segments"]}
    for name, fn, fl in (("fwd", lambda: harts.attn_fwd(q, k, v, qt, kv, scale, o, lse), 2 * (dqk + dv)),
                         ("bwd", lambda: harts.attn_bwd(q, k, v, o, lse, do, qt, kv, kt, ql, scale, dq, dk, dvv, ws),
                          2 * (3 * dqk + 2 * dv))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = fl * pairs * Ha
        res[name] = {"ms": ms, "flops": flops, "tflops": flops / (ms / 1e3) / 1e12,
                     "frac_mfma": flops / (ms / 1e3) / PEAK_BF16}
    out["tree_attention"] = res
    del q, k, v, do, o, dq, dk, dvv


def moe_bench(args, out, plan, C):
    """Multiplicity-weighted router statistics of the benchmark tree's compact rows: 128 experts,
    top-8, fp32 router logits; statistics and the logits' gradient timed with HIP events.
    Algorithmic bytes: statistics read the logits and q and write top-k and lse (C (4E + 4 + 4k + 4));
    the gradient reads the logits and q and writes the gradient (C (8E + 4))."""
    import torch
    import chunkwise_linear_attention_gated_amd as harts
    dev = "cuda"
    E, k = 128, 8
    m = np.asarray(plan.maps()[0], np.int64)
    q = torch.from_numpy(np.bincount(m, minlength=C).astype(np.int32)).to(dev)
    S = len(m)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    z = torch.randn((C, E), generator=gen, device=dev) * 2.0
    bias = torch.randn((E,), generator=gen, device=dev) * 0.01
    top = torch.empty((C, k), dtype=torch.int32, device=dev)
    lse = torch.empty((C,), device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    mass = torch.empty((E,), device=dev)
    losses = torch.empty((2,), device=dev)
    dz = torch.empty_like(z)
    ws = torch.empty(harts.moe_workspace_size(C, E), dtype=torch.uint8, device=dev)
    reps = max(3, min(args.steps, 10))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"C": C, "S": S, "E": E, "k": k}
    for name, fn, by in (("stats", lambda: harts.moe_stats(z, q, k, S, top, lse, counts, mass, losses, ws, bias=bias),
                          C * (4 * E + 8 + 4 * k)),
                         ("grad", lambda: harts.moe_grad(z, q, counts, k, S, 1e-3, 1e-2, dz), C * (8 * E + 4))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"ms": ms, "bytes": by, "achieved_gbps": by / (ms / 1e3) / 1e9, "frac_hbm": by / (ms / 1e3) / PEAK_HBM}
    out["moe_stats"] = res


def logprob_bench(args, out):
    """The log-prob workload (32768 compact rows x 131072 bf16 logits): forward gather and its
    backward, each timed with HIP events, into ``out``."""
    import torch
    import chunkwise_linear_attention_gated_amd as harts
    from synthetic import tensors
    dev = "cuda"
    Cl, V = 32768, 131072
    w = tensors.logprob_map(Cl, V, seed=args.seed)
    logits = tensors.logits_torch(Cl, V, seed=args.seed, device=dev)
    mm = torch.from_numpy(w.m).to(dev)
    lab = torch.from_numpy(w.labels).to(dev)
    logp = torch.empty(len(w.m), dtype=torch.float32, device=dev)
    qq = torch.empty(Cl, dtype=torch.int32, device=dev)
    lws = torch.empty(harts.logprob_workspace_size(Cl), dtype=torch.uint8, device=dev)
    for _ in range(2):
        harts.logprob_gather(logits, mm, lab, logp, q=qq, workspace=lws)
    torch.cuda.synchronize()
    reps = max(3, min(args.steps, 10))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        harts.logprob_gather(logits, mm, lab, logp, q=qq, workspace=lws)
    e1.record()
    torch.cuda.synchronize()
    lms = e0.elapsed_time(e1) / reps
    lbytes = Cl * V * 2 + len(w.m) * (8 + 4 + 4 + 2) + Cl * 8
    out["logprob_gather"] = {"C": Cl, "V": V, "S": int(len(w.m)), "ms": lms, "bytes": lbytes,
                             "achieved_gbps": lbytes / (lms / 1e3) / 1e9,
                             "frac_hbm": lbytes / (lms / 1e3) / PEAK_HBM}
    # backward (equation 19): one read of the logits and one write of their gradient
    lse = torch.empty(Cl, dtype=torch.float32, device=dev)
    harts.logprob_gather(logits, mm, lab, logp, lse=lse)
    off, pos = harts.logprob_rows(w.m, Cl)
    offd, posd = torch.from_numpy(off).to(dev), torch.from_numpy(pos).to(dev)
    gl = torch.from_numpy(np.random.default_rng(args.seed).standard_normal(len(w.m)).astype(np.float32)).to(dev)
    dlog = torch.empty_like(logits)
    for _ in range(2):
        harts.logprob_backward(logits, lse, offd, posd, lab, gl, dlog)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        harts.logprob_backward(logits, lse, offd, posd, lab, gl, dlog)
    e1.record()
    torch.cuda.synchronize()
    bms = e0.elapsed_time(e1) / reps
    bbytes = 2 * Cl * V * 2 + len(w.m) * (8 + 4 + 4) + Cl * (8 + 4)
    out["logprob_backward"] = {"C": Cl, "V": V, "S": int(len(w.m)), "ms": bms, "bytes": bbytes,
                               "achieved_gbps": bbytes / (bms / 1e3) / 1e9,
                               "frac_hbm": bbytes / (bms / 1e3) / PEAK_HBM}
    del logits, dlog


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only (this build has no multi-GPU path); got --gpus %d" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    import chunkwise_linear_attention_gated_amd as harts
    from synthetic import tensors, trees

    dev = "cuda"
    if args.copy_calib:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n}))
        return

    if args.only_logprob:
        out = {}
        logprob_bench(args, out)
        print(json.dumps(out))
        return
    if args.only_moe:
        t = trees.random_rollout_tree(seed=args.seed)
        plan = harts.TreePlan(t.tokens, t.offsets, B)
        out = {}
        moe_bench(args, out, plan, plan.info.C)
        print(json.dumps(out))
        return
    if args.only_attn:
        t = trees.random_rollout_tree(seed=args.seed)
        plan = harts.TreePlan(t.tokens, t.offsets, B)
        out = {}
        attn_bench(args, out, t, plan, plan.info.C)
        print(json.dumps(out))
        return
    if args.only_conv:
        t = trees.random_rollout_tree(seed=args.seed)
        plan = harts.TreePlan(t.tokens, t.offsets, B)
        out = {}
        conv_bench(args, out, t, plan, plan.info.C)
        print(json.dumps(out))
        return

    # ---------------------------------------------------------------- workload
    t = trees.random_rollout_tree(seed=args.seed)
    feats = tensors.draw_features(t.n_nodes, H, D, D, seed=args.seed, dtype="bf16")
    t0 = time.perf_counter()
    plan = harts.TreePlan(t.tokens, t.offsets, B)
    plan_ms = (time.perf_counter() - t0) * 1e3
    info = plan.info
    C, S = info.C, info.S
    m, q_counts, _ = plan.maps()
    nodes = np.empty(C, np.int64)
    nodes[m] = t.node_of_pos
    x = {n: tensors.to_torch(getattr(feats, n)[nodes], "bf16", dev) for n in ("q", "k", "v", "g", "beta", "do")}
    dp = harts.DevicePlan(plan, H, D, D, harts.DTYPE_BF16)
    ns = max(1, info.n_slots)
    o = torch.empty((C, H, D), dtype=torch.bfloat16, device=dev)
    slots = torch.zeros((ns, H, D, D), dtype=torch.float32, device=dev)
    dslots = torch.zeros_like(slots)
    gr = {n: torch.empty_like(x[n]) for n in ("q", "k", "v", "g", "beta")}
    ws = torch.empty(dp.workspace_size(2), dtype=torch.uint8, device=dev)

    def step():
        # the forward keeps the backward's per-chunk operands and chunk-start states
        harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=slots, workspace=ws, keep=True)
        harts.kda_bwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], gr["q"], gr["k"], gr["v"],
                      gr["g"], gr["beta"], states=slots, dstates=dslots, workspace=ws, keep=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # ---------------------------------------------------------------- timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    value = C * args.steps / (ms_total / 1e3)

    # ---------------------------------------------------------------- per-kernel timing (same steps, events on)
    harts.profile_enable(True)
    for _ in range(args.steps):
        step()
    prof = harts.profile_collect()
    harts.profile_enable(False)
    rch = round_chunks(plan)
    all_chunks = [l for r in sorted(rch) for l in rch[r]]
    kernels = {}
    for name, (launches, tot_ms, units) in prof.items():
        per_step_launches = launches / args.steps
        entry = {"launches_per_step": per_step_launches, "avg_ms": tot_ms / launches,
                 "ms_per_step": tot_ms / args.steps}
        try:
            fl = 2 * sum(macs(name, l) for l in all_chunks) * H           # per step
            by = sum(hbm_bytes(name, l) for l in all_chunks) * H
            entry["flops_per_launch"] = fl / per_step_launches
            entry["bytes_per_launch"] = by / per_step_launches
            sec = entry["avg_ms"] / 1e3
            entry["tflops"] = entry["flops_per_launch"] / sec / 1e12
            entry["gbps"] = entry["bytes_per_launch"] / sec / 1e9
        except KeyError:
            pass
        kernels[name] = entry
    dom = max((k for k in kernels if "flops_per_launch" in kernels[k]), key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    intensity = dk["flops_per_launch"] / dk["bytes_per_launch"]
    if intensity < RIDGE:
        roof = {"bound": "hbm", "achieved": dk["gbps"], "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": dk["gbps"] * 1e9 / PEAK_HBM}
    else:
        roof = {"bound": "mfma", "achieved": dk["tflops"], "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": dk["tflops"] * 1e12 / PEAK_BF16}
    roof["kernel"] = dom
    roof["avg_launch_ms"] = dk["avg_ms"]
    roof["traffic"] = traffic_for(dom)

    flops_step = path_flops(all_chunks)
    bytes_step = C * H * (1282 + 2308) + 2 * 2 * info.n_slots * H * D * D * 4
    out = {
        "metric": "compact tokens/s, tree-packed chunkwise gated-delta fwd+bwd; MFMA % of peak",
        "value": value, "unit": "compact tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "64-leaf synthetic rollout tree (seed %d): 16384-token root, fan-out 2-4, "
                               "leaf lengths log-uniform [64, 4096]; H=16, d_k=d_v=128, B=64; "
                               "packed forward + backward over all rounds" % args.seed,
                   "C": C, "S": S, "expansion": S / C, "n_rounds": info.n_rounds, "n_sequences": info.n_sequences,
                   "n_slots": info.n_slots, "replay_tokens": info.replay_total, "n_chunks": info.n_chunks},
        "mfma_pct": 100 * flops_step / (ms_step / 1e3) / PEAK_BF16,
        "hbm_pct_ideal_bytes": 100 * bytes_step / (ms_step / 1e3) / PEAK_HBM,
        "path_flops_per_step": flops_step,
        "plan_ms": plan_ms,
        "wall_s_timed": wall,
        "roofline": roof,
        "kernels": kernels,
    }
    # ---------------------------------------------------------------- tree causal convolution
    if not args.no_conv:
        conv_bench(args, out, t, plan, C)
    # ---------------------------------------------------------------- tree softmax attention
    if not args.no_attn:
        attn_bench(args, out, t, plan, C)
    # ---------------------------------------------------------------- router statistics
    if not args.no_moe:
        moe_bench(args, out, plan, C)
    # ---------------------------------------------------------------- log-prob gather and its backward
    if not args.no_logprob:
        del ws
        torch.cuda.empty_cache()
        logprob_bench(args, out)
    # ---------------------------------------------------------------- oracle on the host cores
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(t, feats, C, S)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
