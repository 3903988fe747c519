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
    ap.add_argument("--no-flat", action="store_true", help="skip the flat packed call (32 sequences, all states)")
    ap.add_argument("--only-kda", action="store_true",
                    help="only the headline step (recompute mode) and its per-kernel table (for profiling it alone)")
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
    ap.add_argument("--save-plan", default=None,
                    help="write the workload's trajectories and its plan (maps, sequences, replay rows, "
                         "emits) to this .npz file")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain device copy of known size (for HBM counter calibration)")
    ap.add_argument("--config", type=int, choices=range(5), default=None,
                    help="only one workload: 0 the tiny tree (H=2, d=16, B=16, fp32, forward + backward), "
                         "1 the flat packed call, 2 the rollout tree forward, 3 the headline step "
                         "(as --only-kda), 4 the log-prob gather and its backward (as --only-logprob)")
    return ap.parse_args()


# ------------------------------------------------------------------ algorithmic work per kernel
# Multiply-accumulates per chunk of l tokens (replay included) and head, d = d_k = d_v, for the
# products each kernel performs (the WY chunk algebra the kernels' source comments state).  In the
# recompute mode (the headline) the forward runs kda_prep_fwd + kda_state_fwd per round and the
# backward kda_prep_bwd + kda_state_bwd (recompute) + kda_dstate + kda_grad per round.  With keep
# the forward's preparation also produces the backward's operands (kda_prep_fwd counts both) and
# the backward runs no preparation or recompute.
def macs(kernel, l, d=D, keep=False):
    l2d, ld2, l3 = l * l * d, l * d * d, l ** 3
    return {
        "kda_prep_fwd": (5 * l2d + l3 / 6) if keep else (4 * l2d + l3 / 6),
        "kda_state_fwd": 3 * ld2,
        "kda_prep_bwd": 4 * l2d + l3 / 6,
        "kda_state_bwd": 2 * ld2,
        "kda_dstate": 3 * ld2,
        "kda_grad": 9 * l2d + 5 * ld2 + 2 * l3,
    }[kernel]


# Algorithmic HBM bytes per token-head (ideal single pass over the path's own inputs and outputs,
# bf16, d = 128): forward 1282 B = q, k, v, g read (4 x 256) + beta (2) + o written (256); backward
# 2308 B = the five inputs read (1026) + dO read (256) + dq, dk, dv, dg (4 x 256) and dbeta (2)
# written.  They are attributed to the kernels that must move them: the forward preparation reads
# the inputs, the forward serial pass writes o (and the handed-off states), and the gradient
# kernel reads the inputs and dO and writes every gradient.  Recompute and state-gradient passes
# only move intermediates, which are not algorithmic bytes.
ALG_BYTES_PER_TOKEN_HEAD = {"kda_prep_fwd": 4 * D * ES + ES, "kda_state_fwd": D * ES,
                            "kda_grad": 8 * D * ES + D * ES + 2 * ES}


def alg_bytes(kernel, tokens, own_tokens, slot_bytes):
    """Algorithmic bytes of one step of ``kernel``: ``tokens`` chunk rows (replay included) and
    ``own_tokens`` compact rows, times heads; the forward serial pass also writes the handed-off
    states (``slot_bytes``)."""
    if kernel == "kda_state_fwd":
        return own_tokens * H * ALG_BYTES_PER_TOKEN_HEAD[kernel] + slot_bytes
    if kernel in ALG_BYTES_PER_TOKEN_HEAD:
        return tokens * H * ALG_BYTES_PER_TOKEN_HEAD[kernel]
    return None


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
    """SHA-256 (16 hex digits) over the sources of the KDA kernels and the headers they include:
    counters recorded in profiles/traffic.json stay valid while these bytes are unchanged."""
    h = hashlib.sha256()
    kdir = os.path.join(ROOT, "chunkwise_linear_attention_gated_amd", "csrc", "kernels")
    files = sorted(glob.glob(os.path.join(kdir, "kda_*.hip"))) + [
        os.path.join(kdir, n) for n in ("common.h", "launch.h", "state_common.h")]
    for f in files:
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


def device_features(N, seed, dev):
    """q, k (unit norm per token-head), v, g = -softplus(N(0,1)), beta = sigmoid(N(0,1)), bf16, drawn by
    torch's generator on the device (the benchmark's distributions, without the host round trip)."""
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    r = lambda *s: torch.randn(s, generator=gen, device=dev, dtype=torch.float32)
    q = torch.nn.functional.normalize(r(N, H, D), dim=-1).to(torch.bfloat16)
    k = torch.nn.functional.normalize(r(N, H, D), dim=-1).to(torch.bfloat16)
    v = r(N, H, D).to(torch.bfloat16)
    g = (-torch.nn.functional.softplus(r(N, H, D))).to(torch.bfloat16)
    beta = torch.sigmoid(r(N, H)).to(torch.bfloat16)
    return q, k, v, g, beta


def tree_forward_bench(args, fwd, timed, plan, C):
    """The rollout tree's packed forward alone (C / t_fwd): every round, o and the handed-off
    states, no backward."""
    for _ in range(2):
        fwd(False)
    ms_f, _ = timed(lambda: fwd(False), args.steps)
    ms_f /= args.steps
    rch = round_chunks(plan)
    fwd_flops = 0.0
    for r in rch:
        for l in rch[r]:
            fwd_flops += 2 * (4 * l * l * D + 3 * l * D * D + l ** 3 / 6) * H
    fwd_bytes = C * H * 1282 + plan.info.n_slots * H * D * D * 4
    return {"ms": ms_f, "value": C / (ms_f / 1e3), "unit": "compact tokens/s",
            "mfma_pct": 100 * fwd_flops / (ms_f / 1e3) / PEAK_BF16,
            "hbm_pct_alg_bytes": 100 * fwd_bytes / (ms_f / 1e3) / PEAK_HBM}


def tiny_bench(args):
    """The tiny CPU-checkable tree (reading G: 4 leaves, C = 124), H=2, d=16, B=16, fp32: one
    packed forward + backward per step.  Launch-bound at this size; reported for completeness."""
    import torch
    import chunkwise_linear_attention_gated_amd as harts
    from synthetic import tensors, trees
    t = trees.tiny_tree("G")
    Ht, Dt, Bt = 2, 16, 16
    feats = tensors.draw_features(t.n_nodes, Ht, Dt, Dt, seed=args.seed, dtype="fp32")
    hp = harts.TreePlan(t.tokens, t.offsets, Bt)
    m, _, _ = hp.maps()
    C = hp.info.C
    nodes = np.empty(C, np.int64)
    nodes[m] = t.node_of_pos
    x = {n: torch.from_numpy(np.ascontiguousarray(getattr(feats, n)[nodes])).cuda() for n in ("q", "k", "v", "g", "beta", "do")}
    dp = harts.DevicePlan(hp, Ht, Dt, Dt, harts.DTYPE_FP32)
    o = torch.empty((C, Ht, Dt), device="cuda")
    slots = torch.zeros((max(1, hp.info.n_slots), Ht, Dt, Dt), device="cuda")
    dslots = torch.zeros_like(slots)
    gr = {n: torch.empty_like(x[n]) for n in ("q", "k", "v", "g", "beta")}
    ws = torch.empty(dp.workspace_size(True), dtype=torch.uint8, device="cuda")

    def step():
        harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=slots, workspace=ws)
        harts.kda_bwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], gr["q"], gr["k"], gr["v"], gr["g"],
                      gr["beta"], states=slots, dstates=dslots, workspace=ws)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"ms_per_step": ms, "value": C / (ms / 1e3), "unit": "compact tokens/s", "C": C, "S": hp.info.S,
            "n_rounds": hp.info.n_rounds, "H": Ht, "d": Dt, "B": Bt, "dtype": "fp32"}


def flat_bench(args, out):
    """The flat packed call: 32 independent sequences (lengths uniform in [1024, 4096], multiples of
    64 rejected), even ones from the zero state and odd ones from an fp32 N(0, 0.1^2) state, one
    forward call writing o, every chunk-boundary state and the final states.  HBM-bound: algorithmic
    bytes = 1282 per token-head + initial states read + boundary and final states written."""
    import torch
    import chunkwise_linear_attention_gated_amd as harts
    from synthetic import trees
    dev = "cuda"
    lens = trees.flat_varlen_lengths(seed=args.seed, n=32)
    n = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    has = (np.arange(n) % 2 == 1).astype(np.uint8)
    vp = harts.VarlenPlan(cu, B, has_init=has, emit_boundaries=True)
    dp = harts.DevicePlan(vp, H, D, D, harts.DTYPE_BF16)
    N = int(cu[-1])
    q, k, v, g, beta = device_features(N, args.seed + 1, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 2)
    init = torch.randn((n, H, D, D), generator=gen, device=dev) * 0.1
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
    nb = vp.info.n_boundaries
    bst = torch.empty((max(nb, 1), H, D, D), dtype=torch.float32, device=dev)
    fin = torch.empty((n, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(dp.workspace_size(False), dtype=torch.uint8, device=dev)

    def call():
        harts.kda_fwd(dp, q, k, v, g, beta, o, states=bst, init_states=init, final_states=fin, workspace=ws)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    reps = max(3, min(args.steps, 10))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    st = H * D * D * 4
    by = N * H * 1282 + int(has.sum()) * st + nb * st + n * st
    chunks = [min(B, int(L) - c) for L in lens for c in range(0, int(L), B)]
    fl = sum(2 * (4 * l * l * D + 3 * l * D * D + l ** 3 / 6) * H for l in chunks)
    out["flat_varlen"] = {"n_seq": n, "tokens": N, "boundary_states": nb, "ms": ms, "value": N / (ms / 1e3),
                          "unit": "tokens/s", "alg_bytes": by, "achieved_gbps": by / (ms / 1e3) / 1e9,
                          "frac_hbm": by / (ms / 1e3) / PEAK_HBM, "mfma_pct": 100 * fl / (ms / 1e3) / PEAK_BF16}
    del q, k, v, g, beta, init, o, bst, fin, ws


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
    # algorithmic bytes: forward reads x and writes out; both gradients read dout and x once and
    # write dx (the weights and their gradient are ch * w floats)
    for name, fn, by in (("fwd", lambda: harts.conv_fwd(x, wt, ancd, y), 2 * C * ch * 2),
                         ("bwd", lambda: harts.conv_bwd(x, wt, ancd, goffd, gld, dout, dx=dx, dweight=dw, workspace=ws),
                          3 * C * ch * 2)):
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


def plan_record(t, plan):
    """The workload's trajectories and the plan built from them as plain arrays, and a SHA-256 over
    all of them: the bench line names the exact rounds it timed, and --save-plan keeps them."""
    m, q, n2r = plan.maps()
    seqs = plan.sequences()
    fields = sorted(seqs[0]) if seqs else []
    sq = np.array([[s[f] for f in fields] for s in seqs], np.int64).reshape(len(seqs), len(fields))
    eb, et = plan.emits()
    arrays = {"tokens": np.asarray(t.tokens, np.int32), "offsets": np.asarray(t.offsets, np.int64),
              "m": m, "q": q, "node_to_row": n2r, "sequences": sq,
              "sequence_fields": np.array(fields), "replay_rows": plan.replay_rows(),
              "emit_chunk": eb, "emit_slot": et}
    h = hashlib.sha256()
    for k in sorted(arrays):
        h.update(k.encode())
        h.update(np.ascontiguousarray(arrays[k]).tobytes())
    return h.hexdigest(), arrays


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

    if args.config == 3:
        args.only_kda = True
    if args.config == 4:
        args.only_logprob = True
    if args.config == 0:
        print(json.dumps({"tiny_tree": tiny_bench(args)}))
        return
    if args.config == 1:
        out = {}
        flat_bench(args, out)
        print(json.dumps(out))
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
    plan_digest, plan_arrays = plan_record(t, plan)
    if args.save_plan:
        np.savez_compressed(args.save_plan, **plan_arrays)
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

    def fwd(keep):
        harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=slots, workspace=ws, keep=keep)

    def step(keep=False):
        # recompute (keep=False): the backward prepares each round again and recomputes its
        # chunk-start states from the round's initial states; keep=True: the forward leaves the
        # backward's per-chunk operands and chunk-start states in the workspace
        fwd(keep)
        harts.kda_bwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], gr["q"], gr["k"], gr["v"],
                      gr["g"], gr["beta"], states=slots, dstates=dslots, workspace=ws, keep=keep)

    def timed(fn, steps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ev0.record()
        for _ in range(steps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1), time.perf_counter() - w0

    if args.config == 2:
        print(json.dumps({"tree_forward": tree_forward_bench(args, fwd, timed, plan, C)}))
        return
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # ---------------------------------------------------------------- timed region (headline)
    ms_total, wall = timed(step, args.steps)
    ms_step = ms_total / args.steps
    value = C * args.steps / (ms_total / 1e3)

    rch = round_chunks(plan)
    all_chunks = [l for r in sorted(rch) for l in rch[r]]
    tokens_step = sum(all_chunks)           # chunk rows per head, replay included
    slot_bytes = info.n_slots * H * D * D * 4
    flops_step = path_flops(all_chunks)
    bytes_step = C * H * (1282 + 2308) + 2 * 2 * slot_bytes

    # ---------------------------------------------------------------- per-kernel timing (same steps, events on)
    def kernel_table(keep):
        harts.profile_collect()  # drop anything recorded before
        harts.profile_enable(True)
        for _ in range(args.steps):
            step(keep)
        torch.cuda.synchronize()
        prof = harts.profile_collect()
        harts.profile_enable(False)
        kernels = {}
        for name, (launches, tot_ms, units) in prof.items():
            per_step_launches = launches / args.steps
            entry = {"launches_per_step": per_step_launches, "avg_ms": tot_ms / launches,
                     "ms_per_step": tot_ms / args.steps}
            try:
                fl = 2 * sum(macs(name, l, keep=keep) for l in all_chunks) * H           # per step
                entry["flops_per_launch"] = fl / per_step_launches
                entry["tflops"] = entry["flops_per_launch"] / (entry["avg_ms"] / 1e3) / 1e12
            except KeyError:
                pass
            by = alg_bytes(name, tokens_step, C, slot_bytes)
            if by is not None:
                entry["alg_bytes_per_launch"] = by / per_step_launches
                entry["alg_gbps"] = entry["alg_bytes_per_launch"] / (entry["avg_ms"] / 1e3) / 1e9
            kernels[name] = entry
        return kernels

    kernels = kernel_table(False)
    dom = max((k for k in kernels if "alg_bytes_per_launch" in kernels[k]), key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    intensity = dk["flops_per_launch"] / dk["alg_bytes_per_launch"]
    if intensity < RIDGE:
        roof = {"bound": "hbm", "achieved": dk["alg_gbps"], "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": dk["alg_gbps"] * 1e9 / PEAK_HBM}
    else:
        roof = {"bound": "mfma", "achieved": dk["tflops"], "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": dk["tflops"] * 1e12 / PEAK_BF16}
    roof["traffic"] = traffic_for(dom)
    roof["kernel"] = dom
    roof["avg_launch_ms"] = dk["avg_ms"]
    roof["alg_bytes_per_launch"] = dk["alg_bytes_per_launch"]
    roof["bytes_per_token_head"] = ALG_BYTES_PER_TOKEN_HEAD[dom]

    if args.only_kda:
        print(json.dumps({"ms_per_step": ms_step, "value": value, "roofline": roof, "kernels": kernels}))
        return
    # ---------------------------------------------------------------- the keep variant (same step, more memory)
    for _ in range(2):
        step(True)
    ms_keep, _ = timed(lambda: step(True), args.steps)
    keep_kernels = kernel_table(True)
    keep_variant = {"ms_per_step": ms_keep / args.steps, "value": C * args.steps / (ms_keep / 1e3),
                    "workspace_bytes": dp.workspace_size(2),
                    "mfma_pct": 100 * flops_step / (ms_keep / args.steps / 1e3) / PEAK_BF16,
                    "kernels": keep_kernels}

    # ---------------------------------------------------------------- tree forward alone (C / t_fwd)
    tree_forward = tree_forward_bench(args, fwd, timed, plan, C)

    out = {
        "metric": "compact tokens/s, tree-packed chunkwise gated-delta fwd+bwd; MFMA % of peak",
        "value": value, "unit": "compact tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "64-leaf synthetic rollout tree (seed %d): 16384-token root, fan-out 2-4, "
                               "leaf lengths log-uniform [64, 4096]; H=16, d_k=d_v=128, B=64, bf16 inputs, fp32 "
                               "state; packed forward + backward over all rounds, activations recomputed in the "
                               "backward (no operands kept between the two)" % args.seed,
                   "mode": "recompute",
                   "C": C, "S": S, "expansion": S / C, "n_rounds": info.n_rounds, "n_sequences": info.n_sequences,
                   "n_slots": info.n_slots, "replay_tokens": info.replay_total, "n_chunks": info.n_chunks,
                   "plan_sha256": plan_digest},
        "mfma_pct": 100 * flops_step / (ms_step / 1e3) / PEAK_BF16,
        "hbm_pct_alg_bytes": 100 * bytes_step / (ms_step / 1e3) / PEAK_HBM,
        "path_flops_per_step": flops_step,
        "path_alg_bytes_per_step": bytes_step,
        "plan_ms": plan_ms,
        "wall_s_timed": wall,
        "roofline": roof,
        "kernels": kernels,
        "keep_variant": keep_variant,
        "tree_forward": tree_forward,
    }
    del ws
    torch.cuda.empty_cache()
    # ---------------------------------------------------------------- flat packed call (forward, all states)
    if not args.no_flat:
        flat_bench(args, out)
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
