"""Full-size workloads on the GPU, checked on outputs the oracle can compute
one trajectory at a time: the 64-leaf rollout tree (forward), the 32-sequence
flat packed call with all boundary states, and the 32768 x 131072 log-prob
gather (sampled rows, exact counts)."""
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from oracle import logprob as olp  # noqa: E402
from oracle import planner  # noqa: E402
from oracle.tree import TreeOracle  # noqa: E402
from synthetic import tensors, trees  # noqa: E402

from gpu_util import TOL, device_inputs, node_of_row, oracle_feats, rel_err  # noqa: E402
from test_gpu_fwd import _varlen_case, _varlen_oracle  # noqa: E402

H, D, B = 16, 128, 64


def test_rollout_tree_forward_sampled():
    t = trees.random_rollout_tree(seed=0)
    feats = tensors.draw_features(t.n_nodes, H, D, D, seed=0, dtype="bf16", with_do=False)
    hp = harts.TreePlan(t.tokens, t.offsets, B)
    m, _, _ = hp.maps()
    nodes = node_of_row(m, t.node_of_pos, hp.info.C)
    x = device_inputs(feats, nodes)
    dp = harts.DevicePlan(hp, H, D, D, harts.DTYPE_BF16)
    C = hp.info.C
    o = torch.full((C, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    slots = torch.zeros((hp.info.n_slots, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(dp.workspace_size(False), dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=slots, workspace=ws)
    torch.cuda.synchronize()
    o_h = o.float().cpu().numpy()
    assert not np.isnan(o_h).any()
    # oracle on the two shortest trajectories
    lens = np.diff(t.offsets)
    which = [int(i) for i in np.argsort(lens)[:2]]
    op = planner.make_plan(t.tokens, t.offsets, B)
    ot = TreeOracle(op, t.offsets, t.node_of_pos, oracle_feats(feats))
    t0 = time.time()
    o_ref, slots_ref = ot.forward(which=which)
    print("oracle %.1fs on %d tokens" % (time.time() - t0, lens[which].sum()))
    pos_h = np.empty(C, np.int64)
    pos_h[nodes] = np.arange(C)
    have = ~np.isnan(o_ref).any(axis=(1, 2))
    err = rel_err(o_h[pos_h[ot.feat_row[have]]], o_ref[have])
    print("rows checked", have.sum(), "rel err", err)
    assert err <= TOL["bf16"]
    okm = ~np.isnan(slots_ref).any(axis=(1, 2, 3))
    if okm.any():
        assert rel_err(slots.cpu().numpy()[okm], slots_ref[okm]) <= TOL["bf16"]


def test_flat_packed_call_sampled():
    lens = trees.flat_varlen_lengths(seed=0, n=32)
    r = _varlen_case(lens, H, D, B, "bf16", seed=0)
    which = [0, 1]
    o_ref, st = _varlen_oracle(r, which, B)
    cu = r["cu"]
    o_sel = np.concatenate([r["o"][cu[i]:cu[i + 1]] for i in which])
    assert rel_err(o_sel, o_ref) <= TOL["bf16"]
    bo = r["vp"].boundary_offsets()
    k = 0
    for i in which:
        nb = int(lens[i]) // B
        assert rel_err(r["bst"][bo[i]:bo[i] + nb], st[k:k + nb]) <= TOL["bf16"]
        assert rel_err(r["fin"][i], st[k + nb]) <= TOL["bf16"]
        k += nb + 1
    assert not np.isnan(r["o"]).any()


def test_logprob_full_size_sampled():
    C, V = 32768, 131072
    w = tensors.logprob_map(C, V, seed=0)
    x = tensors.logits_torch(C, V, seed=0, device="cuda")
    m = torch.from_numpy(w.m).cuda()
    lab = torch.from_numpy(w.labels).cuda()
    logp = torch.empty(len(w.m), dtype=torch.float32, device="cuda")
    q = torch.empty(C, dtype=torch.int32, device="cuda")
    ws = torch.empty(harts.logprob_workspace_size(C), dtype=torch.uint8, device="cuda")
    harts.logprob_gather(x, m, lab, logp, q=q, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), np.bincount(w.m, minlength=C).astype(np.int32))
    rows = np.random.default_rng(0).choice(C, size=64, replace=False)
    sel = np.nonzero(np.isin(w.m, rows))[0]
    xr = x[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    remap = np.full(C, -1, np.int64)
    remap[rows] = np.arange(len(rows))
    ref = olp.logprob(xr, remap[w.m[sel]], w.labels[sel])
    assert np.abs(logp.cpu().numpy()[sel] - ref).max() <= 1e-3
    del x


def test_logprob_backward_full_size_sampled():
    """C = 32768 rows of V = 131072 bf16 logits (the log-prob workload): the gradient of
    sum_s g_s logp_s with respect to the logits, checked on 32 sampled rows (every position of
    those rows) against the float64 per-position definition."""
    C, V = 32768, 131072
    w = tensors.logprob_map(C, V, seed=1)
    x = tensors.logits_torch(C, V, seed=1, device="cuda")
    g = np.random.default_rng(1).standard_normal(len(w.m)).astype(np.float32)
    m = torch.from_numpy(w.m).cuda()
    lab = torch.from_numpy(w.labels).cuda()
    lp = torch.empty(len(w.m), dtype=torch.float32, device="cuda")
    lse = torch.empty(C, dtype=torch.float32, device="cuda")
    harts.logprob_gather(x, m, lab, lp, lse=lse)
    off, pos = harts.logprob_rows(w.m, C)
    dx = torch.empty_like(x)
    harts.logprob_backward(x, lse, torch.from_numpy(off).cuda(), torch.from_numpy(pos).cuda(), lab,
                           torch.from_numpy(g).cuda(), dx)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(2).choice(C, size=32, replace=False))
    sel = np.nonzero(np.isin(w.m, rows))[0]
    remap = np.full(C, -1, np.int64)
    remap[rows] = np.arange(len(rows))
    ri = torch.from_numpy(rows).cuda()
    ref = olp.logprob_backward(x[ri].double().cpu().numpy(), remap[w.m[sel]], w.labels[sel], g[sel])
    got = dx[ri].double().cpu().numpy()
    scale = np.zeros(len(rows))
    np.add.at(scale, remap[w.m[sel]], np.abs(g[sel].astype(np.float64)))
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * scale[:, None]).all()
    del x, dx
