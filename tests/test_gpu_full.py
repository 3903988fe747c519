"""Full-size workloads on the GPU, compared element by element with the float64 oracle:

* the flat packed call: 32 independent sequences (lengths uniform in [1024, 4096], no multiple
  of 64), half of them from an fp32 N(0, 0.1^2) initial state -- every output row, every
  chunk-boundary state and every final state;
* the 64-leaf rollout tree (16384-token root, fan-out 2-4, fork offsets never chunk-aligned,
  leaf lengths log-uniform in [64, 4096]), H = 16, d = 128, B = 64, bf16: the forward's every
  compact row and handed-off state, then the backward in the benchmark's configuration
  (activations recomputed per round) -- every compact row's dq, dk, dv, dg, dbeta and the
  gradient of every handed-off state, against the trajectory-expanded reverse pass; the
  backward that reads the forward's kept operands must agree bit for bit;
* the log-prob workload: 32768 compact rows x 131072 bf16 logits, every semantic position's
  log-probability and the exact occurrence counts, and every element of the logits' gradient.

The oracle runs on the host cores (tens of seconds each on 16 cores)."""
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

from gpu_util import TOL, oracle_feats, rel_err  # noqa: E402
from test_gpu_bwd import run_tree_bwd  # noqa: E402
from test_gpu_fwd import _varlen_case, _varlen_oracle  # noqa: E402

H, D, B = 16, 128, 64


def _log(msg, t0):
    print("%-40s %6.1f s" % (msg, time.time() - t0), flush=True)


@pytest.fixture(scope="module")
def rollout():
    """Device forward + backward of the rollout tree (recompute, then keep) and the oracle's
    forward, backward and handed-off state gradients over all 64 trajectories."""
    t0 = time.time()
    t = trees.random_rollout_tree(seed=0)
    feats = tensors.draw_features(t.n_nodes, H, D, D, seed=0, dtype="bf16")
    _log("features drawn", t0)
    hp, nodes_h, got, _ = run_tree_bwd(t, feats, B, H, D, "bf16")
    kept = run_tree_bwd(t, feats, B, H, D, "bf16", keep=True)[2]
    _log("device forward + backward (recompute, keep)", t0)
    op = planner.make_plan(t.tokens, t.offsets, B)
    F = oracle_feats(feats)
    del feats
    ot = TreeOracle(op, t.offsets, t.node_of_pos, F)
    o_ref, slots_ref = ot.forward()
    _log("oracle forward", t0)
    ref = ot.backward(F["do"][ot.feat_row])
    _log("oracle backward and slot gradients", t0)
    C = hp.info.C
    pos = np.empty(C, np.int64)
    pos[nodes_h] = np.arange(C)
    return dict(got=got, kept=kept, idx=pos[ot.feat_row], o_ref=o_ref, slots_ref=slots_ref, ref=ref,
                n_slots=op.n_slots, C=C)


def _cmp(got, ref, name):
    assert np.isfinite(got).all(), name + ": non-finite or unwritten values"
    e = rel_err(got, ref)
    print("%-8s max rel err %.3e" % (name, e), flush=True)
    assert e <= TOL["bf16"], (name, e)


def test_rollout_tree_forward_full(rollout):
    r = rollout
    assert not np.isnan(r["o_ref"]).any() and not np.isnan(r["slots_ref"]).any()
    _cmp(r["got"]["o"][r["idx"]], r["o_ref"], "o")
    assert r["n_slots"] == 29
    _cmp(r["got"]["slots"], r["slots_ref"], "slots")


def test_rollout_tree_backward_full(rollout):
    r = rollout
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        _cmp(r["got"][n][r["idx"]], r["ref"][n], n)
    _cmp(r["got"]["dslots"], r["ref"]["dslots"], "dslots")


def test_rollout_tree_kept_operands_equal_recompute(rollout):
    for k, v in rollout["got"].items():
        assert np.array_equal(v, rollout["kept"][k], equal_nan=True), k


def test_flat_packed_call_full():
    t0 = time.time()
    lens = trees.flat_varlen_lengths(seed=0, n=32)
    r = _varlen_case(lens, H, D, B, "bf16", seed=0)
    _log("device flat packed call", t0)
    which = list(range(len(lens)))
    o_ref, st = _varlen_oracle(r, which, B)
    _log("oracle forward with every boundary state", t0)
    _cmp(r["o"], o_ref, "o")
    bo = r["vp"].boundary_offsets()
    nb = lens // B
    assert bo[-1] == nb.sum() == r["bst"].shape[0]
    # the oracle's captures per sequence: every multiple of B, then the final state
    k = np.concatenate([[0], np.cumsum(nb + 1)])
    ref_b = np.concatenate([st[k[i]:k[i] + nb[i]] for i in which])
    ref_f = np.stack([st[k[i] + nb[i]] for i in which])
    _cmp(r["bst"], ref_b, "boundary states")
    _cmp(r["fin"], ref_f, "final states")


def test_logprob_full_size():
    """Every semantic position of the 32768 x 131072 workload, rows taken in float64 blocks."""
    t0 = time.time()
    C, V = 32768, 131072
    w = tensors.logprob_map(C, V, seed=0)
    x = tensors.logits_torch(C, V, seed=0, device="cuda")
    m = torch.from_numpy(w.m).cuda()
    lab = torch.from_numpy(w.labels).cuda()
    logp = torch.full((len(w.m),), float("nan"), dtype=torch.float32, device="cuda")
    q = torch.full((C,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(harts.logprob_workspace_size(C), dtype=torch.uint8, device="cuda")
    harts.logprob_gather(x, m, lab, logp, q=q, workspace=ws)
    torch.cuda.synchronize()
    _log("device gather", t0)
    assert np.array_equal(q.cpu().numpy(), np.bincount(w.m, minlength=C).astype(np.int32))
    got = logp.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    order = np.argsort(w.m, kind="stable")
    starts = np.searchsorted(w.m[order], np.arange(0, C + 1, 1024))
    worst = 0.0
    for bi, r0 in enumerate(range(0, C, 1024)):
        sel = order[starts[bi]:starts[bi + 1]]
        rows = x[r0:r0 + 1024].to(device="cpu", dtype=torch.float64)
        ref = olp.logprob_rowwise(rows, w.m[sel] - r0, w.labels[sel])
        worst = max(worst, float(np.abs(got[sel] - ref).max()))
    _log("oracle over every row", t0)
    print("logp max abs err %.3e" % worst, flush=True)
    assert worst <= 1e-3
    del x


def test_logprob_backward_full_size():
    """C = 32768 rows of V = 131072 bf16 logits (the log-prob workload): the gradient of
    sum_s g_s logp_s with respect to the logits, every element of every row, against the float64
    oracle (row-wise form) in blocks of 1024 rows; the output starts as NaN."""
    t0 = time.time()
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
    dx = torch.full_like(x, float("nan"))
    harts.logprob_backward(x, lse, torch.from_numpy(off).cuda(), torch.from_numpy(pos).cuda(), lab,
                           torch.from_numpy(g).cuda(), dx)
    torch.cuda.synchronize()
    _log("device gather + backward", t0)
    order = np.argsort(w.m, kind="stable")
    starts = np.searchsorted(w.m[order], np.arange(0, C + 1, 1024))
    worst = 0.0
    for bi, r0 in enumerate(range(0, C, 1024)):
        sel = order[starts[bi]:starts[bi + 1]]
        rows = x[r0:r0 + 1024].to(device="cpu", dtype=torch.float64)
        ref = olp.logprob_backward_rowwise(rows, w.m[sel] - r0, w.labels[sel], g[sel])
        got = dx[r0:r0 + 1024].to(device="cpu", dtype=torch.float64).numpy()
        scale = np.zeros(1024)
        np.add.at(scale, w.m[sel] - r0, np.abs(g[sel].astype(np.float64)))
        err = np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 1e-6 * scale[:, None])
        assert np.isfinite(got).all()
        worst = max(worst, float(err.max()))
        assert worst <= 0.0, "rows %d..%d" % (r0, r0 + 1023)
    _log("oracle over every row", t0)
    del x, dx
