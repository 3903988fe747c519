"""GPU parity of the tree-packed chunkwise gated-delta backward (HIP, through
the C ABI): dq, dk, dv, dg, dbeta of every compact row and the gradient of
every handed-off boundary state, against the float64 trajectory-expanded
reverse pass (itself pinned by finite differences)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from oracle import planner  # noqa: E402
from oracle.recurrent import Trajectories  # noqa: E402
from oracle.tree import TreeOracle  # noqa: E402
from synthetic import tensors, trees  # noqa: E402

from gpu_util import TOL, device_inputs, harts_dtype, node_of_row, oracle_feats, rel_err, torch_dtype  # noqa: E402

NAMES = ("q", "k", "v", "g", "beta")


def run_tree_bwd(t, feats, B, H, D, dt, keep=False):
    hp = harts.TreePlan(t.tokens, t.offsets, B)
    m, q, _ = hp.maps()
    C = hp.info.C
    nodes = node_of_row(m, t.node_of_pos, C)
    x = device_inputs(feats, nodes)
    dp = harts.DevicePlan(hp, H, D, D, harts_dtype(dt))
    ns = max(1, hp.info.n_slots)
    o = torch.full((C, H, D), float("nan"), dtype=torch_dtype(dt), device="cuda")
    slots = torch.full((ns, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(dp.workspace_size(False), dp.workspace_size(True), dp.workspace_size(2)),
                     dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=slots, workspace=ws, keep=keep)
    gr = {n: torch.full_like(x[n], float("nan")) for n in NAMES}
    dslots = torch.full_like(slots, float("nan"))
    harts.kda_bwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], gr["q"], gr["k"], gr["v"], gr["g"],
                  gr["beta"], states=slots, dstates=dslots, workspace=ws, keep=keep)
    torch.cuda.synchronize()
    out = {"d" + n: gr[n].float().cpu().numpy() for n in NAMES}
    out["dslots"] = dslots[:hp.info.n_slots].cpu().numpy()
    out["o"] = o.float().cpu().numpy()
    out["slots"] = slots[:hp.info.n_slots].cpu().numpy()
    return hp, nodes, out, q


def compare_tree_bwd(t, B, H, D, dt, seed=0, keep=False):
    feats = tensors.draw_features(t.n_nodes, H, D, D, seed=seed, dtype=dt)
    hp, nodes_h, got, _ = run_tree_bwd(t, feats, B, H, D, dt, keep=keep)
    op = planner.make_plan(t.tokens, t.offsets, B)
    F = oracle_feats(feats)
    ot = TreeOracle(op, t.offsets, t.node_of_pos, F)
    ref = ot.backward(F["do"][ot.feat_row])
    C = hp.info.C
    pos_h = np.empty(C, np.int64)
    pos_h[nodes_h] = np.arange(C)
    idx = pos_h[ot.feat_row]
    errs = {}
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert not np.isnan(got[n]).any(), n + " has unwritten rows"
        errs[n] = rel_err(got[n][idx], ref[n])
    if op.n_slots:
        assert not np.isnan(got["dslots"]).any()
        errs["dslots"] = rel_err(got["dslots"], ref["dslots"])
    bad = {k: v for k, v in errs.items() if not v <= TOL[dt]}
    assert not bad, (bad, errs)
    return errs


@pytest.mark.parametrize("reading", ["G", "D"])
def test_tiny_tree_backward_fp32(reading):
    errs = compare_tree_bwd(trees.tiny_tree(reading), 16, 2, 16, "fp32")
    assert max(errs.values()) < 1e-4


def test_figure_trees_backward_bf16():
    for t in [trees.figure1_tree(), trees.figure2_tree(), trees.figureC1_tree()]:
        compare_tree_bwd(t, 64, 2, 128, "bf16", seed=5)


@pytest.mark.parametrize("B,D", [(64, 128), (64, 64), (32, 64), (32, 32)])
def test_random_trees_backward_bf16(B, D):
    rng = np.random.default_rng(31 + B + D)
    for _ in range(3):
        t = trees.random_small_tree(rng, max_segments=7, max_len=3 * B, forest=True)
        compare_tree_bwd(t, B, 3, D, "bf16", seed=int(rng.integers(1000)))


def test_narrow_heads_many_sequences_backward_bf16():
    # d = 32 with 16 heads over a forest and a tree: two slabs of a head per wave in the serial passes
    compare_tree_bwd(trees.forest_of_sequences([70, 33, 95, 64, 129], seed=4), 32, 16, 32, "bf16", seed=13)
    rng = np.random.default_rng(90)
    compare_tree_bwd(trees.random_small_tree(rng, max_segments=7, max_len=96, forest=True), 32, 16, 32, "bf16", seed=14)


def test_random_trees_backward_fp32_b32():
    rng = np.random.default_rng(77)
    for _ in range(2):
        t = trees.random_small_tree(rng, max_segments=6, max_len=90)
        compare_tree_bwd(t, 32, 2, 32, "fp32", seed=int(rng.integers(1000)))


def test_shared_slot_and_aligned_forks_backward():
    # a slot with three consumers; forks exactly on chunk boundaries (no replay)
    for t in [trees.GenTree(parent=[-1, 0, 0, 0, 0], length=[100, 30, 40, 50, 60]).finalize(seed=2),
              trees.GenTree(parent=[-1, 0, 0, 1, 1], length=[128, 64, 3, 64, 1]).finalize(seed=5)]:
        compare_tree_bwd(t, 64, 2, 128, "bf16", seed=8)


def test_varlen_backward_initial_state_gradient():
    lens = np.array([130, 64, 1, 200])
    B, H, D = 64, 2, 128
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = len(lens)
    has = np.array([0, 1, 1, 0], np.uint8)
    g = trees.forest_of_sequences(lens, seed=4)
    feats = tensors.draw_features(g.n_nodes, H, D, D, seed=4, dtype="bf16")
    init = tensors.initial_states(n, H, D, D, seed=4)
    vp = harts.VarlenPlan(cu, B, has_init=has)
    dp = harts.DevicePlan(vp, H, D, D, harts.DTYPE_BF16)
    x = device_inputs(feats, np.arange(cu[-1]))
    init_t = torch.from_numpy(init).cuda()
    o = torch.zeros((int(cu[-1]), H, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(dp.workspace_size(False), dp.workspace_size(True)), dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, init_states=init_t, workspace=ws)
    gr = {nm: torch.zeros_like(x[nm]) for nm in NAMES}
    dinit = torch.zeros((n, H, D, D), dtype=torch.float32, device="cuda")
    harts.kda_bwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], gr["q"], gr["k"], gr["v"], gr["g"],
                  gr["beta"], init_states=init_t, dinit=dinit, workspace=ws)
    torch.cuda.synchronize()
    F = oracle_feats(feats)
    S0 = np.stack([init[i] if has[i] else np.zeros_like(init[i]) for i in range(n)]).astype(np.float64)
    tr = Trajectories([np.arange(cu[i], cu[i + 1]) for i in range(n)], F["q"], F["k"], F["v"], F["g"], F["beta"],
                      S0=S0)
    ref = tr.backward(F["do"])
    for nm in NAMES:
        assert rel_err(gr[nm].float().cpu().numpy(), ref["d" + nm]) <= TOL["bf16"], nm
    assert rel_err(dinit.cpu().numpy(), ref["dS0"]) <= TOL["bf16"]


@pytest.mark.parametrize("B,D", [(64, 128), (64, 64), (32, 64), (32, 32)])
def test_kept_forward_operands_backward_bf16(B, D):
    # the forward keeps the backward's per-chunk operands and chunk-start states
    rng = np.random.default_rng(57 + B + D)
    for _ in range(3):
        t = trees.random_small_tree(rng, max_segments=7, max_len=3 * B, forest=True)
        compare_tree_bwd(t, B, 3, D, "bf16", seed=int(rng.integers(1000)), keep=True)


def test_kept_operands_equal_recompute_bitwise():
    # the kept operands are computed by the same arithmetic as the recomputed ones
    for seed, t in [(3, trees.figure2_tree()),
                    (4, trees.random_small_tree(np.random.default_rng(4), max_segments=9, max_len=300, forest=True)),
                    (5, trees.GenTree(parent=[-1, 0, 0, 0, 0], length=[100, 30, 40, 50, 60]).finalize(seed=2))]:
        feats = tensors.draw_features(t.n_nodes, 2, 128, 128, seed=seed, dtype="bf16")
        a = run_tree_bwd(t, feats, 64, 2, 128, "bf16")[2]
        b = run_tree_bwd(t, feats, 64, 2, 128, "bf16", keep=True)[2]
        for k in a:
            assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_kept_backward_needs_the_kept_workspace():
    """A backward that reads kept operands refuses a workspace no forward with keep filled, and
    one whose record a later forward without keep cleared."""
    t = trees.figure2_tree()
    feats = tensors.draw_features(t.n_nodes, 2, 128, 128, seed=1, dtype="bf16")
    hp = harts.TreePlan(t.tokens, t.offsets, 64)
    m, _, _ = hp.maps()
    C = hp.info.C
    x = device_inputs(feats, node_of_row(m, t.node_of_pos, C))
    dp = harts.DevicePlan(hp, 2, 128, 128, harts.DTYPE_BF16)
    o = torch.zeros((C, 2, 128), dtype=torch.bfloat16, device="cuda")
    slots = torch.zeros((max(1, hp.info.n_slots), 2, 128, 128), device="cuda")
    ws = torch.empty(dp.workspace_size(2), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws)
    gr = {n: torch.zeros_like(x[n]) for n in NAMES}
    dsl = torch.zeros_like(slots)

    def bwd(w):
        harts.kda_bwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], gr["q"], gr["k"], gr["v"], gr["g"],
                      gr["beta"], states=slots, dstates=dsl, workspace=w, keep=True)

    with pytest.raises(harts.HartsError):
        bwd(ws)
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=slots, workspace=ws, keep=True)
    with pytest.raises(harts.HartsError):
        bwd(ws2)
    bwd(ws)
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=slots, workspace=ws)
    with pytest.raises(harts.HartsError):
        bwd(ws)
    torch.cuda.synchronize()


def test_kept_operands_fp32_fall_back_to_recompute():
    t = trees.random_small_tree(np.random.default_rng(78), max_segments=6, max_len=90)
    errs = compare_tree_bwd(t, 32, 2, 32, "fp32", seed=3, keep=True)
    assert max(errs.values()) < 1e-4


def test_backward_repeat_runs_are_identical():
    t = trees.random_small_tree(np.random.default_rng(9), max_segments=7, max_len=200)
    feats = tensors.draw_features(t.n_nodes, 2, 128, 128, seed=2, dtype="bf16")
    a = run_tree_bwd(t, feats, 64, 2, 128, "bf16")[2]
    b = run_tree_bwd(t, feats, 64, 2, 128, "bf16")[2]
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_graph_replay_equals_eager():
    """The forward + backward step captured into a HIP graph (its work forked onto the
    library's own streams joins the capture) replays bit for bit what the eager calls
    produce, replay after replay, with eager work between the replays."""
    t = trees.random_small_tree(np.random.default_rng(31), max_segments=9, max_len=300, forest=True)
    H, D, B = 4, 128, 64
    feats = tensors.draw_features(t.n_nodes, H, D, D, seed=8, dtype="bf16")
    hp = harts.TreePlan(t.tokens, t.offsets, B)
    m, _, _ = hp.maps()
    C = hp.info.C
    x = device_inputs(feats, node_of_row(m, t.node_of_pos, C))
    dp = harts.DevicePlan(hp, H, D, D, harts.DTYPE_BF16)
    ns = max(1, hp.info.n_slots)
    o = torch.zeros((C, H, D), dtype=torch.bfloat16, device="cuda")
    slots = torch.zeros((ns, H, D, D), dtype=torch.float32, device="cuda")
    dslots = torch.zeros_like(slots)
    gr = {n: torch.zeros_like(x[n]) for n in NAMES}
    ws = torch.empty(dp.workspace_size(2), dtype=torch.uint8, device="cuda")

    def step():
        harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=slots, workspace=ws, keep=True)
        harts.kda_bwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], gr["q"], gr["k"], gr["v"], gr["g"],
                      gr["beta"], states=slots, dstates=dslots, workspace=ws, keep=True)

    n_slots = hp.info.n_slots
    outs = lambda: [o.clone(), slots[:n_slots].clone(), dslots[:n_slots].clone()] + [gr[n].clone() for n in NAMES]  # noqa: E731
    step()
    torch.cuda.synchronize()
    ref = outs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for z in [o, dslots[:n_slots]] + list(gr.values()):
            z.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs()):
            assert torch.equal(a, b), "replay %d" % r
        step()  # eager work between replays
        torch.cuda.synchronize()
