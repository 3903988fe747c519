"""GPU parity of the tree-packed chunkwise gated-delta forward (HIP, through
the C ABI) against the float64 trajectory-expanded oracle, plus the pages'
"same floating-point path" claim as a bitwise tree == expanded test."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from oracle import planner  # noqa: E402
from oracle.tree import TreeOracle  # noqa: E402
from synthetic import tensors, trees  # noqa: E402

from gpu_util import TOL, device_inputs, harts_dtype, node_of_row, oracle_feats, rel_err, torch_dtype  # noqa: E402


def run_tree_fwd(t, feats, B, H, D, dt):
    """Device forward of a tree: returns (plan, node_of_row, o [C,H,D] fp32 numpy, slots)."""
    hp = harts.TreePlan(t.tokens, t.offsets, B)
    m, q, _ = hp.maps()
    nodes = node_of_row(m, t.node_of_pos, hp.info.C)
    x = device_inputs(feats, nodes)
    dp = harts.DevicePlan(hp, H, D, D, harts_dtype(dt))
    C = hp.info.C
    o = torch.full((C, H, D), float("nan"), dtype=torch_dtype(dt), device="cuda")
    slots = torch.zeros((max(1, hp.info.n_slots), H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(dp.workspace_size(False), dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=slots, workspace=ws)
    torch.cuda.synchronize()
    return hp, nodes, o.float().cpu().numpy(), slots[:hp.info.n_slots].cpu().numpy()


def oracle_tree_fwd(t, feats, B, which=None):
    op = planner.make_plan(t.tokens, t.offsets, B)
    ot = TreeOracle(op, t.offsets, t.node_of_pos, oracle_feats(feats))
    o, slots = ot.forward(which=which)
    return op, ot, o, slots


def compare_tree_fwd(t, B, H, D, dt, seed=0, which=None):
    feats = tensors.draw_features(t.n_nodes, H, D, D, seed=seed, dtype=dt, with_do=False)
    hp, nodes_h, o_h, slots_h = run_tree_fwd(t, feats, B, H, D, dt)
    op, ot, o_ref, slots_ref = oracle_tree_fwd(t, feats, B, which=which)
    nodes_o = ot.feat_row
    # align by generator node
    pos_h = np.empty(len(nodes_h), np.int64)
    pos_h[nodes_h] = np.arange(len(nodes_h))
    o_h_al = o_h[pos_h[nodes_o]]
    have = ~np.isnan(o_ref).any(axis=(1, 2))
    assert have.sum() > 0
    assert not np.isnan(o_h).any(), "rows left unwritten"
    err = rel_err(o_h_al[have], o_ref[have])
    assert err <= TOL[dt], ("o", err)
    # slots: both planners number slots in first-use order over identical sequence orders
    okm = ~np.isnan(slots_ref).any(axis=(1, 2, 3))
    if okm.any():
        e2 = rel_err(slots_h[okm], slots_ref[okm])
        assert e2 <= TOL[dt], ("slots", e2)
    return err


@pytest.mark.parametrize("reading", ["G", "D"])
def test_tiny_tree_fp32(reading):
    t = trees.tiny_tree(reading)
    err = compare_tree_fwd(t, 16, 2, 16, "fp32")
    assert err < 1e-4


def test_figure_trees_bf16():
    for t in [trees.figure1_tree(), trees.figure2_tree(), trees.figureC1_tree()]:
        compare_tree_fwd(t, 64, 2, 128, "bf16", seed=3)


@pytest.mark.parametrize("B,D", [(64, 128), (64, 64), (32, 64), (32, 32)])
def test_random_trees_bf16(B, D):
    rng = np.random.default_rng(11 + B + D)
    for _ in range(3):
        t = trees.random_small_tree(rng, max_segments=7, max_len=3 * B, forest=True)
        compare_tree_fwd(t, B, 3, D, "bf16", seed=int(rng.integers(1000)))


def test_narrow_heads_many_sequences_bf16():
    # d = 32 with 16 heads over a forest: enough (sequence, head) pairs per round that each
    # workgroup of the serial pass runs both 16-column slabs of a head on one wave
    t = trees.forest_of_sequences([70, 33, 95, 64, 129], seed=4)
    compare_tree_fwd(t, 32, 16, 32, "bf16", seed=12)


def test_fp32_b32():
    rng = np.random.default_rng(5)
    t = trees.random_small_tree(rng, max_segments=6, max_len=100)
    compare_tree_fwd(t, 32, 2, 32, "fp32", seed=9)


def _expanded_fwd(t, feats, B, H, D, dt):
    """Every trajectory as an independent sequence of one packed call."""
    lens = np.diff(t.offsets)
    vp = harts.VarlenPlan(t.offsets, B)
    x = device_inputs(feats, t.node_of_pos)
    dp = harts.DevicePlan(vp, H, D, D, harts_dtype(dt))
    o = torch.zeros((int(t.offsets[-1]), H, D), dtype=torch_dtype(dt), device="cuda")
    ws = torch.empty(dp.workspace_size(False), dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, workspace=ws)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


@pytest.mark.parametrize("dt,B,D", [("bf16", 64, 128), ("fp32", 16, 16)])
def test_tree_equals_expanded_bitwise(dt, B, D):
    """Replay keeps every chunk identical to trajectory-wise chunking, so the
    tree execution reproduces the expanded execution bit for bit."""
    rng = np.random.default_rng(21)
    for _ in range(4):
        t = trees.random_small_tree(rng, max_segments=7, max_len=3 * B)
        H = 2
        feats = tensors.draw_features(t.n_nodes, H, D, D, seed=int(rng.integers(1000)), dtype=dt, with_do=False)
        hp, nodes_h, o_tree, _ = run_tree_fwd(t, feats, B, H, D, dt)
        o_exp = _expanded_fwd(t, feats, B, H, D, dt)
        m, _, _ = hp.maps()
        assert np.array_equal(o_tree[m], o_exp)


def test_no_replay_changes_the_floating_point_path():
    """Negative control: starting a side branch from its parent's exact state
    at the fork (chunks counted from the fork) is close but not bitwise equal."""
    t = trees.GenTree(parent=[-1, 0, 0], length=[100, 90, 70]).finalize(seed=3)
    B, H, D, dt = 64, 2, 128, "bf16"
    feats = tensors.draw_features(t.n_nodes, H, D, D, seed=4, dtype=dt, with_do=False)
    hp, nodes_h, o_tree, _ = run_tree_fwd(t, feats, B, H, D, dt)
    # side branch = the child whose rows were not in round 1
    seqs = hp.sequences()
    side = [s for s in seqs if s["round"] == 2][0]
    side_nodes = nodes_h[side["row_begin"]:side["row_end"]]
    prefix_nodes = np.arange(0, 100)  # segment 0 is generator nodes [0, 100)
    # prefix run -> exact final state at the fork
    vp = harts.VarlenPlan(np.array([0, 100]), B)
    dp = harts.DevicePlan(vp, H, D, D, harts.DTYPE_BF16)
    x = device_inputs(feats, prefix_nodes)
    fin = torch.zeros((1, H, D, D), dtype=torch.float32, device="cuda")
    o = torch.zeros((100, H, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(dp.workspace_size(False), dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, final_states=fin, workspace=ws)
    L = len(side_nodes)
    vp2 = harts.VarlenPlan(np.array([0, L]), B, has_init=np.array([1], np.uint8))
    dp2 = harts.DevicePlan(vp2, H, D, D, harts.DTYPE_BF16)
    x2 = device_inputs(feats, side_nodes)
    o2 = torch.zeros((L, H, D), dtype=torch.bfloat16, device="cuda")
    ws2 = torch.empty(dp2.workspace_size(False), dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp2, x2["q"], x2["k"], x2["v"], x2["g"], x2["beta"], o2, init_states=fin, workspace=ws2)
    torch.cuda.synchronize()
    a = o_tree[side["row_begin"]:side["row_end"]]
    b = o2.float().cpu().numpy()
    assert not np.array_equal(a, b)
    assert rel_err(b, a) < 5e-2


def test_repeat_runs_are_identical():
    t = trees.random_small_tree(np.random.default_rng(8), max_segments=7, max_len=200)
    feats = tensors.draw_features(t.n_nodes, 2, 128, 128, seed=1, dtype="bf16", with_do=False)
    r1 = run_tree_fwd(t, feats, 64, 2, 128, "bf16")
    r2 = run_tree_fwd(t, feats, 64, 2, 128, "bf16")
    assert np.array_equal(r1[2], r2[2]) and np.array_equal(r1[3], r2[3])


def _varlen_case(lens, H, D, B, dt, seed, emit=True):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = len(lens)
    has = (np.arange(n) % 2 == 1).astype(np.uint8)
    g = trees.forest_of_sequences(lens, seed=seed)
    feats = tensors.draw_features(g.n_nodes, H, D, D, seed=seed, dtype=dt, with_do=False)
    init = tensors.initial_states(n, H, D, D, seed=seed)
    vp = harts.VarlenPlan(cu, B, has_init=has, emit_boundaries=emit)
    dp = harts.DevicePlan(vp, H, D, D, harts_dtype(dt))
    x = device_inputs(feats, np.arange(cu[-1]))
    N = int(cu[-1])
    o = torch.full((N, H, D), float("nan"), dtype=torch_dtype(dt), device="cuda")
    nb = vp.info.n_boundaries
    bst = torch.full((max(nb, 1), H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    fin = torch.full((n, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    init_t = torch.from_numpy(init).cuda()
    ws = torch.empty(dp.workspace_size(False), dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, states=bst if emit else None,
                  init_states=init_t, final_states=fin, workspace=ws)
    torch.cuda.synchronize()
    return dict(cu=cu, has=has, feats=feats, init=init, vp=vp, o=o.float().cpu().numpy(),
                bst=bst[:nb].cpu().numpy(), fin=fin.cpu().numpy())


def _varlen_oracle(r, which, B):
    from oracle.recurrent import Trajectories
    cu, has, init = r["cu"], r["has"], r["init"]
    F = oracle_feats(r["feats"])
    S0 = np.stack([init[i] if has[i] else np.zeros_like(init[i]) for i in which]).astype(np.float64)
    rows = [np.arange(cu[i], cu[i + 1]) for i in which]
    tr = Trajectories(rows, F["q"], F["k"], F["v"], F["g"], F["beta"], S0=S0)
    caps = []
    for j, i in enumerate(which):
        L = int(cu[i + 1] - cu[i])
        caps += [(j, a) for a in range(B, L + 1, B)] + [(j, L)]
    return tr.forward(captures=caps)


def test_varlen_small_bf16():
    lens = np.array([130, 64, 1, 257, 300, 75])
    B, H, D = 64, 2, 128
    r = _varlen_case(lens, H, D, B, "bf16", seed=2)
    which = list(range(len(lens)))
    o_ref, st = _varlen_oracle(r, which, B)
    assert rel_err(r["o"], o_ref) <= TOL["bf16"]
    bo = r["vp"].boundary_offsets()
    k = 0
    for i in which:
        L = int(lens[i])
        nb = L // B
        got = r["bst"][bo[i]:bo[i] + nb]
        ref = st[k:k + nb]
        if nb:
            assert rel_err(got, ref) <= TOL["bf16"]
        assert rel_err(r["fin"][i], st[k + nb]) <= TOL["bf16"]
        k += nb + 1


@pytest.mark.parametrize("dt,B,D,mask", [("bf16", 64, 128, "alternate"), ("bf16", 32, 64, "all"),
                                         ("fp32", 16, 16, "none")])
def test_kda_fwd_varlen_one_call_equals_the_planned_call(dt, B, D, mask):
    """harts_kda_fwd_varlen (plan, upload, workspace and forward in one call) writes the same
    bytes as harts_plan_create_varlen + harts_plan_upload + harts_kda_fwd, and both match the
    oracle."""
    lens = np.array([3 * B + 5, B, 1, 2 * B, 7])
    H, n = 2, len(lens)
    r = _varlen_case(lens, H, D, B, dt, seed=5)
    cu, init = r["cu"], r["init"]
    feats = r["feats"]
    x = device_inputs(feats, np.arange(cu[-1]))
    init_t = torch.from_numpy(init).cuda()
    if mask == "alternate":
        init_mask, has = r["has"], r["has"]
    elif mask == "all":
        init_mask, has = None, np.ones(n, np.uint8)
    else:
        init_mask, has, init_t = None, np.zeros(n, np.uint8), None
    vp = harts.VarlenPlan(cu, B, has_init=has if init_t is not None else None, emit_boundaries=True)
    dp = harts.DevicePlan(vp, H, D, D, harts_dtype(dt))
    N, nb = int(cu[-1]), vp.info.n_boundaries

    def bufs():
        return (torch.full((N, H, D), float("nan"), dtype=torch_dtype(dt), device="cuda"),
                torch.full((nb, H, D, D), float("nan"), dtype=torch.float32, device="cuda"),
                torch.full((n, H, D, D), float("nan"), dtype=torch.float32, device="cuda"))

    o1, b1, f1 = bufs()
    ws = torch.empty(dp.workspace_size(False), dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o1, states=b1, init_states=init_t,
                  final_states=f1, workspace=ws)
    o2, b2, f2 = bufs()
    offs = harts.kda_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, o2, B, init_states=init_t,
                                init_mask=init_mask, boundary_states=b2, final_states=f2)
    torch.cuda.synchronize()
    assert np.array_equal(offs, vp.boundary_offsets())
    for a, b in ((o1, o2), (b1, b2), (f1, f2)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    # the one-call result against the oracle
    which = list(range(n))
    r2 = dict(r, has=has)
    o_ref, st = _varlen_oracle(r2, which, B)
    assert rel_err(o2.float().cpu().numpy(), o_ref) <= TOL[dt]
    k = 0
    for i in which:
        m = int(lens[i]) // B
        if m:
            assert rel_err(b2[offs[i]:offs[i] + m].cpu().numpy(), st[k:k + m]) <= TOL[dt]
        assert rel_err(f2[i].cpu().numpy(), st[k + m]) <= TOL[dt]
        k += m + 1
