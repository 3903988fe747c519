"""GPU parity of the gated delta rule's special cases and extreme gates, forward and backward,
fp32 and bf16, against the float64 trajectory-expanded oracle (through the C ABI):

* beta = 0: no write, the state only decays;
* g = -1e4 (e^g = 0 in every precision): the state is one outer product, o_t = beta_t (k_t . q_t) v_t;
* g = 0, beta = 1, one-hot keys: a row-overwrite memory;
* gates steep enough that a 16-token block's log-decay passes -60 (the kernels then sum those
  channels' diagonal-block terms pairwise) or lies far beyond fp32's exponent range, and a mix of
  gentle and steep channels in one head.

The recurrence (equation (1) as the close-reading blog cites it, section 7.1) is defined for any
log-decay g <= 0, so every output element must be finite and within the tolerance."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from oracle import planner  # noqa: E402
from oracle.recurrent import Trajectories  # noqa: E402
from oracle.tree import TreeOracle  # noqa: E402
from synthetic import tensors, trees  # noqa: E402

from gpu_util import TOL, device_inputs, harts_dtype, oracle_feats, rel_err, torch_dtype  # noqa: E402
from test_gpu_bwd import run_tree_bwd  # noqa: E402
from test_gpu_fwd import _expanded_fwd, run_tree_fwd  # noqa: E402

KINDS = ["beta0", "gneg", "overwrite", "steep3", "steep5", "mixed"]
CONFIGS = [("fp32", 16, 16), ("fp32", 32, 32), ("bf16", 64, 128), ("bf16", 64, 64), ("bf16", 32, 64), ("bf16", 32, 32)]


def _rnd(x, dt):
    return tensors.round_bf16(x) if dt == "bf16" else np.asarray(x, dtype=np.float32)


def _softplus(x):
    return np.logaddexp(0.0, x)


def edge_features(n_nodes, H, D, dt, seed, kind):
    """The seeded features with the special case's tensors replaced (rounded to ``dt``)."""
    f = tensors.draw_features(n_nodes, H, D, D, seed=seed, dtype=dt)
    rng = np.random.default_rng(np.random.PCG64([seed, 0xED6E]))
    if kind == "beta0":
        f.beta = np.zeros_like(f.beta)
    elif kind == "gneg":
        f.g = _rnd(np.full(f.g.shape, -1e4), dt)
    elif kind == "overwrite":
        f.g = np.zeros_like(f.g)
        f.beta = np.ones_like(f.beta)
        k = np.zeros_like(f.k)
        j = rng.integers(0, D, size=(n_nodes, H))
        k[np.arange(n_nodes)[:, None], np.arange(H)[None, :], j] = 1.0
        f.k = k
    elif kind == "steep3":
        f.g = _rnd(-_softplus(rng.normal(3.0, 1.0, f.g.shape)), dt)
    elif kind == "steep5":
        f.g = _rnd(-_softplus(rng.normal(5.0, 1.0, f.g.shape)), dt)
    elif kind == "mixed":
        # per (head, channel) gate scale log-uniform over [0.05, 200]: gentle and steep channels side by side
        s = np.exp(rng.uniform(np.log(0.05), np.log(200.0), size=(1, H, D)))
        f.g = _rnd(-_softplus(rng.normal(0.0, 1.0, f.g.shape)) * s, dt)
    else:
        raise ValueError(kind)
    return f


def _tree(dt, B, seed):
    if B == 16:
        return trees.tiny_tree("G")
    rng = np.random.default_rng(seed)
    return trees.random_small_tree(rng, max_segments=6, max_len=3 * B, forest=True)


def _check(got, ref, dt, name):
    assert np.isfinite(got).all(), name + ": non-finite values"
    e = rel_err(got, ref)
    print("  %-26s %.3e" % (name, e))
    assert e <= TOL[dt], (name, e)
    return e


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dt,B,D", CONFIGS)
def test_special_case_forward_backward(kind, dt, B, D):
    H = 2
    seed = 100 + 7 * KINDS.index(kind) + B + D
    t = _tree(dt, B, seed)
    feats = edge_features(t.n_nodes, H, D, dt, seed, kind)
    hp, nodes_h, got, _ = run_tree_bwd(t, feats, B, H, D, dt)
    op = planner.make_plan(t.tokens, t.offsets, B)
    F = oracle_feats(feats)
    ot = TreeOracle(op, t.offsets, t.node_of_pos, F)
    o_ref, slots_ref = ot.forward()
    ref = ot.backward(F["do"][ot.feat_row])
    C = hp.info.C
    pos = np.empty(C, np.int64)
    pos[nodes_h] = np.arange(C)
    idx = pos[ot.feat_row]
    _check(got["o"][idx], o_ref, dt, "o")
    if op.n_slots:
        _check(got["slots"], slots_ref, dt, "slots")
        _check(got["dslots"], ref["dslots"], dt, "dslots")
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        _check(got[n][idx], ref[n], dt, n)
    if kind == "gneg":
        # closed form, independent of the oracle: S_t = beta_t k_t v_t^T, o_t = beta_t (k_t . q_t) v_t
        row = ot.feat_row
        q, k, v, b = (F[n][row] for n in ("q", "k", "v", "beta"))
        o_cf = b[:, :, None] * (k * q).sum(-1)[:, :, None] * v
        _check(got["o"][idx], o_cf, dt, "o (closed form)")


@pytest.mark.parametrize("kind", ["steep5", "mixed", "gneg"])
def test_steep_gates_tree_equals_expanded_bitwise(kind):
    """The pairwise diagonal path depends only on the chunk's own gates, so the tree execution
    still reproduces the expanded execution bit for bit."""
    B, D, H, dt = 64, 128, 2, "bf16"
    rng = np.random.default_rng(71)
    for _ in range(2):
        t = trees.random_small_tree(rng, max_segments=7, max_len=3 * B)
        feats = edge_features(t.n_nodes, H, D, dt, int(rng.integers(1000)), kind)
        feats.do = None
        hp, _, o_tree, _ = run_tree_fwd(t, feats, B, H, D, dt)
        o_exp = _expanded_fwd(t, feats, B, H, D, dt)
        m, _, _ = hp.maps()
        assert np.isfinite(o_tree).all()
        assert np.array_equal(o_tree[m], o_exp)


@pytest.mark.parametrize("dt,B,D", [("fp32", 32, 32), ("bf16", 64, 128)])
def test_beta0_decays_initial_states(dt, B, D):
    """beta = 0 from nonzero initial states (flat packed call): o_t = (prod_{i<=t} diag(e^{g_i}) S0)^T q_t,
    the final state the decayed S0; the initial-state gradient against the oracle."""
    lens = np.array([2 * B + 5, B, 3, B + 17])
    H = 2
    n = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    g = trees.forest_of_sequences(lens, seed=3)
    feats = edge_features(g.n_nodes, H, D, dt, 3, "beta0")
    init = tensors.initial_states(n, H, D, D, seed=3, std=1.0)
    has = np.ones(n, np.uint8)
    vp = harts.VarlenPlan(cu, B, has_init=has)
    dp = harts.DevicePlan(vp, H, D, D, harts_dtype(dt))
    x = device_inputs(feats, np.arange(cu[-1]))
    N = int(cu[-1])
    o = torch.full((N, H, D), float("nan"), dtype=torch_dtype(dt), device="cuda")
    fin = torch.zeros((n, H, D, D), dtype=torch.float32, device="cuda")
    init_t = torch.from_numpy(init).cuda()
    ws = torch.empty(max(dp.workspace_size(False), dp.workspace_size(True)), dtype=torch.uint8, device="cuda")
    harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, init_states=init_t, final_states=fin, workspace=ws)
    gr = {nm: torch.full_like(x[nm], float("nan")) for nm in ("q", "k", "v", "g", "beta")}
    dinit = torch.zeros((n, H, D, D), dtype=torch.float32, device="cuda")
    harts.kda_bwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], gr["q"], gr["k"], gr["v"], gr["g"],
                  gr["beta"], init_states=init_t, dinit=dinit, workspace=ws)
    torch.cuda.synchronize()
    F = oracle_feats(feats)
    # closed form
    o_cf = np.empty((N, H, D))
    fin_cf = np.empty((n, H, D, D))
    for i in range(n):
        S = init[i].astype(np.float64)
        for t_ in range(cu[i], cu[i + 1]):
            S = np.exp(F["g"][t_])[:, :, None] * S
            o_cf[t_] = np.einsum("hkv,hk->hv", S, F["q"][t_])
        fin_cf[i] = S
    _check(o.float().cpu().numpy(), o_cf, dt, "o (closed form)")
    _check(fin.cpu().numpy(), fin_cf, dt, "final state (closed form)")
    tr = Trajectories([np.arange(cu[i], cu[i + 1]) for i in range(n)], F["q"], F["k"], F["v"], F["g"], F["beta"],
                      S0=init.astype(np.float64))
    ref = tr.backward(F["do"])
    for nm in ("q", "k", "v", "g", "beta"):
        _check(gr[nm].float().cpu().numpy(), ref["d" + nm], dt, "d" + nm)
    _check(dinit.cpu().numpy(), ref["dS0"], dt, "dS0")


def test_nan_in_one_sequence_stays_in_that_sequence():
    """Inputs are not checked for NaN: a NaN value in one sequence of a packed call reaches that
    sequence's outputs and final state, and every other sequence (forward and backward) is bit for
    bit what it is without it."""
    B, D, H, dt = 64, 128, 2, "bf16"
    lens = np.array([150, 200, 90])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    g = trees.forest_of_sequences(lens, seed=5)
    feats = tensors.draw_features(g.n_nodes, H, D, D, seed=5, dtype=dt)
    vp = harts.VarlenPlan(cu, B)
    dp = harts.DevicePlan(vp, H, D, D, harts_dtype(dt))
    ws = torch.empty(max(dp.workspace_size(False), dp.workspace_size(True)), dtype=torch.uint8, device="cuda")

    def run(poison):
        x = device_inputs(feats, np.arange(cu[-1]))
        if poison:
            x["v"][cu[1] + 70, 1, 5] = float("nan")
        N = int(cu[-1])
        o = torch.full((N, H, D), 7.0, dtype=torch_dtype(dt), device="cuda")
        fin = torch.zeros((len(lens), H, D, D), device="cuda")
        harts.kda_fwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], o, final_states=fin, workspace=ws)
        gr = {n: torch.zeros_like(x[n]) for n in ("q", "k", "v", "g", "beta")}
        harts.kda_bwd(dp, x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], gr["q"], gr["k"], gr["v"], gr["g"],
                      gr["beta"], workspace=ws)
        torch.cuda.synchronize()
        out = {"o": o.float().cpu().numpy(), "fin": fin.cpu().numpy()}
        out.update({n: t.float().cpu().numpy() for n, t in gr.items()})
        return out

    clean, bad = run(False), run(True)
    other = np.r_[cu[0]:cu[1], cu[2]:cu[3]]
    for n in ("o", "q", "k", "v", "g", "beta"):
        assert np.array_equal(clean[n][other], bad[n][other]), n
    assert np.array_equal(clean["fin"][[0, 2]], bad["fin"][[0, 2]])
    assert np.isnan(bad["o"][cu[1] + 70:cu[2]]).any() and np.isnan(bad["fin"][1]).any()
    assert np.isfinite(clean["o"]).all() and np.isfinite(clean["fin"]).all()


@pytest.mark.parametrize("kind", ["steep5", "mixed", "gneg", "beta0"])
def test_kept_operands_equal_recompute_under_special_gates(kind):
    """The forward that keeps its operands for the backward (preparation in both modes at once)
    and the backward that recomputes them take the same steep-row and diagonal-block decisions:
    every output and gradient agrees bit for bit."""
    B, D, H, dt = 64, 128, 2, "bf16"
    rng = np.random.default_rng(83)
    t = trees.random_small_tree(rng, max_segments=7, max_len=3 * B)
    feats = edge_features(t.n_nodes, H, D, dt, int(rng.integers(1000)), kind)
    a = run_tree_bwd(t, feats, B, H, D, dt)[2]
    b = run_tree_bwd(t, feats, B, H, D, dt, keep=True)[2]
    for n in a:
        assert np.isfinite(a[n]).all(), n
        assert np.array_equal(a[n], b[n]), n
