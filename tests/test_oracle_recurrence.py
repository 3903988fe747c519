"""Pins of the float64 recurrent oracle: closed-form special cases, an
invariant of the delta rule, the chunkwise form, central finite differences
for the hand-derived reverse pass, and tree execution with replay."""
import numpy as np
import pytest

from oracle import chunkwise, planner
from oracle.recurrent import Trajectories
from oracle.tree import TreeOracle
from synthetic import tensors, trees


def _rand(L, H, dk, dv, seed, unit=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, H, dk))
    k = rng.standard_normal((L, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((L, H, dv))
    g = -np.logaddexp(0, rng.standard_normal((L, H, dk)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((L, H))))
    return q, k, v, g, beta


def test_beta_zero_is_pure_decay():
    L, H, dk, dv = 40, 2, 8, 6
    q, k, v, g, beta = _rand(L, H, dk, dv, 1)
    beta[:] = 0.0
    S0 = np.random.default_rng(2).standard_normal((1, H, dk, dv))
    o, _ = Trajectories([np.arange(L)], q, k, v, g, beta, S0=S0).forward()
    for t in range(L):
        decay = np.exp(g[:t + 1].sum(0))  # [H, dk]
        want = np.einsum("hc,hcj,hc->hj", decay, S0[0], q[t])
        np.testing.assert_allclose(o[t], want, rtol=1e-12, atol=1e-14)


def test_full_forgetting_gives_single_outer_product():
    L, H, dk, dv = 30, 2, 8, 6
    q, k, v, g, beta = _rand(L, H, dk, dv, 3)
    g[:] = -1e4  # exp(g) == 0 exactly in float64
    o, _ = Trajectories([np.arange(L)], q, k, v, g, beta).forward()
    want = beta[..., None] * np.einsum("thc,thc->th", k, q)[..., None] * v
    np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-15)


def test_row_overwrite_memory():
    # g = 0, beta = 1, k_t = e_{j(t)}: S[j(t), :] <- v_t^T, other rows unchanged
    L, H, dk, dv = 50, 1, 8, 5
    rng = np.random.default_rng(4)
    j = rng.integers(0, dk, size=L)
    k = np.zeros((L, H, dk)); k[np.arange(L), 0, j] = 1.0
    q = rng.standard_normal((L, H, dk))
    v = rng.standard_normal((L, H, dv))
    g = np.zeros((L, H, dk)); beta = np.ones((L, H))
    o, _ = Trajectories([np.arange(L)], q, k, v, g, beta).forward()
    table = np.zeros((dk, dv))
    for t in range(L):
        table[j[t]] = v[t, 0]
        np.testing.assert_allclose(o[t, 0], table.T @ q[t, 0], rtol=1e-13, atol=1e-14)


def test_unit_key_delta_invariant():
    # for ||k_t|| = 1:  k_t^T S_t = (1 - beta_t) k_t^T S'_t + beta_t v_t^T
    L, H, dk, dv = 25, 2, 16, 16
    q, k, v, g, beta = _rand(L, H, dk, dv, 5)
    tr = Trajectories([np.arange(L)], q, k, v, g, beta)
    _, st = tr.forward(captures=[(0, t) for t in range(L + 1)])
    for t in range(L):
        Sp = np.exp(g[t])[:, :, None] * st[t]
        lhs = np.einsum("hc,hcj->hj", k[t], st[t + 1])
        rhs = (1 - beta[t])[:, None] * np.einsum("hc,hcj->hj", k[t], Sp) + beta[t][:, None] * v[t]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("L,B", [(150, 16), (37, 16), (64, 16), (5, 16), (100, 32)])
def test_chunkwise_equals_recurrent(L, B):
    H, dk, dv = 2, 16, 16
    q, k, v, g, beta = _rand(L, H, dk, dv, 10 + L)
    S0 = np.random.default_rng(L).standard_normal((1, H, dk, dv)) * 0.1
    o, st = Trajectories([np.arange(L)], q, k, v, g, beta, S0=S0).forward(
        captures=[(0, a) for a in range(B, L + 1, B)] + [(0, L)])
    O, S, states = chunkwise.run_sequence(q, k, v, g, beta, S0[0], B, boundaries=True)
    scale = np.abs(o).max()
    assert np.abs(O - o).max() <= 1e-12 * scale
    for i, s in enumerate(states):
        assert np.abs(s - st[i]).max() <= 1e-12 * np.abs(st[i]).max()
    assert np.abs(S - st[-1]).max() <= 1e-12 * np.abs(st[-1]).max()


def _loss_and_grads(q, k, v, g, beta, dO, S0):
    tr = Trajectories([np.arange(q.shape[0])], q, k, v, g, beta, S0=S0)
    o, _ = tr.forward()
    return float((o * dO).sum()), tr.backward(dO)


def test_reverse_pass_matches_central_differences():
    L, H, dk, dv = 23, 2, 6, 5
    q, k, v, g, beta = _rand(L, H, dk, dv, 21)
    S0 = np.random.default_rng(22).standard_normal((1, H, dk, dv)) * 0.3
    dO = np.random.default_rng(23).standard_normal((L, H, dv))
    _, gr = _loss_and_grads(q, k, v, g, beta, dO, S0)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S0="dS0")
    h = 1e-6
    rng = np.random.default_rng(24)
    for name, arr in args.items():
        flat = arr.reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, 120), replace=False)
        for i in idx:
            old = flat[i]
            flat[i] = old + h
            lp, _ = _loss_and_grads(**args, dO=dO)
            flat[i] = old - h
            lm, _ = _loss_and_grads(**args, dO=dO)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            an = gr[names[name]].reshape(-1)[i]
            assert abs(fd - an) <= 2e-7 * max(1.0, abs(fd)), (name, i, fd, an)


def test_lambda_capture_equals_suffix_initial_state_gradient():
    # dL/dS_a read inside a trajectory == dS0 of the suffix run from S_a
    L, H, dk, dv = 40, 2, 8, 8
    q, k, v, g, beta = _rand(L, H, dk, dv, 31)
    dO = np.random.default_rng(32).standard_normal((L, H, dv))
    a = 17
    tr = Trajectories([np.arange(L)], q, k, v, g, beta)
    _, st = tr.forward(captures=[(0, a)])
    lam = tr.backward(dO, captures=[(0, a)])["lam"][0]
    suf = Trajectories([np.arange(a, L)], q, k, v, g, beta, S0=st)
    dS0 = suf.backward(dO[a:])["dS0"][0]
    np.testing.assert_allclose(lam, dS0, rtol=1e-12, atol=1e-13)


def _tree_feats(t, H, d, seed):
    f = tensors.draw_features(t.n_nodes, H, d, d, seed=seed, dtype="fp32")
    return {n: getattr(f, n).astype(np.float64) for n in ("q", "k", "v", "g", "beta", "do")}


@pytest.mark.parametrize("reading", ["G", "D"])
def test_tree_replay_is_bitwise_trajectory_chunking(reading):
    t = trees.tiny_tree(reading)
    B = 16
    p = planner.make_plan(t.tokens, t.offsets, B)
    F = _tree_feats(t, 2, 16, 0)
    Fc = {n: F[n][TreeOracle(p, t.offsets, t.node_of_pos, F).feat_row] for n in F}
    o_tree, slots = chunkwise.run_tree_replay(p, Fc)
    per_traj = chunkwise.run_trajectories_chunked(p, Fc, t.offsets, B)
    for x, O in per_traj.items():
        assert np.array_equal(o_tree[p.m[t.offsets[x]:t.offsets[x + 1]]], O)
    # the no-replay ablation changes the floating-point path
    o_nr = chunkwise.run_tree_no_replay(p, Fc)
    assert not np.array_equal(o_nr, o_tree)
    assert np.abs(o_nr - o_tree).max() <= 1e-12 * np.abs(o_tree).max()
    # and the recurrent oracle agrees with both up to rounding
    ot = TreeOracle(p, t.offsets, t.node_of_pos, F)
    o_rec, slots_rec = ot.forward()
    assert np.abs(o_rec - o_tree).max() <= 1e-12 * np.abs(o_rec).max()
    assert np.abs(slots_rec - slots).max() <= 1e-12 * np.abs(slots_rec).max()


def test_tree_replay_bitwise_on_random_trees():
    rng = np.random.default_rng(77)
    for _ in range(12):
        t = trees.random_small_tree(rng, max_segments=7, max_len=40, forest=True)
        B = int(rng.choice([4, 8, 16]))
        p = planner.make_plan(t.tokens, t.offsets, B)
        F = _tree_feats(t, 1, 8, int(rng.integers(1000)))
        Fc = {n: F[n][TreeOracle(p, t.offsets, t.node_of_pos, F).feat_row] for n in F}
        o_tree, _ = chunkwise.run_tree_replay(p, Fc)
        for x, O in chunkwise.run_trajectories_chunked(p, Fc, t.offsets, B).items():
            assert np.array_equal(o_tree[p.m[t.offsets[x]:t.offsets[x + 1]]], O)


@pytest.mark.parametrize("reading", ["G", "D"])
def test_slot_gradients_by_finite_differences(reading):
    # perturb a handed-off state and rerun the consumer subtrees from it
    t = trees.tiny_tree(reading)
    p = planner.make_plan(t.tokens, t.offsets, 16)
    F = _tree_feats(t, 2, 16, 1)
    ot = TreeOracle(p, t.offsets, t.node_of_pos, F)
    do_c = F["do"][ot.feat_row]
    grads = ot.backward(do_c)
    _, slots = ot.forward()
    dO_pos = np.zeros((p.S, 2, 16)); dO_pos[ot.owner] = do_c
    seg = p.segments
    node_row = np.empty(p.C, dtype=np.int64); node_row[p.trie.m_node] = p.m
    rng = np.random.default_rng(9)
    for sl in range(p.n_slots):
        cons = [s for s in p.seqs if s.init_slot == sl]

        def loss(S):
            tot = 0.0
            for sp in cons:
                s_v = seg.start[sp.head]
                head_row = node_row[seg.nodes[sp.head][0]]
                for x in range(t.n_traj):
                    o0 = t.offsets[x]
                    if t.offsets[x + 1] - o0 > s_v and p.m[o0 + s_v] == head_row:
                        rows = t.node_of_pos[o0 + sp.start:t.offsets[x + 1]]
                        tr = Trajectories([rows], F["q"], F["k"], F["v"], F["g"], F["beta"], S0=S[None])
                        o, _ = tr.forward()
                        d = dO_pos[o0 + sp.start:t.offsets[x + 1]].copy()
                        d[:s_v - sp.start] = 0.0
                        tot += float((o * d).sum())
            return tot

        for _ in range(20):
            idx = tuple(int(rng.integers(n)) for n in slots.shape[1:])
            S = slots[sl].copy()
            S[idx] += 1e-6
            lp = loss(S)
            S[idx] -= 2e-6
            lm = loss(S)
            fd = (lp - lm) / 2e-6
            assert abs(fd - grads["dslots"][sl][idx]) <= 1e-7 * max(1.0, abs(fd))


def test_tree_gradients_by_finite_differences_on_compact_rows():
    t = trees.tiny_tree("G")
    p = planner.make_plan(t.tokens, t.offsets, 16)
    F = _tree_feats(t, 2, 16, 2)
    ot = TreeOracle(p, t.offsets, t.node_of_pos, F)
    do_c = F["do"][ot.feat_row]
    grads = ot.backward(do_c, slot_grads=False)

    def loss():
        o, _ = TreeOracle(p, t.offsets, t.node_of_pos, F).forward()
        return float((o * do_c).sum())

    rng = np.random.default_rng(12)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta")
    for name in names:
        for _ in range(25):
            row = int(rng.integers(p.C))
            node = ot.feat_row[row]
            idx = (node,) + tuple(int(rng.integers(n)) for n in F[name].shape[1:])
            old = F[name][idx]
            F[name][idx] = old + 1e-6
            lp = loss()
            F[name][idx] = old - 1e-6
            lm = loss()
            F[name][idx] = old
            fd = (lp - lm) / 2e-6
            an = grads[names[name]][(row,) + idx[1:]]
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, row, fd, an)
