"""Pins of the float64 tree-attention oracle: a single trajectory against the library's
causal attention, a tree against the same library routine run on every expanded
trajectory (forward, and backward through autograd with each compact row counted once),
a closed form, and central finite differences."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as att


def _tree():
    # trajectories [a b c d e] [a b c f] [a b g h i j] [a b c d]; rows a..j = 0..9
    m = np.array([0, 1, 2, 3, 4, 0, 1, 2, 5, 0, 1, 6, 7, 8, 9, 0, 1, 2, 3])
    off = np.array([0, 5, 9, 15, 19])
    return m, off, 10


def _inputs(C, H, dqk, dv, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((C, H, dqk)), rng.standard_normal((C, H, dqk)), rng.standard_normal((C, H, dv)))


def _sdpa(q, k, v, scale):
    # [L, H, d] -> library causal attention over the L positions, float64
    t = lambda x: x.permute(1, 0, 2).unsqueeze(0)
    return F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=scale)[0].permute(1, 0, 2)


def test_single_trajectory_is_causal_attention():
    L, H, dqk, dv, scale = 11, 2, 6, 5, 0.37
    q, k, v = _inputs(L, H, dqk, dv, 0)
    o, lse = att.attention_forward(q, k, v, np.arange(L), np.array([0, L]), scale)
    ref = _sdpa(*(torch.from_numpy(x) for x in (q, k, v)), scale).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    s = scale * torch.einsum("ihd,jhd->hij", torch.from_numpy(q), torch.from_numpy(k))
    s = s.masked_fill(~torch.ones(L, L, dtype=torch.bool).tril(), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).T.numpy(), rtol=0, atol=1e-12)


def test_tree_rows_equal_every_expanded_trajectory():
    m, off, C = _tree()
    q, k, v = _inputs(C, 3, 8, 4, 1)
    o, _ = att.attention_forward(q, k, v, m, off, 0.5)
    for tr in range(len(off) - 1):
        rows = m[off[tr]:off[tr + 1]]
        ref = _sdpa(*(torch.from_numpy(x[rows]) for x in (q, k, v)), 0.5).numpy()
        np.testing.assert_allclose(o[rows], ref, rtol=0, atol=1e-12)


def test_backward_equals_autograd_of_the_expanded_trajectories():
    m, off, C = _tree()
    H, dqk, dv, scale = 2, 5, 3, 0.8
    q, k, v = _inputs(C, H, dqk, dv, 2)
    dout = np.random.default_rng(3).standard_normal((C, H, dv))
    dq, dk, dvv = att.attention_backward(q, k, v, dout, m, off, scale)
    # each compact row's output is reached by q_c semantic positions; weighting each position
    # by 1/q_c makes the expanded loss equal sum_t <dout[t], o[t]>
    qc = np.bincount(m, minlength=C).astype(np.float64)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    loss = 0
    for tr in range(len(off) - 1):
        rows = torch.from_numpy(m[off[tr]:off[tr + 1]])
        o = _sdpa(tq[rows], tk[rows], tv[rows], scale)
        w = torch.from_numpy(dout)[rows] / torch.from_numpy(qc)[rows][:, None, None]
        loss = loss + (o * w).sum()
    loss.backward()
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dvv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-11)


def test_constant_scores_average_the_path_values():
    m, off, C = _tree()
    _, _, v = _inputs(C, 1, 4, 3, 4)
    q = np.zeros((C, 1, 4))
    k = np.random.default_rng(5).standard_normal((C, 1, 4))
    o, lse = att.attention_forward(q, k, v, m, off, 1.0)
    P = att.paths(m, off, C)
    for t in range(C):
        np.testing.assert_allclose(o[t, 0], v[P[t], 0].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[t, 0] - np.log(len(P[t]))) < 1e-13
    # the path of row j (= 9) is a b g h i j
    assert list(P[9]) == [0, 1, 6, 7, 8, 9]


def test_finite_differences():
    m, off, C = _tree()
    H, dqk, dv, scale = 1, 3, 2, 0.6
    q, k, v = _inputs(C, H, dqk, dv, 6)
    dout = np.random.default_rng(7).standard_normal((C, H, dv))
    grads = att.attention_backward(q, k, v, dout, m, off, scale)
    loss = lambda q_, k_, v_: float((att.attention_forward(q_, k_, v_, m, off, scale)[0] * dout).sum())
    eps = 1e-6
    rng = np.random.default_rng(8)
    for which in range(3):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in (q, k, v)[which].shape)
            xs = [x.copy() for x in (q, k, v)]
            xs[which][idx] += eps
            up = loss(*xs)
            xs[which][idx] -= 2 * eps
            dn = loss(*xs)
            assert abs((up - dn) / (2 * eps) - grads[which][idx]) < 1e-7


def test_rejects_a_row_with_two_prefixes():
    with pytest.raises(ValueError):
        att.paths(np.array([0, 1, 2, 1]), np.array([0, 2, 4]), 3)
    with pytest.raises(ValueError):
        att.paths(np.array([0, 1]), np.array([0, 2]), 3)


def test_row_terms_assemble_the_library_gradients():
    m, off, C = _tree()
    H, dqk, dv, scale = 2, 4, 3, 0.9
    q, k, v = _inputs(C, H, dqk, dv, 9)
    dout = np.random.default_rng(10).standard_normal((C, H, dv))
    P = att.paths(m, off, C)
    o = np.zeros((C, H, dv))
    dq, dk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for t in range(C):
        for h in range(H):
            o[t, h], _, p, ds = att.row_terms(q, k, v, dout, P[t], t, h, scale)
            dq[t, h] = scale * ds @ k[P[t], h]
            for a, pa, dsa in zip(P[t], p, ds):
                dk[a, h] += scale * dsa * q[t, h]
                dvv[a, h] += pa * dout[t, h]
    qc = np.bincount(m, minlength=C).astype(np.float64)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    loss = 0
    for tr in range(len(off) - 1):
        rows = torch.from_numpy(m[off[tr]:off[tr + 1]])
        out = _sdpa(tq[rows], tk[rows], tv[rows], scale)
        np.testing.assert_allclose(o[rows.numpy()], out.detach().numpy(), rtol=0, atol=1e-12)
        loss = loss + (out * torch.from_numpy(dout)[rows] / torch.from_numpy(qc)[rows][:, None, None]).sum()
    loss.backward()
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dvv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-11)
